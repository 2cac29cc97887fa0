"""Test-side glue: hands the seeded input tensors to the CPU oracle as host arrays.

Only value copies happen here (bf16 and fp32 widen exactly to float64); no step of the
method is computed.  For the big workloads only the rows a test samples are copied
for the per-row tensors (q, q_idx, weights); the key/value tensors are copied whole.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle


def host(x: torch.Tensor) -> np.ndarray:
    return x.detach().to("cpu", torch.float64).numpy()


class RowMap:
    """Indexable by global row id, holding only a subset of rows."""

    def __init__(self, full: torch.Tensor, rows):
        rows = sorted(set(int(r) for r in rows))
        idx = torch.tensor(rows, dtype=torch.long, device=full.device)
        vals = host(full.index_select(0, idx)) if rows else np.zeros((0,) + tuple(full.shape[1:]))
        self._pos = {r: i for i, r in enumerate(rows)}
        self._vals = vals

    def __getitem__(self, t):
        return self._vals[self._pos[int(t)]]


def layout_of(inp, with_offsets=True) -> oracle.Layout:
    return oracle.Layout(cu_q=inp.cu_q.cpu().numpy().astype(np.int64),
                         cu_k=inp.cu_k.cpu().numpy().astype(np.int64),
                         ratio=inp.wl.ratio,
                         off=inp.offsets.cpu().numpy().astype(np.int64) if with_offsets else None,
                         cu_q_real=(inp.cu_q_real.cpu().numpy().astype(np.int64)
                                    if inp.cu_q_real is not None else None))


def problem_of(inp, rows=None) -> oracle.Problem:
    """oracle.Problem over the inputs; with ``rows`` only those query rows are usable."""
    wl = inp.wl
    if rows is None:
        q, q_idx, w = host(inp.q), host(inp.q_idx), host(inp.weights)
    else:
        q, q_idx, w = RowMap(inp.q, rows), RowMap(inp.q_idx, rows), RowMap(inp.weights, rows)
    return oracle.Problem(layout=layout_of(inp), q=q, kv=host(inp.kv), ckv=host(inp.ckv),
                          q_idx=q_idx, k_idx=host(inp.k_idx), weights=w,
                          sink=host(inp.sink), topk=wl.topk, window=wl.window,
                          scale=inp.scale, idx_scale=inp.idx_scale,
                          sparse_loss=wl.sparse_loss, per_token=False)
