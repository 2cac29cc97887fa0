"""Tiny hand-built problems for the oracle's CPU pins (oracle-only inputs)."""
from __future__ import annotations

import numpy as np

import oracle


def layout(seg_lens, ratio, off=None, cu_k=None):
    cu_q = np.concatenate([[0], np.cumsum(seg_lens)]).astype(np.int64)
    if cu_k is None:
        cu_k = oracle.compressed_cu_seqlens(cu_q, ratio)
    return oracle.Layout(cu_q=cu_q, cu_k=np.asarray(cu_k, dtype=np.int64), ratio=ratio,
                         off=None if off is None else np.asarray(off, dtype=np.int64))


def problem(seg_lens=(48,), ratio=4, H=3, D=8, Hi=3, Di=6, topk=5, window=4, seed=0,
            sink=None, sparse=True, integer_idx=False, L=None):
    rng = np.random.default_rng(seed)
    L = L or layout(seg_lens, ratio)
    T, Tk = L.total_q, L.total_k
    if integer_idx:
        q_idx = rng.integers(-3, 4, size=(T, Hi, Di)).astype(np.float64)
        k_idx = rng.integers(-3, 4, size=(Tk, Di)).astype(np.float64)
        w = (rng.integers(0, 16, size=(T, Hi)) / 16.0).astype(np.float32)
        idx_scale = 0.125
    else:
        q_idx = rng.standard_normal((T, Hi, Di)) / np.sqrt(Di)
        k_idx = rng.standard_normal((Tk, Di)) / np.sqrt(Di)
        w = rng.random((T, Hi)).astype(np.float32)
        idx_scale = 1.0 / np.sqrt(Di)
    q = rng.standard_normal((T, H, D)) / np.sqrt(D)
    kv = rng.standard_normal((T, D)) / np.sqrt(D)
    ckv = rng.standard_normal((Tk, D)) / np.sqrt(D)
    if sink is None:
        sink = rng.standard_normal(H)
    return oracle.Problem(layout=L, q=q, kv=kv, ckv=ckv, q_idx=q_idx, k_idx=k_idx, weights=w,
                          sink=np.asarray(sink, dtype=np.float64), topk=topk, window=window,
                          scale=1.0 / np.sqrt(D), idx_scale=float(idx_scale), sparse_loss=sparse)


def parse(v):
    """Golden-file scalars: numbers, '-inf', 'lnN' (natural log of N)."""
    if isinstance(v, str):
        if v == "-inf":
            return -np.inf
        if v.startswith("ln"):
            return float(np.log(float(v[2:])))
        return float(v)
    return float(v)
