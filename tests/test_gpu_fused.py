"""GPU parity of the fused score + top-k call (csa_indexer_topk, through the C ABI).

The fused call computes the same fp32 scores as csa_indexer_score (same MFMA arithmetic)
and selects on them in on-chip memory, so against the two-call path its ids and selected
scores must be bit-identical, and so must everything downstream that reads them (the
teacher/KL with scores_selected, the backward).  The oracle pins the rest: row_lse against
the oracle's float64 log-sum-exp of its own scores (within the fp32 score band plus 1e-6
relative), the exact-integer family end to end, and the oracle's top-k of the two-call
scores (tests/gpu_check.py) on sampled rows.  Layouts cover ragged packed documents, rows
with no visible key, chunk offsets whose two blocks overflow one score area (the two-phase
path), and every supported (Hi, Di).
"""
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import oracle
from deepseek_v4_csa_amd import inputs as I
from tests import gpu_check as C
from tests import oracle_bridge as B
from tests.test_gpu_backward import _close, nan_workspaces

pytestmark = pytest.mark.gpu


def _ops():
    from deepseek_v4_csa_amd import ops
    ops.load()
    return ops


def _both(ops, L, inp, topk):
    s = ops.csa_indexer_score(L, inp.q_idx, inp.k_idx, inp.weights, inp.idx_scale)
    ids = ops.csa_topk(L, s, topk)
    fid, sel, lse = ops.csa_indexer_topk(L, inp.q_idx, inp.k_idx, inp.weights, inp.idx_scale, topk,
                                         want_lse=True)
    torch.cuda.synchronize()
    return s, ids, fid, sel, lse


def _check_against_two_calls(L, inp, s, ids, fid, sel, lse, rows=None):
    assert torch.equal(fid, ids)
    cu_k = inp.cu_k.long()
    T = ids.shape[0]
    seg = torch.searchsorted(inp.cu_q.long(), torch.arange(T, device=ids.device), right=True) - 1
    loc = torch.where(ids >= 0, ids.long() - cu_k[seg][:, None], torch.zeros_like(ids, dtype=torch.long))
    want = torch.where(ids >= 0, s.gather(1, loc), torch.full_like(sel, -float("inf")))
    assert torch.equal(sel, want)
    # row_lse against the oracle's float64 log-sum-exp of its own scores
    P = B.problem_of(inp, rows) if rows is not None else B.problem_of(inp)
    lse_h = B.host(lse)
    for t in (rows if rows is not None else range(T)):
        g = oracle.row_geometry(P.layout, t)
        if g.n_valid == 0:
            assert lse_h[t] == -np.inf, t
            continue
        k_seg = P.k_idx[g.k_base:int(P.layout.cu_k[g.seg + 1])]
        o = oracle.indexer_scores_row(P.q_idx[t], P.weights[t], k_seg, P.idx_scale, g.n_valid)[:g.n_valid]
        band = C.score_band(P, t, g)[:g.n_valid].max()
        ref = float(np.log(np.sum(np.exp(o - o.max()))) + o.max())
        assert abs(lse_h[t] - ref) <= band + 1e-6 * abs(ref) + 1e-6, (t, lse_h[t], ref)


SHAPES = [(8, 64), (16, 64), (4, 128), (8, 128), (32, 64), (64, 64), (16, 128), (32, 128)]


@pytest.mark.parametrize("Hi,Di", SHAPES)
def test_fused_equals_two_calls_every_row(gpu_ok, Hi, Di):
    """Ragged packed documents (short ones have rows with no visible key)."""
    ops = _ops()
    wl = I.scaled_down(I.WORKLOADS[1], (100, 37, 300, 16, 520), topk=40, Hi=Hi, Di=Di,
                       name=f"fused-hi{Hi}-di{Di}")
    inp = I.make_inputs(wl, device="cuda", seed=Hi + Di)
    L = ops.layout_of_inputs(inp)
    s, ids, fid, sel, lse = _both(ops, L, inp, wl.topk)
    _check_against_two_calls(L, inp, s, ids, fid, sel, lse)


def test_fused_exact_family_end_to_end(gpu_ok):
    """Integer inputs: the scores are exact in any summation order, so the fused ids equal
    the oracle's top-k of its own scores, ties (frequent here) to the lower index."""
    ops = _ops()
    wl = I.scaled_down(I.WORKLOADS[1], (512, 300), topk=40)
    inp = I.make_inputs(wl, device="cuda", family="exact")
    L = ops.layout_of_inputs(inp)
    fid, sel, lse = ops.csa_indexer_topk(L, inp.q_idx, inp.k_idx, inp.weights, inp.idx_scale, wl.topk,
                                         want_lse=True)
    torch.cuda.synchronize()
    P = B.problem_of(inp)
    k_eff = fid.shape[1]
    g_ids = fid.cpu().numpy().astype(np.int64)
    g_sel = B.host(sel)
    for t in range(wl.total_q):
        g = oracle.row_geometry(P.layout, t)
        o = oracle.indexer_scores_row(P.q_idx[t], P.weights[t], P.k_idx[g.k_base:int(P.layout.cu_k[g.seg + 1])],
                                      P.idx_scale, g.n_valid)
        o_ids = oracle.topk_row(o, g.n_valid, k_eff, g.k_base)
        assert np.array_equal(o_ids, g_ids[t]), t
        v = o_ids >= 0
        assert np.array_equal(g_sel[t][v], o[o_ids[v] - g.k_base]), t


def test_fused_two_phase_chunk_offsets(gpu_ok):
    """A query chunk scored against its key prefix with offset = chunk start: both blocks
    of a pair see most of the prefix, more than one score area holds, so the kernel takes
    the pair's blocks one after the other."""
    ops = _ops()
    wl = I.scaled_down(I.WORKLOADS[1], (2560,), topk=64)
    inp = I.make_inputs(wl, device="cuda", seed=3)
    c0 = 2048
    Lc = ops.Layout.from_lengths([2560 - c0], [640], 4, offsets=[c0])
    sub = SimpleNamespace(q_idx=inp.q_idx[c0:].contiguous(), weights=inp.weights[c0:].contiguous(),
                          k_idx=inp.k_idx, idx_scale=inp.idx_scale)
    s, ids, fid, sel, lse = _both(ops, Lc, sub, wl.topk)
    assert torch.equal(fid, ids)
    # and against the whole sequence's rows
    Lf = ops.layout_of_inputs(inp)
    sf = ops.csa_indexer_score(Lf, inp.q_idx, inp.k_idx, inp.weights, inp.idx_scale)
    idf = ops.csa_topk(Lf, sf, wl.topk)
    torch.cuda.synchronize()
    assert torch.equal(fid, idf[c0:])


@pytest.mark.parametrize("index", [1, 2])
def test_fused_full_workload_forward_and_backward(gpu_ok, index):
    """bshd-b2-s4096 (two blocks per workgroup) and thd-varlen-16k (32 x 64: one block per
    workgroup, heads in groups): fused ids / selected scores / KL / loss / backward equal
    the two-call path bit for bit on every row; row_lse against the oracle on sampled rows."""
    ops = _ops()
    wl = I.WORKLOADS[index]
    inp = I.make_inputs(wl, device="cuda")
    L = ops.layout_of_inputs(inp)
    r2 = ops.forward(inp, want_teacher=True, poison=True)
    rf = ops.forward(inp, want_teacher=True, poison=True, fused=True)
    torch.cuda.synchronize()
    rows = I.sample_rows(wl, 24)
    _check_against_two_calls(L, inp, r2["scores"], r2["ids"], rf["ids"], rf["sel"], rf["row_lse"], rows)
    for k in ("out", "lse", "cmass", "teacher", "kl_row", "loss"):
        assert torch.equal(rf[k], r2[k]), k
    # the oracle's top-k of the two-call scores on sampled rows (scores within the band)
    C.check_rows(inp, r2, rows, tag="fused-" + wl.name)
    g, ws = nan_workspaces(ops, L, inp)
    a = ops.csa_indexer_loss_bwd(L, True, inp.q_idx, inp.k_idx, inp.weights, inp.idx_scale, r2["scores"],
                                 r2["ids"], r2["teacher"], grad_scores=g, workspace=ws)
    a = [x.clone() for x in a]
    g, ws = nan_workspaces(ops, L, inp)
    b = ops.csa_indexer_loss_bwd(L, True, inp.q_idx, inp.k_idx, inp.weights, inp.idx_scale, rf["sel"],
                                 rf["ids"], rf["teacher"], grad_scores=g, workspace=ws, scores_selected=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
