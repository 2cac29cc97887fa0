"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Small workloads (same head shapes as the five configurations, shorter and ragged
sequences) are checked on every row; the full-size workloads on seeded row samples
(always including the first ratio+1 rows and the last row of every segment), plus
properties checked on every row (top-k recall, loss = reduction of kl_row, determinism).
Tolerances are stated in tests/gpu_check.py.
"""
import gc

import numpy as np
import pytest
import torch

from deepseek_v4_csa_amd import inputs as I
from tests import gpu_check as C

pytestmark = pytest.mark.gpu


def _ops():
    from deepseek_v4_csa_amd import ops
    ops.load()
    return ops


def _run(inp):
    res = _ops().forward(inp, want_teacher=True, poison=True)
    torch.cuda.synchronize()
    return res


SMALL = {
    "tiny-fp32": I.WORKLOADS[0],
    "bshd-small": I.scaled_down(I.WORKLOADS[1], (512, 300), topk=40),
    "thd-small": I.scaled_down(I.WORKLOADS[2], (128, 256, 200, 68), topk=24),
    "long-small": I.scaled_down(I.WORKLOADS[3], (384,), topk=48),
    "dense-small": I.scaled_down(I.WORKLOADS[4], (640,), topk=16),
}


@pytest.mark.parametrize("family", ["gauss", "exact"])
@pytest.mark.parametrize("name", list(SMALL))
def test_small_workloads_every_row(gpu_ok, name, family):
    wl = SMALL[name]
    inp = I.make_inputs(wl, device="cuda", family=family)
    res = _run(inp)
    rep = C.check_rows(inp, res, list(range(wl.total_q)), exact_scores=(family == "exact"),
                       tag=f"{name}-{family}", loss_rows=True)
    print(name, family, dict(rep), flush=True)
    # the loss is the documented reduction of kl_row (mean over every physical row)
    kl = res["kl_row"].double()
    assert abs(float(res["loss"][0]) - float(kl.sum() / wl.total_q)) <= 1e-6 * abs(float(kl.sum() / wl.total_q)) + 1e-9


@pytest.mark.parametrize("index", [1, 2, 3, 4])
def test_full_workloads_sampled_rows(gpu_ok, index):
    wl = I.WORKLOADS[index]
    inp = I.make_inputs(wl, device="cuda")
    res = _run(inp)
    rows = I.sample_rows(wl, 40 if index != 3 else 24)
    if index == 3:
        # rows with fewer causal keys than k_eff (their compressed chunks end early)
        rows = sorted(set(rows) | set(range(37, 8192, 331)))
    rep = C.check_rows(inp, res, rows, tag=wl.name)
    mean, mn = C.recall_all_rows(inp, res)
    print(wl.name, dict(rep), "recall", mean, mn, flush=True)
    assert mean == 1.0 and mn == 1.0
    kl = res["kl_row"].double()
    want = float(kl.sum() / wl.total_q)
    assert abs(float(res["loss"][0]) - want) <= 1e-6 * abs(want) + 1e-9
    assert torch.isfinite(res["kl_row"]).all()
    # determinism: a second run is bitwise identical (no atomics anywhere)
    res2 = _run(inp)
    for k in ("scores", "ids", "out", "lse", "cmass", "kl_row", "loss"):
        if res[k] is not None:
            assert torch.equal(res[k], res2[k]), k
    del inp, res, res2
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("index", [1, 2, 3, 4])
def test_full_workloads_exact_family_ids(gpu_ok, index):
    """Exact-integer indexer inputs: the ids of sampled rows are bit-exact end to end."""
    wl = I.WORKLOADS[index]
    inp = I.make_inputs(wl, device="cuda", family="exact")
    ops = _ops()
    L = ops.layout_of_inputs(inp)
    scores = ops.csa_indexer_score(L, inp.q_idx, inp.k_idx, inp.weights, inp.idx_scale)
    ids = ops.csa_topk(L, scores, wl.topk)
    torch.cuda.synchronize()
    import oracle
    from tests.oracle_bridge import problem_of, host
    rows = I.sample_rows(wl, 32)
    P = problem_of(inp, rows)
    k_eff = oracle.k_eff_of(P.layout, wl.topk)
    idx = torch.tensor(rows, device="cuda")
    gs = host(scores.index_select(0, idx))
    gi = ids.index_select(0, idx).cpu().numpy()
    for n, t in enumerate(rows):
        g = oracle.row_geometry(P.layout, t)
        s_k = int(P.layout.cu_k[g.seg + 1]) - g.k_base
        o = oracle.indexer_scores_row(P.q_idx[t], P.weights[t], P.k_idx[g.k_base:g.k_base + s_k],
                                      P.idx_scale, g.n_valid)
        assert np.array_equal(gs[n, :s_k], o), f"row {t}"
        assert np.array_equal(gi[n], oracle.topk_row(o, g.n_valid, k_eff, g.k_base)), f"row {t}"
    del inp, scores, ids
    gc.collect()
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------- invariants
def test_window_and_sink_perturbation_moves_teacher_only(gpu_ok):
    """Perturbing only the window KV or one head's sink leaves the scores and ids
    bit-identical and changes the teacher (page 'Static reproduction / invariant')."""
    wl = SMALL["bshd-small"]

    def mk():
        x = I.make_inputs(wl, device="cuda")
        x.q = (x.q.float() * 32.0).to(x.q.dtype)  # heads with distinct preferences
        return x
    base = mk()
    r0 = _run(base)
    p1 = mk()
    p1.kv = (p1.kv.float() * 3.0).to(p1.kv.dtype)
    p2 = mk()
    p2.sink = p2.sink.clone()
    p2.sink[0] += 3.0
    for p in (p1, p2):
        r = _run(p)
        assert torch.equal(r["scores"], r0["scores"])
        assert torch.equal(r["ids"], r0["ids"])
        moved = (r["teacher"] - r0["teacher"]).abs()
        tol = 1e-5 * r0["teacher"].abs() + 1e-9          # the teacher parity tolerance
        print("teacher moved by up to", moved.max().item(), flush=True)
        assert bool((moved > 100 * tol).any())
        assert not torch.equal(r["kl_row"], r0["kl_row"])


def test_batch_of_two_equals_two_single_runs(gpu_ok):
    """[Megatron-LM PR 8539 test plan]: a micro-batch of two matches two b=1 runs; the
    second batch's ids are shifted by S_k (global ids)."""
    wl2 = I.scaled_down(I.WORKLOADS[1], (1024, 1024), topk=64)
    inp = I.make_inputs(wl2, device="cuda")
    r = _run(inp)
    wl1 = I.scaled_down(I.WORKLOADS[1], (1024,), topk=64)
    S, Sk = 1024, 256
    for b in range(2):
        one = I.make_inputs(wl1, device="cuda")
        sl, kl_ = slice(b * S, (b + 1) * S), slice(b * Sk, (b + 1) * Sk)
        one.q, one.kv, one.q_idx, one.weights = inp.q[sl], inp.kv[sl], inp.q_idx[sl], inp.weights[sl]
        one.ckv, one.k_idx, one.sink = inp.ckv[kl_], inp.k_idx[kl_], inp.sink
        r1 = _run(one)
        assert torch.equal(r["scores"][sl], r1["scores"])
        shifted = torch.where(r1["ids"] >= 0, r1["ids"] + b * Sk, r1["ids"])
        assert torch.equal(r["ids"][sl], shifted)
        assert torch.equal(r["out"][sl], r1["out"])
        assert torch.equal(r["kl_row"][sl], r1["kl_row"])


def test_packed_documents_equal_independent_runs(gpu_ok):
    wl = SMALL["thd-small"]
    inp = I.make_inputs(wl, device="cuda")
    r = _run(inp)
    cu_q, cu_k = inp.cu_q.tolist(), inp.cu_k.tolist()
    for s, n in enumerate(wl.seg_lens):
        w1 = I.scaled_down(wl, (n,), topk=wl.topk)
        one = I.make_inputs(w1, device="cuda")
        sl, kl_ = slice(cu_q[s], cu_q[s + 1]), slice(cu_k[s], cu_k[s + 1])
        one.q, one.kv, one.q_idx, one.weights = inp.q[sl], inp.kv[sl], inp.q_idx[sl], inp.weights[sl]
        one.ckv, one.k_idx, one.sink = inp.ckv[kl_], inp.k_idx[kl_], inp.sink
        # the single-document run has k_eff = min(topk, its own S_k); the packed run's is the
        # batch maximum, so compare the valid ids
        r1 = _run(one)
        k1 = r1["ids"].shape[1]
        assert torch.equal(r["scores"][sl, :cu_k[s + 1] - cu_k[s]], r1["scores"])
        shifted = torch.where(r1["ids"] >= 0, r1["ids"] + cu_k[s], r1["ids"])
        assert torch.equal(r["ids"][sl, :k1], shifted)
        assert bool((r["ids"][sl, k1:] == -1).all())
        assert torch.equal(r["out"][sl], r1["out"])
        assert torch.allclose(r["kl_row"][sl], r1["kl_row"], rtol=1e-6, atol=1e-9)


def test_chunk_offsets_and_negative_control(gpu_ok):
    """[PR 8539, item 2]: a query chunk scored against the key prefix with offset = chunk
    start selects exactly the full run's keys; without the offset it does not."""
    ops = _ops()
    wl = I.scaled_down(I.WORKLOADS[1], (2048,), topk=64)
    inp = I.make_inputs(wl, device="cuda")
    Lf = ops.layout_of_inputs(inp)
    sf = ops.csa_indexer_score(Lf, inp.q_idx, inp.k_idx, inp.weights, inp.idx_scale)
    idf = ops.csa_topk(Lf, sf, wl.topk)
    c0 = 1280
    changed = 0
    for off in (c0, 0):
        Lc = ops.Layout.from_lengths([2048 - c0], [512], 4, offsets=[off])
        sc = ops.csa_indexer_score(Lc, inp.q_idx[c0:].contiguous(), inp.k_idx, inp.weights[c0:].contiguous(),
                                   inp.idx_scale)
        idc = ops.csa_topk(Lc, sc, wl.topk)
        torch.cuda.synchronize()
        if off == c0:
            assert torch.equal(sc, sf[c0:])
            assert torch.equal(idc, idf[c0:])
        else:
            changed = int((idc != idf[c0:]).any(1).sum())
    assert changed > 0


# ----------------------------------------------------------------------------- edge cases
def test_edge_layouts(gpu_ok):
    """Empty and short segments, lengths not divisible by the ratio (negative default
    offsets), window 0, top-k above every segment's key count, a sink of -inf; every row
    against the oracle (tolerances of tests/gpu_check.py, the loss included)."""
    ops = _ops()
    rng = torch.Generator(device="cuda")
    rng.manual_seed(5)
    seg_q = [70, 0, 3, 129, 1]
    ratio = 4
    seg_k = [a // ratio for a in seg_q]
    H, D, Hi, Di = 16, 128, 4, 64
    T, Tk = sum(seg_q), sum(seg_k)
    for window, topk, sink_val in ((0, 8, None), (5, 64, -float("inf")), (3, 2, None)):
        L = ops.Layout.from_lengths(seg_q, seg_k, ratio)     # NULL offsets: the bottom-right default
        rnd = lambda *s: (torch.randn(*s, generator=rng, device="cuda") / 8).to(torch.bfloat16)
        q, kv, ckv = rnd(T, H, D), rnd(T, D), rnd(Tk, D)
        qi, ki = rnd(T, Hi, Di), rnd(Tk, Di)
        w = torch.rand(T, Hi, generator=rng, device="cuda")
        sink = torch.randn(H, generator=rng, device="cuda")
        if sink_val is not None:
            sink[:] = sink_val
        with ops.poisoned_outputs():
            sc = ops.csa_indexer_score(L, qi, ki, w, 0.125)
            ids = ops.csa_topk(L, sc, topk)
            out, lse, lse_nc, cm = ops.csa_sparse_attn_fwd(L, q, kv, ckv, sink, ids, window, D ** -0.5)
            te, klr, loss = ops.csa_indexer_teacher_kl(L, True, sc, ids, cm, q, ckv, lse_nc, D ** -0.5,
                                                       want_teacher=True)
        torch.cuda.synchronize()
        wl = I.scaled_down(I.WORKLOADS[1], seg_q, H=H, D=D, Hi=Hi, Di=Di, topk=topk, window=window,
                           name=f"edge-w{window}-k{topk}")
        # the oracle takes the offsets explicitly: seg_k * ratio - seg_q
        off = torch.tensor([k * ratio - n for n, k in zip(seg_q, seg_k)], dtype=torch.int32, device="cuda")
        inp = I.Inputs(wl, L.cu_q, L.cu_k, off, q, kv, ckv, qi, ki, w, sink, 0.125, D ** -0.5)
        assert ids.shape[1] == min(topk, max(seg_k))
        res = dict(scores=sc, ids=ids, out=out, lse=lse, lse_nc=lse_nc, cmass=cm, teacher=te, kl_row=klr,
                   loss=loss)
        rep = C.check_rows(inp, res, list(range(T)), tag="edge-layouts", loss_rows=True)
        print(wl.name, dict(rep), flush=True)
