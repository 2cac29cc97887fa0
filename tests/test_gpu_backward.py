"""GPU parity of the indexer-loss backward (csa_indexer_loss_bwd, through the C ABI)
against the CPU oracle's ``indexer_loss_backward``.

The backward takes the forward's scores, ids and teacher as saved inputs, so the oracle
is run on exactly those (ids/scores overridden, teacher replaced by the GPU's) and the
comparison isolates the backward.  Small workloads: every element of dq_idx, dweights
and dk_idx.  Full-size: seeded row samples for dq/dweights and a few keys for dk_idx.

Both workspaces (score gradients, dk partials) are handed in filled with NaN, so a read
of an element the kernels did not write first fails the comparison.

Tolerance (derived): the gradient factors enter the bf16 MFMAs as a hi/lo pair, 2^-17
relative each; products accumulate in fp32 over at most a few thousand terms per MFMA
chain (dk adds its per-token-block partials with compensated summation), so every
element is within 5e-5 of the tensor's largest magnitude (plus 1e-4 relative).
"""
import numpy as np
import pytest
import torch

import oracle
from deepseek_v4_csa_amd import inputs as I
from tests import oracle_bridge as B

pytestmark = pytest.mark.gpu

SMALL = {
    "bshd-small": I.scaled_down(I.WORKLOADS[1], (512, 300), topk=40),
    "thd-small": I.scaled_down(I.WORKLOADS[2], (128, 256, 200, 68), topk=24),
    "dense-small": I.scaled_down(I.WORKLOADS[4], (640,), topk=16),
}


def _ops():
    from deepseek_v4_csa_amd import ops
    ops.load()
    return ops


def nan_workspaces(ops, L, inp):
    """The score-gradient and dk-partial workspaces filled with NaN: any element the
    kernels read without writing first poisons the result."""
    wl = inp.wl
    g = torch.full((wl.total_q, L.max_seqlen_k), float("nan"), dtype=torch.float32, device="cuda")
    n = max(ops.csa_indexer_loss_bwd_workspace(L, wl.Hi, wl.Di), 4)
    ws = torch.full((n // 4,), float("nan"), dtype=torch.float32, device="cuda").view(torch.uint8)
    return g, ws


def _gpu(inp, grad_loss=1.0, per_token=False, res=None):
    ops = _ops()
    if res is None:
        res = ops.forward(inp, want_teacher=True, poison=True)
    L = ops.layout_of_inputs(inp)
    g, ws = nan_workspaces(ops, L, inp)
    dq, dw, dk = ops.csa_indexer_loss_bwd(L, inp.wl.sparse_loss, inp.q_idx, inp.k_idx, inp.weights,
                                          inp.idx_scale, res["scores"], res["ids"], res["teacher"],
                                          grad_loss=grad_loss, per_token=per_token, grad_scores=g,
                                          workspace=ws)
    torch.cuda.synchronize()
    return res, dq, dw, dk


def _oracle_rows(P, res, rows):
    """RowResults of `rows` on the GPU's scores and ids, with the GPU's teacher (host copies
    of those rows only)."""
    L = P.layout
    ids = B.RowMap(res["ids"], rows)
    sc = B.RowMap(res["scores"], rows)
    te = B.RowMap(res["teacher"], rows)
    out = []
    for t in rows:
        g = oracle.row_geometry(L, t)
        s_k = int(L.cu_k[g.seg + 1] - L.cu_k[g.seg])
        ids_t = ids[t].astype(np.int64)
        r = oracle.run_row(P, t, ids_override=ids_t, scores_override=sc[t][:s_k])
        if g.n_valid > 0:
            r.teacher = te[t][:ids_t.shape[0]].copy() if P.sparse_loss else te[t][:g.n_valid].copy()
        out.append(r)
    return out


def _close(name, got, ref):
    got = np.asarray(got, dtype=np.float64)
    scale = float(np.abs(ref).max())
    err = np.abs(got - ref)
    bound = 5e-5 * scale + 1e-4 * np.abs(ref)
    worst = float((err / np.maximum(scale, 1e-30)).max()) if err.size else 0.0
    print(f"{name}: max |err| / max |ref| = {worst:.3e} (scale {scale:.3e})", flush=True)
    assert scale > 0, name
    assert np.all(err <= bound), (name, worst)


@pytest.mark.parametrize("name", list(SMALL))
def test_small_workloads_every_element(gpu_ok, name):
    wl = SMALL[name]
    inp = I.make_inputs(wl, device="cuda")
    res, dq, dw, dk = _gpu(inp)
    P = B.problem_of(inp)
    rows = _oracle_rows(P, res, range(wl.total_q))
    rdq, rdw, rdk = oracle.indexer_loss_backward(P, rows)
    _close(f"{name} dq", B.host(dq), rdq)
    _close(f"{name} dw", B.host(dw), rdw)
    _close(f"{name} dk", B.host(dk), rdk)


@pytest.mark.parametrize("Hi,Di", [(4, 64), (8, 64), (32, 64), (64, 64), (4, 128), (8, 128), (16, 128),
                                   (32, 128), (64, 128)])
def test_every_supported_indexer_shape(gpu_ok, Hi, Di):
    """Each (Hi, Di) the backward supports, every element, on a ragged two-segment batch
    (q rows of 4 x 64 bf16 are 512 bytes: the staging path for rows under 1 KiB)."""
    wl = I.scaled_down(I.WORKLOADS[1], (272, 200), topk=24, Hi=Hi, Di=Di, name=f"bshd-hi{Hi}-di{Di}")
    inp = I.make_inputs(wl, device="cuda", seed=Hi * 1000 + Di)
    res, dq, dw, dk = _gpu(inp)
    P = B.problem_of(inp)
    rows = _oracle_rows(P, res, range(wl.total_q))
    rdq, rdw, rdk = oracle.indexer_loss_backward(P, rows)
    _close(f"Hi={Hi} Di={Di} dq", B.host(dq), rdq)
    _close(f"Hi={Hi} Di={Di} dw", B.host(dw), rdw)
    _close(f"Hi={Hi} Di={Di} dk", B.host(dk), rdk)


def test_per_token_loss_and_upstream_gradient(gpu_ok):
    wl = SMALL["bshd-small"]
    inp = I.make_inputs(wl, device="cuda", seed=77)
    res, dq, dw, dk = _gpu(inp, grad_loss=2.5, per_token=True)
    P = B.problem_of(inp)
    P.per_token = True
    rows = _oracle_rows(P, res, range(wl.total_q))
    rdq, rdw, rdk = oracle.indexer_loss_backward(P, rows, grad_loss=2.5)
    _close("per-token dq", B.host(dq), rdq)
    _close("per-token dw", B.host(dw), rdw)
    _close("per-token dk", B.host(dk), rdk)


def test_batch_of_two_equals_two_single_runs_scaled(gpu_ok):
    """The cuDNN-frontend pull request's GPU check: a two-sequence batch against the same
    rows run as two single-sequence calls, scaled for the row-mean loss."""
    wl = I.scaled_down(I.WORKLOADS[1], (384, 384), topk=32)
    inp = I.make_inputs(wl, device="cuda", seed=5)
    res, dq, dw, dk = _gpu(inp)
    T = wl.total_q
    wl1 = I.scaled_down(I.WORKLOADS[1], (384,), topk=32)
    for s in range(2):
        a, b = int(inp.cu_q[s]), int(inp.cu_q[s + 1])
        ka, kb = int(inp.cu_k[s]), int(inp.cu_k[s + 1])
        sub = I.make_inputs(wl1, device="cuda")
        sub.q, sub.kv, sub.q_idx, sub.weights = inp.q[a:b], inp.kv[a:b], inp.q_idx[a:b], inp.weights[a:b]
        sub.ckv, sub.k_idx, sub.sink = inp.ckv[ka:kb], inp.k_idx[ka:kb], inp.sink
        rs, dqs, dws, dks = _gpu(sub)
        f = (b - a) / T
        _close(f"seg{s} dq", B.host(dq[a:b]), f * B.host(dqs))
        _close(f"seg{s} dw", B.host(dw[a:b]), f * B.host(dws))
        _close(f"seg{s} dk", B.host(dk[ka:kb]), f * B.host(dks))


@pytest.mark.parametrize("index", [1, 2, 4])
def test_full_workloads_sampled(gpu_ok, index):
    """Full-size workloads: dq/dweights on sampled rows, dk on sampled keys (each from every
    row whose support holds the key), in the launch configuration of the forward path."""
    wl = I.WORKLOADS[index]
    inp = I.make_inputs(wl, device="cuda")
    res, dq, dw, dk = _gpu(inp)
    rows = I.sample_rows(wl, 16)
    P = B.problem_of(inp, rows)
    orows = _oracle_rows(P, res, rows)
    rdq, rdw = [], []
    for r in orows:   # the per-row part of oracle.indexer_loss_backward, on the sampled rows
        cols, tch, prd = oracle.loss_support(P, r)
        g = r.geom
        seg_k = slice(g.k_base, int(P.layout.cu_k[g.seg + 1]))
        gs = oracle.kl_grad_scores(tch, prd) / wl.total_q
        dq_t, dw_t, _ = oracle.indexer_grads_row(P.q_idx[r.t], P.weights[r.t], P.k_idx[seg_k],
                                                 P.idx_scale, cols, gs)
        rdq.append(dq_t)
        rdw.append(dw_t)
    idx = torch.tensor(rows, device="cuda")
    _close(f"{wl.name} dq rows", B.host(dq.index_select(0, idx)), np.stack(rdq))
    _close(f"{wl.name} dw rows", B.host(dw.index_select(0, idx)), np.stack(rdw))
    # dk on a few keys of the first segment: all rows of the segment, the GPU's scores,
    # ids and teacher, the oracle's score gradient and per-row key gradient
    L = P.layout
    T = wl.total_q
    keys = sorted({0, 1, int(L.cu_k[1]) // 2, int(L.cu_k[1]) - 1})
    ids = res["ids"].cpu().numpy().astype(np.int64)
    sc = B.host(res["scores"])
    te = B.host(res["teacher"])
    q_idx, w, k_idx = B.host(inp.q_idx), B.host(inp.weights), B.host(inp.k_idx)
    ref = np.zeros((len(keys), k_idx.shape[1]))
    kpos = {k: i for i, k in enumerate(keys)}
    k_seg = k_idx[int(L.cu_k[0]):int(L.cu_k[1])]
    for t in range(int(L.cu_q[0]), int(L.cu_q[1])):
        g = oracle.row_geometry(L, t)
        if g.n_valid == 0:
            continue
        if wl.sparse_loss:
            valid = ids[t] >= 0
            cols = ids[t][valid] - g.k_base
            tch = te[t, :ids.shape[1]][valid]
        else:
            cols = np.arange(g.n_valid)
            tch = te[t, :g.n_valid]
        sel = np.array([c in kpos for c in cols])
        if not sel.any():
            continue
        gs = oracle.kl_grad_scores(tch, oracle.predictor(sc[t, cols])) / T
        _, _, dk_c = oracle.indexer_grads_row(q_idx[t], w[t], k_seg, inp.idx_scale, cols[sel], gs[sel])
        for c, v in zip(cols[sel], dk_c):
            ref[kpos[int(c)]] += v
    _close(f"{wl.name} dk keys", B.host(dk[keys]), ref)


def test_long_context_sampled(gpu_ok):
    """The long-context workload (64 indexer heads x 128 dims, 16384 compressed keys, top-k
    2048): dq/dweights on sampled rows, dk on keys of the tail of the key range (each seen
    by a few thousand rows' supports), from host copies of only the rows involved."""
    wl = I.WORKLOADS[3]
    inp = I.make_inputs(wl, device="cuda")
    res, dq, dw, dk = _gpu(inp)
    T = wl.total_q
    rows = I.sample_rows(wl, 16)
    P = B.problem_of(inp, rows)
    rdq, rdw = [], []
    for r in _oracle_rows(P, res, rows):
        cols, tch, prd = oracle.loss_support(P, r)
        g = r.geom
        seg_k = slice(g.k_base, int(P.layout.cu_k[g.seg + 1]))
        gs = oracle.kl_grad_scores(tch, prd) / T
        dq_t, dw_t, _ = oracle.indexer_grads_row(P.q_idx[r.t], P.weights[r.t], P.k_idx[seg_k],
                                                 P.idx_scale, cols, gs)
        rdq.append(dq_t)
        rdw.append(dw_t)
    idx = torch.tensor(rows, device="cuda")
    _close("long-64k dq rows", B.host(dq.index_select(0, idx)), np.stack(rdq))
    _close("long-64k dw rows", B.host(dw.index_select(0, idx)), np.stack(rdw))
    # dk: every row whose support holds one of the keys, found on the GPU
    keys = [12000, 16000, 16383]
    kt = torch.tensor(keys, device="cuda", dtype=res["ids"].dtype)
    hit = (res["ids"].unsqueeze(-1) == kt).any(-1).any(-1)
    krows = torch.nonzero(hit).flatten().tolist()
    assert len(krows) > 100, len(krows)
    k_idx = B.host(inp.k_idx)
    ref = np.zeros((len(keys), k_idx.shape[1]))
    kpos = {k: i for i, k in enumerate(keys)}
    for b0 in range(0, len(krows), 1024):
        part = krows[b0:b0 + 1024]
        pi = torch.tensor(part, device="cuda")
        ids_p = res["ids"].index_select(0, pi)
        sc_p = B.host(torch.gather(res["scores"].index_select(0, pi), 1, ids_p.clamp(min=0).long()))
        te_p = B.host(res["teacher"].index_select(0, pi)[:, :ids_p.shape[1]])
        q_p, w_p = B.host(inp.q_idx.index_select(0, pi)), B.host(inp.weights.index_select(0, pi))
        ids_p = ids_p.cpu().numpy().astype(np.int64)
        for i in range(len(part)):
            valid = ids_p[i] >= 0
            cols = ids_p[i][valid]          # one segment: global ids are local ids
            sel = np.isin(cols, keys)
            gs = oracle.kl_grad_scores(te_p[i][valid], oracle.predictor(sc_p[i][valid])) / T
            _, _, dk_c = oracle.indexer_grads_row(q_p[i], w_p[i], k_idx, inp.idx_scale, cols[sel], gs[sel])
            for c, v in zip(cols[sel], dk_c):
                ref[kpos[int(c)]] += v
    _close("long-64k dk keys", B.host(dk[keys]), ref)
