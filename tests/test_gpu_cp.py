"""GPU: one rank's share of context-parallel (CP) scoring ([PR8539], item 2 and the recall
table of its test plan), laid out by csa_cp_plan and scored with the ordinary
csa_indexer_score + csa_topk calls.

Per scenario of the recall table (single sequence at CP = 1 and at CP = 2 on both ranks;
documents of 1024 and 2048 tokens packed, CP = 2 on both ranks):
  * every share row's scores and ids equal the whole-batch run's, bit for bit (the ids
    mapped back to batch key rows);
  * on sampled rows the scores are within the oracle's fp32 band and the ids are the
    oracle's top-k of the same scores;
  * recall against an fp32 torch top-k over each row's absolute causal keys (of the
    whole-batch scores) is 1 on every row; with the offsets removed (top-left
    alignment) it drops -- the negative control.
"""
import numpy as np
import pytest
import torch

import oracle
from deepseek_v4_csa_amd import inputs as I
from tests import gpu_check as C

pytestmark = pytest.mark.gpu

SCENARIOS = {
    "single-cp1-rank0": (I.WORKLOADS[1], (4096,), 1, 0),
    "single-cp2-rank0": (I.WORKLOADS[1], (4096,), 2, 0),
    "single-cp2-rank1": (I.WORKLOADS[1], (4096,), 2, 1),
    "packed-cp2-rank0": (I.WORKLOADS[2], (1024, 2048), 2, 0),
    "packed-cp2-rank1": (I.WORKLOADS[2], (1024, 2048), 2, 1),
}


def _ops():
    from deepseek_v4_csa_amd import ops
    ops.load()
    return ops


def _share(ops, inp, plan, offsets):
    dev = inp.q_idx.device
    nseg = len(plan["off"])
    rows, keys, seg_of_row = [], [], []
    for s in range(nseg):
        c = plan["cu_q"][s + 1] - plan["cu_q"][s]
        nk = plan["cu_k"][s + 1] - plan["cu_k"][s]
        rows += range(plan["q_src"][s], plan["q_src"][s] + c)
        keys += range(plan["k_src"][s], plan["k_src"][s] + nk)
        seg_of_row += [s] * c
    rt = torch.tensor(rows, device=dev)
    kt = torch.tensor(keys, device=dev)
    off = plan["off"] if offsets == "explicit" else [0] * nseg
    seg_q = [plan["cu_q"][s + 1] - plan["cu_q"][s] for s in range(nseg)]
    seg_k = [plan["cu_k"][s + 1] - plan["cu_k"][s] for s in range(nseg)]
    L = ops.Layout.from_lengths(seg_q, seg_k, inp.wl.ratio, offsets=off)
    q_idx = inp.q_idx.index_select(0, rt).contiguous()
    w = inp.weights.index_select(0, rt).contiguous()
    k_idx = inp.k_idx.index_select(0, kt).contiguous()
    return L, rows, seg_of_row, q_idx, w, k_idx


def _to_batch_ids(ids, plan, seg_of_row):
    seg = torch.tensor(seg_of_row, device=ids.device)
    base = torch.tensor(plan["cu_k"][:-1], device=ids.device)[seg][:, None]
    src = torch.tensor(plan["k_src"], device=ids.device)[seg][:, None]
    return torch.where(ids >= 0, ids - base + src, torch.full_like(ids, -1))


@pytest.mark.parametrize("name", list(SCENARIOS))
def test_cp_share_scores_like_the_whole_batch(gpu_ok, name):
    ops = _ops()
    base, docs, cp, rank = SCENARIOS[name]
    wl = I.scaled_down(base, docs, name=f"{base.name}-{'-'.join(map(str, docs))}")
    inp = I.make_inputs(wl, device="cuda")
    Lf = ops.layout_of_inputs(inp)
    sf = ops.csa_indexer_score(Lf, inp.q_idx, inp.k_idx, inp.weights, inp.idx_scale)
    idf = ops.csa_topk(Lf, sf, wl.topk)
    plan = ops.csa_cp_plan(docs, wl.ratio, cp, rank)
    recalls = {}
    for offsets in ("explicit", "top-left"):
        L, rows, seg_of_row, q_idx, w, k_idx = _share(ops, inp, plan, offsets)
        ss = ops.csa_indexer_score(L, q_idx, k_idx, w, inp.idx_scale)
        ids = ops.csa_topk(L, ss, wl.topk)
        torch.cuda.synchronize()
        bid = _to_batch_ids(ids.long(), plan, seg_of_row)
        rt = torch.tensor(rows, device=sf.device)
        k_s = ids.shape[1]
        recalls[offsets] = C.recall_rows(inp, sf, bid, rows)
        if offsets != "explicit":
            continue
        ref_ids = idf.index_select(0, rt).long()
        assert torch.equal(bid, ref_ids[:, :k_s])
        assert bool((ref_ids[:, k_s:] == -1).all())
        ld = L.max_seqlen_k
        assert torch.equal(ss[:, :ld], sf.index_select(0, rt)[:, :ld])
        # the oracle on sampled share rows: fp32 band on the scores, its top-k of the
        # GPU's scores equal to the GPU's ids
        _oracle_rows(L, plan, seg_of_row, q_idx, w, k_idx, inp, ss, ids)
    print(f"{name}: recall mean/min with offsets {recalls['explicit'][0]:.3f} / "
          f"{recalls['explicit'][1]:.3f}, top-left {recalls['top-left'][0]:.3f} / "
          f"{recalls['top-left'][1]:.3f}", flush=True)
    assert recalls["explicit"] == (1.0, 1.0)
    assert recalls["top-left"][0] < 0.99


def _oracle_rows(L, plan, seg_of_row, q_idx, w, k_idx, inp, ss, ids, n=12):
    cu_q = np.asarray(plan["cu_q"])
    cu_k = np.asarray(plan["cu_k"])
    OL = oracle.Layout(cu_q=cu_q, cu_k=cu_k, ratio=inp.wl.ratio, off=np.asarray(plan["off"]))
    k_eff = ids.shape[1]
    T = int(cu_q[-1])
    pick = sorted(set(np.linspace(0, T - 1, n).astype(int).tolist()) | {int(c) for c in cu_q[1:-1]})
    kh = k_idx.double().cpu().numpy()
    for t in pick:
        g = oracle.row_geometry(OL, t)
        seg_keys = kh[g.k_base:int(cu_k[g.seg + 1])]
        qt = q_idx[t].double().cpu().numpy()
        wt = w[t].cpu().numpy()
        o = oracle.indexer_scores_row(qt, wt, seg_keys, inp.idx_scale, g.n_valid)
        gs = ss[t].double().cpu().numpy()
        if g.n_valid:
            ws = np.abs(oracle.indexer_weight_scale(wt, inp.idx_scale).astype(np.float64))
            band = (qt.shape[1] + qt.shape[0] + 2) * 2.0 ** -24 * ((np.abs(seg_keys) @ np.abs(qt).T) @ ws)
            assert np.all(np.abs(gs[:g.n_valid] - o[:g.n_valid]) <= band[:g.n_valid] + 1e-30), t
        assert np.all(gs[g.n_valid:cu_k[g.seg + 1] - g.k_base] == -np.inf)
        o_ids = oracle.topk_row(gs[:int(cu_k[g.seg + 1]) - g.k_base], g.n_valid, k_eff, g.k_base)
        assert np.array_equal(o_ids, ids[t].cpu().numpy().astype(np.int64)), t
