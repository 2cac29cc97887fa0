"""Row-by-row comparison of the HIP path against the CPU oracle (test helper).

Tolerances (written here, used by every GPU parity test):
  scores    exact-integer family: bit-exact.  Gaussian: |I_gpu - I_oracle| <= B_tj with
            B_tj = gamma * sum_h ws_h * sum_d |q_hd k_jd|, gamma = (Di + Hi + 2) * 2^-24,
            the worst-case fp32 accumulation error of Di + Hi + 2 rounded operations.
  ids       bit-exact against the oracle's top-k of the GPU's own fp32 score row
            (identical inputs to the selection); end-to-end bit-exact on the exact family.
  out       |delta| <= 2e-2 absolute (bf16 output, bf16 probabilities in P.V); the fp32
            workload uses the same bound.
  lse, lse_nc  |delta| <= 1e-5 * |x| + 1e-6.
  cmass, teacher  |delta| <= 1e-5 * |x| + 1e-9 per element, on identical ids.
  kl_row    |delta| <= 1e-5 * |KL| + 1e-8, on identical ids.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from tests.oracle_bridge import host, problem_of

TOL_OUT = 2e-2
REL = 1e-5


def score_band(P, t, g):
    """Worst-case fp32 accumulation bound of every score of row t."""
    L = P.layout
    k = np.abs(np.asarray(P.k_idx[g.k_base:int(L.cu_k[g.seg + 1])], dtype=np.float64))
    q = np.abs(np.asarray(P.q_idx[t], dtype=np.float64))
    ws = np.abs(oracle.indexer_weight_scale(P.weights[t], P.idx_scale).astype(np.float64))
    Hi, Di = q.shape
    gamma = (Di + Hi + 2) * 2.0 ** -24
    return gamma * ((k @ q.T) @ ws) + 1e-30


class Report(dict):
    def bump(self, key, val):
        self[key] = max(self.get(key, 0.0), float(val))


def check_rows(inp, res, rows, exact_scores=False, check_scores=True, dense=None):
    """Compare GPU results `res` (dict from ops.forward with want_teacher) with the oracle on
    `rows`.  Raises AssertionError on the first violation; returns max error statistics."""
    wl = inp.wl
    P = problem_of(inp, rows)
    dense = (not wl.sparse_loss) if dense is None else dense
    L = P.layout
    k_eff = oracle.k_eff_of(L, P.topk)
    rep = Report()
    idx = torch.tensor(rows, dtype=torch.long, device=res["scores"].device)
    g_scores = host(res["scores"].index_select(0, idx))
    g_ids = res["ids"].index_select(0, idx).cpu().numpy().astype(np.int64)
    g_out = host(res["out"].index_select(0, idx))
    g_lse = host(res["lse"].index_select(0, idx))
    g_lnc = host(res["lse_nc"].index_select(0, idx))
    g_cm = host(res["cmass"].index_select(0, idx)) if res.get("cmass") is not None else None
    g_teach = host(res["teacher"].index_select(0, idx)) if res.get("teacher") is not None else None
    g_kl = host(res["kl_row"].index_select(0, idx))
    for n, t in enumerate(rows):
        g = oracle.row_geometry(L, t)
        s_k = int(L.cu_k[g.seg + 1]) - g.k_base
        # ---- scores
        o_sc = oracle.indexer_scores_row(P.q_idx[t], P.weights[t], P.k_idx[g.k_base:g.k_base + s_k],
                                         P.idx_scale, g.n_valid)
        gs = g_scores[n, :s_k]
        assert np.all(gs[g.n_valid:] == -np.inf), f"row {t}: masked columns not -inf"
        if wl.max_seqlen_k > s_k:
            assert np.all(g_scores[n, s_k:wl.max_seqlen_k] == -np.inf), f"row {t}: tail not -inf"
        if check_scores and g.n_valid:
            d = np.abs(gs[:g.n_valid] - o_sc[:g.n_valid])
            if exact_scores:
                assert np.all(d == 0), f"row {t}: exact-family score differs by {d.max()}"
            else:
                band = score_band(P, t, g)[:g.n_valid]
                assert np.all(d <= band), f"row {t}: score error {d.max()} above band"
                rep.bump("score_err_over_band", np.max(d / band))
        # ---- ids: the oracle's selection on the GPU's own scores
        o_ids = oracle.topk_row(gs, g.n_valid, k_eff, g.k_base)
        assert np.array_equal(o_ids, g_ids[n]), f"row {t}: ids differ from the oracle top-k of the same scores"
        if exact_scores:
            o_ids2 = oracle.topk_row(o_sc, g.n_valid, k_eff, g.k_base)
            assert np.array_equal(o_ids2, g_ids[n]), f"row {t}: exact-family ids differ end to end"
        # ---- attention, teacher, KL on identical ids
        r = oracle.run_row(P, t, ids_override=g_ids[n])
        A = r.attn
        e_out = np.max(np.abs(g_out[n] - A.out))
        assert e_out <= TOL_OUT, f"row {t}: out error {e_out}"
        rep.bump("out_abs", e_out)
        for name, gv, ov in (("lse", g_lse[n], A.lse), ("lse_nc", g_lnc[n], A.lse_nc)):
            fin = np.isfinite(ov)
            assert np.array_equal(np.isfinite(gv), fin), f"row {t}: {name} finiteness"
            e = np.abs(gv[fin] - ov[fin])
            assert np.all(e <= REL * np.abs(ov[fin]) + 1e-6), f"row {t}: {name} error {e.max()}"
            rep.bump(name + "_abs", e.max() if e.size else 0)
        if g_cm is not None:
            e = np.abs(g_cm[n] - A.cmass)
            assert np.all(e <= REL * np.abs(A.cmass) + 1e-9), f"row {t}: cmass error {e.max()}"
            rep.bump("cmass_abs", e.max())
        if g_teach is not None:
            ot = r.teacher
            gt = g_teach[n, :len(ot)]
            e = np.abs(gt - ot)
            assert np.all(e <= REL * np.abs(ot) + 1e-9), f"row {t}: teacher error {e.max()}"
            assert np.all(g_teach[n, len(ot):] == 0), f"row {t}: teacher tail not 0"
            rep.bump("teacher_abs", e.max() if e.size else 0)
        e = abs(g_kl[n] - r.kl)
        assert e <= REL * abs(r.kl) + 1e-8, f"row {t}: KL {g_kl[n]} vs {r.kl}"
        rep.bump("kl_abs", e)
    return rep


def recall_all_rows(inp, res, chunk=4096):
    """Top-k recall of every row against torch.topk in fp32 on the GPU over the row's
    causally visible keys: the fraction of the selected keys whose score is at least
    the reference K_t-th largest.  Every row must also hold exactly K_t valid ids.
    Returns (mean, min)."""
    return recall_rows(inp, res["scores"], res["ids"], None, strict=True, chunk=chunk)


def recall_rows(inp, scores, ids, rows=None, strict=False, chunk=4096):
    """Recall of `ids` ([len(rows), k] global ids of the batch `inp`) for the batch rows
    `rows` (all rows if None) against torch.topk of the batch `scores` over each row's
    causally visible keys.  strict: also require exactly K_t valid ids per row."""
    wl = inp.wl
    sc = scores
    dev = sc.device
    T = wl.total_q
    cu_q = inp.cu_q.cpu().tolist()
    cu_k = inp.cu_k.cpu().tolist()
    seg = torch.zeros(T, dtype=torch.long)
    for s in range(len(cu_q) - 1):
        seg[cu_q[s]:cu_q[s + 1]] = s
    seg = seg.to(dev)
    cu_q_t = torch.tensor(cu_q, device=dev)
    cu_k_t = torch.tensor(cu_k, device=dev)
    off = inp.offsets.to(dev).long()
    local = torch.arange(T, device=dev) - cu_q_t[seg]
    pos = local + 1 + off[seg]
    s_k = (cu_k_t[1:] - cu_k_t[:-1])[seg]
    n_valid = torch.clamp(torch.div(pos, wl.ratio, rounding_mode="floor"), min=0)
    n_valid = torch.minimum(n_valid, s_k)
    row_idx = torch.arange(T, device=dev) if rows is None else torch.tensor(list(rows), device=dev)
    k_eff = min(wl.topk, wl.max_seqlen_k)
    recalls = []
    for r0 in range(0, row_idx.numel(), chunk):
        r1 = min(row_idx.numel(), r0 + chunk)
        ri = row_idx[r0:r1]
        x = sc.index_select(0, ri)[:, :wl.max_seqlen_k].clone()
        cols = torch.arange(wl.max_seqlen_k, device=dev)[None, :]
        nv = n_valid[ri]
        x = torch.where(cols < nv[:, None], x, torch.full_like(x, -float("inf")))
        kt = torch.clamp(nv, max=k_eff)
        vals = torch.topk(x, k_eff, dim=1).values                      # [rows, k_eff]
        kth = vals.gather(1, torch.clamp(kt - 1, min=0)[:, None]).squeeze(1)
        gid = ids[r0:r1].long()
        base = cu_k_t[seg[ri]][:, None]
        loc = torch.where(gid >= 0, gid - base, torch.zeros_like(gid))
        picked = x.gather(1, loc)
        ok = (gid >= 0) & (picked >= kth[:, None])
        cnt = ok.sum(1).float()
        has = kt > 0
        rec = torch.where(has, cnt / torch.clamp(kt.float(), min=1), torch.ones_like(cnt))
        if strict:
            nvalid_ids = (gid >= 0).sum(1)
            assert torch.equal(nvalid_ids, kt), "a row holds a wrong number of valid ids"
        recalls.append(rec)
    rec = torch.cat(recalls)
    return float(rec.mean()), float(rec.min())
