"""Row-by-row comparison of the HIP path against the CPU oracle (test helper).

Tolerances (written here, used by every GPU parity test).  u = 2^-24 is the fp32 unit
roundoff, u_bf = 2^-8 the bf16 one.

  scores    exact-integer family: bit-exact.  Gaussian: |I_gpu - I_oracle| <= B_tj with
            B_tj = gamma * sum_h ws_h * sum_d |q_hd k_jd|, gamma = (Di + Hi + 2) * u,
            the worst-case fp32 accumulation error of Di + Hi + 2 rounded operations.
  ids       bit-exact against the oracle's top-k of the GPU's own fp32 score row
            (identical inputs to the selection); end-to-end bit-exact on the exact family.
  out       per element |out_gpu - out_oracle| <= 2e-2 (absolute, the stated bar) AND
            <= beta * A_hd with A_hd = sum_r P_hr |V_rd| (the probability-weighted sum of
            the value magnitudes over the row's window and compressed rows):
              bf16: beta = 2 u_bf + u (4 n + 256).  P is rounded to bf16 before the P.V
                    product (|dP| <= u_bf P, so |d(sum P V)| <= u_bf A) and the output is
                    stored in bf16 (|d out| <= u_bf |out| <= u_bf A); the fp32 logits,
                    exponentials, the row sum over n = |window| + K_t terms and the fp32
                    accumulation stay below u (4 n + 256) A.
              fp32: beta = u (4 n + 256) (no bf16 rounding anywhere).
            A wrong, missing or permuted value row moves out by a multiple of sum P V, which
            is of the order of A itself, so this catches P.V mistakes an absolute bound on
            small outputs cannot.
  lse, lse_nc  |delta| <= 1e-5 * |x| + 1e-6.
  cmass, teacher  |delta| <= 1e-5 * |x| + 1e-9 per element, on identical ids.
  kl_row    two checks, on identical ids:
            step:  the oracle's teacher/predictor/KL (float64) applied to the very fp32
                   values the KL kernel reads -- cmass and the selected scores (sparse
                   loss), or the GPU's fp32 teacher (renormalised in fp64) and score row
                   (dense loss) -- |dKL| <= 1e-5 |KL| + 1e-12, plus, in the dense case
                   only, the first-order effect of the fp32 rounding of the teacher the
                   oracle reads, 2u sum_j t_j |L_j - KL|.  This is the 1e-5 relative bar on
                   the KL step.
            end to end (the oracle from the raw inputs):
                   |dKL| <= 1e-5 |KL| + F_t, with F_t the first-order change of the KL that
                   the tolerances of its inputs allow.  Writing L_j = log((t_j+e)/(p_j+e)):
                   a teacher change dt with sum dt = 0 moves the KL by
                   sum_j dt_j (L_j + 1) = sum_j dt_j (L_j - KL), and a score change dI moves
                   log p_j by dI_j - sum_i p_i dI_i, hence the KL by sum_j (p_j - t_j) dI_j.
                   With |dt_j| <= 1e-5 t_j + 1e-9 (the teacher tolerance) and |dI_j| <= B_tj:
                   F_t = sum_j (1e-5 t_j + 1e-9) |L_j - KL| + sum_j |p_j - t_j| B_tj.
                   fp32 teacher masses carry relative errors near 1e-6, and for nearly
                   equal t and p the KL is second order in t - p, so the first term can
                   exceed 1e-5 |KL|: that is the reason for F_t.
  loss      |loss_gpu - mean_t KL_step| <= 1e-5 |loss| + 1e-12 (every row of the small
            workloads), and |loss_gpu - oracle loss| <= 1e-5 |loss| + mean_t F_t.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

import oracle
from tests.oracle_bridge import host, problem_of

TOL_OUT = 2e-2
REL = 1e-5
U32 = 2.0 ** -24
U_BF16 = 2.0 ** -8
KL_FLOOR = 1e-12

# worst figures of the session, printed by the terminal-summary hook of conftest.py
WORST: dict = {}


def record(tag: str, rep: dict):
    d = WORST.setdefault(tag, {})
    for k, v in rep.items():
        d[k] = max(d.get(k, 0.0), float(v))


def score_band(P, t, g):
    """Worst-case fp32 accumulation bound of every score of row t."""
    L = P.layout
    k = np.abs(np.asarray(P.k_idx[g.k_base:int(L.cu_k[g.seg + 1])], dtype=np.float64))
    q = np.abs(np.asarray(P.q_idx[t], dtype=np.float64))
    ws = np.abs(oracle.indexer_weight_scale(P.weights[t], P.idx_scale).astype(np.float64))
    Hi, Di = q.shape
    gamma = (Di + Hi + 2) * U32
    return gamma * ((k @ q.T) @ ws) + 1e-30


def value_scale(P, t, g, attn, ids_row):
    """A_hd = sum_r P_hr |V_rd| over the row's window and valid compressed rows, from the
    oracle's logits and lse (the scale of the output's rounding error)."""
    win = oracle.window_rows(t, g.q_start, P.window)
    ids = np.asarray(ids_row)
    valid = ids[ids >= 0]
    D = attn.out.shape[1]
    lse = attn.lse.reshape(-1, 1)
    fin = np.isfinite(lse[:, 0])
    A = np.zeros_like(attn.out)
    if len(win):
        pw = np.where(fin[:, None], np.exp(attn.w - np.where(fin[:, None], lse, 0.0)), 0.0)
        A += pw @ np.abs(np.asarray(P.kv[win], dtype=np.float64).reshape(len(win), D))
    if len(valid):
        pc = np.where(fin[:, None], np.exp(attn.c - np.where(fin[:, None], lse, 0.0)), 0.0)
        A += pc @ np.abs(np.asarray(P.ckv[valid], dtype=np.float64).reshape(len(valid), D))
    return A, len(win) + len(valid)


def out_bound(A, n, fp32: bool):
    beta = U32 * (4 * n + 256) + (0.0 if fp32 else 2 * U_BF16)
    return beta * A + 1e-30


def kl_sensitivity(teacher, pred, kl, band, tol_rel=REL, tol_abs=1e-9):
    """F_t: the first-order KL change that teacher errors |dt_j| <= tol_rel t_j + tol_abs
    and score errors |dI_j| <= band_j allow (derivation in the module docstring)."""
    t = np.asarray(teacher, dtype=np.float64)
    p = np.asarray(pred, dtype=np.float64)
    if t.size == 0:
        return 0.0
    Lj = np.log(t + oracle.EPS_LOG) - np.log(p + oracle.EPS_LOG)
    f = np.sum((tol_rel * t + tol_abs) * np.abs(Lj - kl))
    return float(f + np.sum(np.abs(p - t) * np.asarray(band, dtype=np.float64)))


@dataclass
class RowCheck:
    """Failures of one row (empty: the row passes) and its error figures."""
    t: int
    fails: list = field(default_factory=list)
    stats: dict = field(default_factory=dict)
    kl_step: float = 0.0      # the oracle's KL on the GPU's own fp32 inputs
    kl_oracle: float = 0.0    # the oracle's KL from the raw inputs
    f_t: float = 0.0          # end-to-end KL floor


class Checker:
    """Per-row comparison of one forward result against the oracle.

    res: dict of ops.forward (scores or sel, ids, out, lse, lse_nc, cmass, teacher,
    kl_row); only the rows given are copied to the host."""

    def __init__(self, inp, res, rows, exact_scores=False, check_scores=True, dense=None):
        self.inp = inp
        self.wl = inp.wl
        self.rows = list(rows)
        self.P = problem_of(inp, self.rows)
        self.dense = (not self.wl.sparse_loss) if dense is None else dense
        self.exact = exact_scores
        self.check_scores = check_scores and res.get("scores") is not None
        self.fp32 = inp.q.dtype == torch.float32
        self.k_eff = oracle.k_eff_of(self.P.layout, self.P.topk)
        dev = res["ids"].device
        idx = torch.tensor(self.rows, dtype=torch.long, device=dev)
        take = lambda x: host(x.index_select(0, idx)) if x is not None else None
        self.sc = take(res.get("scores"))
        self.sel = take(res.get("sel"))
        self.ids = res["ids"].index_select(0, idx).cpu().numpy().astype(np.int64)
        self.out = take(res["out"])
        self.lse = take(res["lse"])
        self.lnc = take(res["lse_nc"])
        self.cm = take(res.get("cmass"))
        self.teach = take(res.get("teacher"))
        self.kl = take(res["kl_row"])
        self.pos = {t: n for n, t in enumerate(self.rows)}

    def row(self, t) -> RowCheck:
        n = self.pos[t]
        P, L, wl = self.P, self.P.layout, self.wl
        rc = RowCheck(t)
        g = oracle.row_geometry(L, t)
        s_k = int(L.cu_k[g.seg + 1]) - g.k_base
        o_sc = oracle.indexer_scores_row(P.q_idx[t], P.weights[t], P.k_idx[g.k_base:g.k_base + s_k],
                                         P.idx_scale, g.n_valid)
        band = np.zeros(s_k) if self.exact else score_band(P, t, g)
        # ---- scores (full rows) or the selected scores
        if self.sc is not None:
            gs = self.sc[n, :s_k]
            if not np.all(gs[g.n_valid:] == -np.inf):
                rc.fails.append("masked columns not -inf")
            if wl.max_seqlen_k > s_k and not np.all(self.sc[n, s_k:wl.max_seqlen_k] == -np.inf):
                rc.fails.append("tail not -inf")
            if self.check_scores and g.n_valid:
                d = np.abs(gs[:g.n_valid] - o_sc[:g.n_valid])
                if self.exact:
                    if not np.all(d == 0):
                        rc.fails.append(f"exact-family score differs by {d.max()}")
                else:
                    b = band[:g.n_valid]
                    if not np.all(d <= b):
                        rc.fails.append(f"score error {d.max()} above band")
                    rc.stats["score_err_over_band"] = float(np.max(d / b))
            o_ids = oracle.topk_row(gs, g.n_valid, self.k_eff, g.k_base)
            if not np.array_equal(o_ids, self.ids[n]):
                rc.fails.append("ids differ from the oracle top-k of the same scores")
        ids = self.ids[n]
        valid = ids >= 0
        if self.exact:
            o_ids2 = oracle.topk_row(o_sc, g.n_valid, self.k_eff, g.k_base)
            if not np.array_equal(o_ids2, ids):
                rc.fails.append("exact-family ids differ end to end")
        # GPU scores as the KL kernel reads them
        if self.dense:
            g_pred_in = self.sc[n, :g.n_valid] if self.sc is not None else None
        elif self.sel is not None:
            g_pred_in = self.sel[n, :self.k_eff][valid]
        else:
            g_pred_in = self.sc[n][ids[valid] - g.k_base]
        if self.sel is not None and not self.dense:
            sv = self.sel[n, :self.k_eff]
            if not np.all(sv[~valid] == -np.inf):
                rc.fails.append("selected scores at -1 slots not -inf")
            d = np.abs(sv[valid] - o_sc[ids[valid] - g.k_base])
            if self.exact and not np.all(d == 0):
                rc.fails.append("exact-family selected score differs")
            if not self.exact and not np.all(d <= band[ids[valid] - g.k_base]):
                rc.fails.append(f"selected score error {d.max()} above band")
        # ---- attention, teacher, KL on identical ids
        r = oracle.run_row(P, t, ids_override=ids)
        A = r.attn
        e = np.abs(self.out[n] - A.out)
        Ascale, nrow = value_scale(P, t, g, A, ids)
        bnd = out_bound(Ascale, nrow, self.fp32)
        if not np.all(e <= TOL_OUT):
            rc.fails.append(f"out error {e.max()} above {TOL_OUT}")
        if not np.all(e <= bnd):
            k = np.unravel_index(np.argmax(e / bnd), e.shape)
            rc.fails.append(f"out error {e[k]:.3e} above its rounding bound {bnd[k]:.3e} at (h, d) = {k}")
        rc.stats["out_abs"] = float(e.max())
        rc.stats["out_over_bound"] = float(np.max(e / bnd))
        for name, gv, ov in (("lse", self.lse[n], A.lse), ("lse_nc", self.lnc[n], A.lse_nc)):
            fin = np.isfinite(ov)
            if not np.array_equal(np.isfinite(gv), fin):
                rc.fails.append(f"{name} finiteness")
                continue
            err = np.abs(gv[fin] - ov[fin])
            if not np.all(err <= REL * np.abs(ov[fin]) + 1e-6):
                rc.fails.append(f"{name} error {err.max()}")
            rc.stats[name + "_abs"] = float(err.max()) if err.size else 0.0
        if self.cm is not None:
            err = np.abs(self.cm[n] - A.cmass)
            if not np.all(err <= REL * np.abs(A.cmass) + 1e-9):
                rc.fails.append(f"cmass error {err.max()}")
            rc.stats["cmass_rel"] = float(np.max(err / np.maximum(np.abs(A.cmass), 1e-30) * (A.cmass != 0)))
        if self.teach is not None:
            ot = r.teacher
            gt = self.teach[n, :len(ot)]
            err = np.abs(gt - ot)
            if not np.all(err <= REL * np.abs(ot) + 1e-9):
                rc.fails.append(f"teacher error {err.max()}")
            if not np.all(self.teach[n, len(ot):] == 0):
                rc.fails.append("teacher tail not 0")
            rc.stats["teacher_abs"] = float(err.max()) if err.size else 0.0
        # ---- KL: step level (identical fp32 inputs) and end to end
        g_kl = float(self.kl[n])
        empty = g.n_valid == 0 or g.padding
        step_floor = KL_FLOOR
        if empty:
            kl_step = 0.0
        elif self.dense:
            if self.teach is None or g_pred_in is None:
                kl_step = None
            else:
                # the kernel's teacher is normalised in fp64; rounding each value to fp32
                # for the output leaves its sum off 1 by up to n u, which would move the KL
                # by as much in absolute terms, so the oracle renormalises it first
                tt = self.teach[n, :g.n_valid]
                tt = tt / np.sum(tt)
                pp = oracle.predictor(g_pred_in)
                kl_step = oracle.kl_row(tt, pp)
                step_floor += kl_sensitivity(tt, pp, kl_step, np.zeros(len(pp)), tol_rel=2 * U32, tol_abs=0.0)
        else:
            if self.cm is None:
                kl_step = None
            else:
                tt = oracle.teacher_from_mass(self.cm[n][valid])
                kl_step = oracle.kl_row(tt, oracle.predictor(g_pred_in))
        if kl_step is not None:
            d = abs(g_kl - kl_step)
            if not d <= REL * abs(kl_step) + step_floor:
                rc.fails.append(f"KL step: {g_kl} vs {kl_step} (|d| = {d:.3e})")
            rc.kl_step = kl_step
            if abs(kl_step) > 1e-30:
                rc.stats["kl_step_rel"] = d / abs(kl_step)
        if empty:
            f_t = 0.0
        elif self.dense:
            f_t = kl_sensitivity(r.teacher, r.pred, r.kl, band[:g.n_valid])
        else:
            f_t = kl_sensitivity(r.teacher[valid], r.pred[valid], r.kl, band[ids[valid] - g.k_base])
        d = abs(g_kl - r.kl)
        if not d <= REL * abs(r.kl) + f_t + KL_FLOOR:
            rc.fails.append(f"KL end to end: {g_kl} vs {r.kl} (|d| = {d:.3e}, floor {f_t:.3e})")
        if abs(r.kl) > 1e-30:
            rc.stats["kl_e2e_rel"] = d / abs(r.kl)
        rc.stats["kl_e2e_over_bound"] = d / (REL * abs(r.kl) + f_t + KL_FLOOR)
        rc.kl_oracle, rc.f_t = r.kl, f_t
        return rc


class Report(dict):
    def bump(self, key, val):
        self[key] = max(self.get(key, 0.0), float(val))


def check_rows(inp, res, rows, exact_scores=False, check_scores=True, dense=None, tag=None, loss_rows=False):
    """Compare GPU results `res` (dict from ops.forward with want_teacher) with the oracle on
    `rows`.  Raises AssertionError on the first violating row; returns the worst error
    figures.  loss_rows=True (rows = every row of the batch): also checks res["loss"]
    against the oracle's loss (step level and end to end)."""
    ck = Checker(inp, res, rows, exact_scores, check_scores, dense)
    rep = Report()
    kls, klo, fts = [], [], []
    for t in ck.rows:
        rc = ck.row(t)
        assert not rc.fails, f"row {t}: " + "; ".join(rc.fails)
        for k, v in rc.stats.items():
            rep.bump(k, v)
        kls.append(rc.kl_step)
        klo.append(rc.kl_oracle)
        fts.append(rc.f_t)
    if loss_rows:
        T = inp.wl.total_q
        assert len(ck.rows) == T, "the loss check needs every row"
        g_loss = float(res["loss"][0])
        per_tok = False
        l_step = oracle.reduce_loss(kls, T, per_tok)
        l_or = oracle.reduce_loss(klo, T, per_tok)
        d1, d2 = abs(g_loss - l_step), abs(g_loss - l_or)
        assert d1 <= REL * abs(l_step) + KL_FLOOR, f"loss step: {g_loss} vs {l_step}"
        assert d2 <= REL * abs(l_or) + float(np.sum(fts)) / T + KL_FLOOR, f"loss end to end: {g_loss} vs {l_or}"
        if l_step:
            rep.bump("loss_step_rel", d1 / abs(l_step))
        if l_or:
            rep.bump("loss_e2e_rel", d2 / abs(l_or))
    if tag:
        record(tag, rep)
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
