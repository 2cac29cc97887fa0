"""CPU tests of the GPU parity checker (tests/gpu_check.py): it must pass exact results and
catch planted mistakes of the kinds the attention, teacher and KL kernels could make.

A "perfect" result is built from the oracle itself, rounded to what the GPU returns (bf16
output, fp32 scores, statistics, teacher masses and KL; the KL taken from the fp32 teacher
masses and scores, as the KL kernel does).  Then one mistake at a time is planted in every
row and the checker's per-row verdict is counted:
  * an all-zero output, or two 16-byte pieces of V swapped (a wrong transposing read or
    swizzle): caught on every row;
  * the P.V contribution of the first compressed chunk dropped (a skipped chunk): caught on
    nearly every row that has one;
  * the compressed-only teacher in the KL (the bug the pages report): caught on nearly
    every row whose heads weigh the window and sink differently;
  * a KL off by 3e-5 relative (an fp32 slip in the log-ratio): caught on every row with a
    KL above 1e-9, which the former 1e-8 absolute floor let through on most rows;
  * unwritten outputs (NaN from the poisoned allocation): caught.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from deepseek_v4_csa_amd import inputs as I
from tests import gpu_check as C


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


def _perfect(wl, family="exact", seed=None, qmul=1.0):
    """Inputs on the CPU and the oracle's results rounded as the GPU returns them (qmul
    scales q, so that heads prefer different keys)."""
    inp = I.make_inputs(wl, device="cpu", family=family, seed=seed)
    if qmul != 1.0:
        inp.q = (inp.q.float() * qmul).to(inp.q.dtype)
    from tests.oracle_bridge import problem_of
    P = problem_of(inp)
    L = P.layout
    T, k_eff = wl.total_q, oracle.k_eff_of(L, wl.topk)
    sc = np.full((T, wl.max_seqlen_k), -np.inf, dtype=np.float32)
    ids = np.full((T, k_eff), -1, dtype=np.int32)
    out = np.zeros((T, wl.H, wl.D))
    lse = np.zeros((T, wl.H), dtype=np.float32)
    lnc = np.zeros((T, wl.H), dtype=np.float32)
    cm = np.zeros((T, k_eff), dtype=np.float32)
    te = np.zeros((T, k_eff), dtype=np.float32)
    kl = np.zeros(T, dtype=np.float32)
    attn = []
    for t in range(T):
        g = oracle.row_geometry(L, t)
        s_k = int(L.cu_k[g.seg + 1]) - g.k_base
        s = oracle.indexer_scores_row(P.q_idx[t], P.weights[t], P.k_idx[g.k_base:g.k_base + s_k], P.idx_scale,
                                      g.n_valid).astype(np.float32)
        sc[t, :s_k] = s
        ids[t] = oracle.topk_row(s.astype(np.float64), g.n_valid, k_eff, g.k_base)
        r = oracle.run_row(P, t, ids_override=ids[t])
        attn.append(r.attn)
        out[t] = r.attn.out
        lse[t], lnc[t], cm[t] = r.attn.lse, r.attn.lse_nc, r.attn.cmass
        v = ids[t] >= 0
        if g.n_valid:
            tt = oracle.teacher_from_mass(cm[t][v].astype(np.float64))
            te[t][v] = tt
            kl[t] = oracle.kl_row(tt, oracle.predictor(sc[t][ids[t][v] - g.k_base].astype(np.float64)))
    res = dict(scores=torch.from_numpy(sc), ids=torch.from_numpy(ids), out=_bf16(out),
               lse=torch.from_numpy(lse), lse_nc=torch.from_numpy(lnc), cmass=torch.from_numpy(cm),
               teacher=torch.from_numpy(te), kl_row=torch.from_numpy(kl),
               loss=torch.tensor([float(np.sum(kl.astype(np.float64)) / T)], dtype=torch.float32))
    return inp, P, res, attn, out


WL = {
    "bshd-small": I.scaled_down(I.WORKLOADS[1], (300, 140), topk=40),
    "long-small": I.scaled_down(I.WORKLOADS[3], (160,), topk=48),
}
# (workload, indexer input family): the exact family gives large, integer scores and a
# peaked predictor; the Gaussian one the small KLs of the workload draws
CASES = {"bshd-small-exact": ("bshd-small", "exact"), "long-small-gauss": ("long-small", "gauss")}
_EXACT = {}


@pytest.fixture(scope="module", params=sorted(CASES))
def perfect(request):
    name, family = CASES[request.param]
    r = _perfect(WL[name], family=family)
    _EXACT[id(r[0])] = family == "exact"
    return (request.param,) + r


@pytest.fixture(scope="module")
def peaky():
    """bshd-small with q scaled by 32: the heads' compressed distributions differ, so the
    window and sink terms of Z_h reweight them (as in the GPU perturbation test)."""
    r = _perfect(WL["bshd-small"], qmul=32.0)
    _EXACT[id(r[0])] = True
    return r


def _verdicts(inp, res, rows):
    ck = C.Checker(inp, res, rows, exact_scores=_EXACT[id(inp)])
    return {t: ck.row(t).fails for t in rows}


def test_perfect_result_passes(perfect):
    name, inp, P, res, attn, out = perfect
    rep = C.check_rows(inp, res, list(range(inp.wl.total_q)), exact_scores=_EXACT[id(inp)], loss_rows=True)
    assert rep["out_over_bound"] < 1.0


def _plant_out(res, new_out):
    r = dict(res)
    r["out"] = _bf16(new_out)
    return r


def test_zero_output_caught_on_every_row(perfect):
    name, inp, P, res, attn, out = perfect
    rows = list(range(inp.wl.total_q))
    v = _verdicts(inp, _plant_out(res, np.zeros_like(out)), rows)
    assert all(v[t] for t in rows), [t for t in rows if not v[t]][:10]


def test_swapped_value_pieces_caught_on_every_row(perfect):
    name, inp, P, res, attn, out = perfect
    bad = out.copy()
    bad[:, :, 0:8], bad[:, :, 8:16] = out[:, :, 8:16], out[:, :, 0:8]
    rows = list(range(inp.wl.total_q))
    v = _verdicts(inp, _plant_out(res, bad), rows)
    assert all(v[t] for t in rows), [t for t in rows if not v[t]][:10]


def test_dropped_compressed_chunk_caught(perfect):
    """out without the P.V terms of the first 32 compressed slots (lse and cmass intact)."""
    name, inp, P, res, attn, out = perfect
    ids = res["ids"].numpy()
    bad = out.copy()
    rows = []
    for t in range(inp.wl.total_q):
        sl = ids[t, :32]
        v = sl >= 0
        if v.sum() < 8:
            continue
        A = attn[t]
        pc = np.exp(A.c[:, :int(v.sum())] - A.lse[:, None])    # the valid slots come first in c
        bad[t] = out[t] - pc @ np.asarray(P.ckv[sl[v]], dtype=np.float64)
        rows.append(t)
    assert len(rows) > 50
    verdict = _verdicts(inp, _plant_out(res, bad), rows)
    caught = sum(1 for t in rows if verdict[t])
    assert caught / len(rows) >= 0.98, (caught, len(rows))


def test_compressed_only_teacher_caught(peaky):
    """The KL of the compressed-only teacher (softmax over the selected keys per head,
    without the window and sink terms in Z_h).  With near-uniform heads (the plain
    workload draws) the two teachers agree to second order, so heads with distinct
    preferences are used."""
    inp, P, res, attn, out = peaky
    C.check_rows(inp, res, list(range(inp.wl.total_q)), exact_scores=True, loss_rows=True)
    ids, sc = res["ids"].numpy(), res["scores"].numpy()
    kl = res["kl_row"].numpy().copy()
    rows = []
    for t in range(inp.wl.total_q):
        v = ids[t] >= 0
        if v.sum() < 2:
            continue
        g = oracle.row_geometry(P.layout, t)
        c = attn[t].c
        p_co = np.exp(c - oracle._logsumexp(c, axis=1)[:, None])
        t_co = oracle.teacher_from_mass(p_co.sum(axis=0))
        kl[t] = oracle.kl_row(t_co, oracle.predictor(sc[t][ids[t][v] - g.k_base].astype(np.float64)))
        rows.append(t)
    r = dict(res)
    r["kl_row"] = torch.from_numpy(kl.astype(np.float32))
    verdict = _verdicts(inp, r, rows)
    caught = sum(1 for t in rows if verdict[t])
    assert caught / len(rows) >= 0.95, (caught, len(rows))


def test_small_relative_kl_slip_caught(perfect):
    name, inp, P, res, attn, out = perfect
    kl = res["kl_row"].numpy().astype(np.float64)
    rows = [t for t in range(inp.wl.total_q) if kl[t] > 1e-9]
    assert len(rows) > 50
    if _EXACT[id(inp)]:
        pytest.skip("the exact family's KLs are large; the small-KL regime is the Gaussian case")
    r = dict(res)
    r["kl_row"] = torch.from_numpy((kl * (1 + 3e-5)).astype(np.float32))
    verdict = _verdicts(inp, r, rows)
    assert all(verdict[t] for t in rows), [t for t in rows if not verdict[t]][:10]
    # the former tolerance 1e-5 |KL| + 1e-8 let most of these rows through
    old_pass = sum(1 for t in rows if abs(kl[t] * 3e-5) <= 1e-5 * kl[t] + 1e-8)
    assert old_pass > len(rows) // 2


@pytest.mark.parametrize("key", ["out", "lse", "cmass", "teacher", "kl_row"])
def test_unwritten_output_caught(perfect, key):
    name, inp, P, res, attn, out = perfect
    r = dict(res)
    x = res[key].clone()
    t = inp.wl.total_q - 3
    x[t] = float("nan")
    r[key] = x
    assert _verdicts(inp, r, [t])[t]
