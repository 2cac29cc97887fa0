"""CPU pins of the oracle's attention, teacher, KL and loss reduction."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from tests import tiny

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows_with_keys(P, n=12):
    L = P.layout
    rows = [t for t in range(L.total_q) if oracle.row_geometry(L, t).n_valid > 0]
    return rows[:: max(1, len(rows) // n)]


# ----------------------------------------------------------------------------- attention
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_two_attention_formulations_agree(seed):
    """Explicit softmax over [sink | window | compressed] (the Z_h equation) against the
    LSE decomposition u_h -> l_h of the proposal comment: same lse, lse_nc, out, and
    the per-head compressed probabilities summed over heads."""
    P = tiny.problem(seg_lens=(40, 28), H=4, D=8, topk=5, window=6, seed=seed)
    L = P.layout
    k_eff = oracle.k_eff_of(L, P.topk)
    for t in range(L.total_q):
        g = oracle.row_geometry(L, t)
        sc = oracle.indexer_scores_row(P.q_idx[t], P.weights[t], P.k_idx[g.k_base:int(L.cu_k[g.seg + 1])], P.idx_scale, g.n_valid)
        ids = oracle.topk_row(sc, g.n_valid, k_eff, g.k_base)
        win = oracle.window_rows(t, g.q_start, P.window)
        A = oracle.attention_row(P.q[t], P.kv, P.ckv, P.sink, ids, win, P.scale)
        lse, u, p, pw, out = oracle.attention_row_lse_form(P.q[t], P.kv, P.ckv, P.sink, ids, win, P.scale)
        np.testing.assert_allclose(A.lse, lse, rtol=0, atol=1e-12)
        np.testing.assert_allclose(A.lse_nc, u, rtol=0, atol=1e-12)
        np.testing.assert_allclose(A.out, out, rtol=0, atol=1e-12)
        np.testing.assert_allclose(A.cmass[ids >= 0], p.sum(axis=0), rtol=0, atol=1e-12)
        assert np.all(A.cmass[ids < 0] == 0)


def test_no_window_no_sink_full_selection_is_causal_softmax_attention():
    """W = 0, sink = -inf and top-k >= every row's visible keys reduce the path to plain
    causal softmax attention over the compressed KV, which torch computes on the CPU
    with an explicit boolean mask."""
    S, ratio, H, D = 64, 4, 3, 8
    P = tiny.problem(seg_lens=(S,), ratio=ratio, H=H, D=D, topk=64, window=0,
                     sink=[-np.inf] * H, seed=4)
    L = P.layout
    Tk = L.total_k
    q = torch.from_numpy(P.q).permute(1, 0, 2).unsqueeze(0)             # [1, H, S, D]
    kk = torch.from_numpy(P.ckv)[None, None].expand(1, H, Tk, D)
    mask = torch.zeros(S, Tk, dtype=torch.bool)
    for t in range(S):
        mask[t, : oracle.row_geometry(L, t).n_valid] = True
    ref = torch.nn.functional.scaled_dot_product_attention(q, kk, kk, attn_mask=mask, scale=P.scale)
    ref = ref[0].permute(1, 0, 2).numpy()
    for t in range(S):
        r = oracle.run_row(P, t)
        if r.geom.n_valid == 0:
            assert np.all(r.attn.out == 0) and np.all(r.attn.lse == -np.inf)
            continue
        np.testing.assert_allclose(r.attn.out, ref[t], rtol=0, atol=1e-12)


def test_sink_closed_form():
    """Adding a sink a to a row that has none scales every probability by
    Z'/(Z' + e^a) and sets lse = logaddexp(lse', a)."""
    P0 = tiny.problem(seg_lens=(48,), H=3, topk=6, window=5, sink=[-np.inf] * 3, seed=6)
    a = np.array([0.7, -1.3, 2.0])
    P1 = tiny.problem(seg_lens=(48,), H=3, topk=6, window=5, sink=a, seed=6)
    for t in _rows_with_keys(P0):
        r0, r1 = oracle.run_row(P0, t), oracle.run_row(P1, t)
        np.testing.assert_allclose(r1.attn.lse, np.logaddexp(r0.attn.lse, a), rtol=0, atol=1e-12)
        f = np.exp(r0.attn.lse - r1.attn.lse)[:, None]
        np.testing.assert_allclose(r1.attn.out, r0.attn.out * f, rtol=0, atol=1e-12)
        np.testing.assert_allclose(r1.attn.lse_nc, np.logaddexp(r0.attn.lse_nc, a), rtol=0, atol=1e-12)


def test_sink_only_row_and_lse_nc_limits():
    P = tiny.problem(seg_lens=(16,), H=2, topk=4, window=0, sink=[0.5, -0.25], seed=7)
    r = oracle.run_row(P, 0)                                   # no key, no window
    assert np.all(r.attn.out == 0)
    np.testing.assert_allclose(r.attn.lse, [0.5, -0.25])
    np.testing.assert_allclose(r.attn.lse_nc, [0.5, -0.25])
    Pn = tiny.problem(seg_lens=(32,), H=2, topk=4, window=3, seed=8)
    ids = np.full(4, -1)
    g = oracle.row_geometry(Pn.layout, 20)
    win = oracle.window_rows(20, g.q_start, 3)
    A = oracle.attention_row(Pn.q[20], Pn.kv, Pn.ckv, Pn.sink, ids, win, Pn.scale)
    np.testing.assert_allclose(A.lse, A.lse_nc, rtol=0, atol=1e-14)    # no compressed key


def test_cmass_total_is_the_compressed_share_of_each_head():
    """sum_j cmass_j = sum_h (1 - exp(lse_nc_h - lse_h)) (each head's probabilities sum
    to one, and its sink+window share is exp(u_h - l_h))."""
    P = tiny.problem(seg_lens=(60,), H=4, topk=7, window=5, seed=9)
    for t in _rows_with_keys(P):
        A = oracle.run_row(P, t).attn
        np.testing.assert_allclose(A.cmass.sum(), np.sum(1 - np.exp(A.lse_nc - A.lse)), rtol=1e-12)


def test_window_rows_reading():
    """The reading: `window` most recent rows of the segment, the query row included."""
    assert list(oracle.window_rows(10, 0, 4)) == [7, 8, 9, 10]
    assert list(oracle.window_rows(10, 9, 4)) == [9, 10]
    assert list(oracle.window_rows(10, 0, 0)) == []


# ----------------------------------------------------------------------------- teacher
def _two_head_problem(c, sink, win_logit):
    """H = 2, D = 3, scale 1: ckv rows are e1, e2 (two compressed keys), the kv row of
    the query is e3, so q[h] = (c_h0, c_h1, window logit) gives exactly those logits."""
    q = np.zeros((1, 2, 3))
    for h in range(2):
        q[0, h, :2] = c[h]
        q[0, h, 2] = win_logit[h] if np.isfinite(win_logit[h]) else -1e4
    kv = np.array([[0.0, 0.0, 1.0]])
    ckv = np.eye(3)[:2]
    return q, kv, ckv


def test_worked_two_head_example():
    g = json.load(open(os.path.join(GOLDEN, "teacher_worked_example.json")))
    for case in g["cases"]:
        c = [[tiny.parse(v) for v in row] for row in case["c"]]
        sink = np.array([tiny.parse(v) for v in case["sink"]])
        wl = [tiny.parse(v) for v in case["window_logit"]]
        q, kv, ckv = _two_head_problem(c, sink, wl)
        A = oracle.attention_row(q[0], kv, ckv, sink, np.array([0, 1]), np.array([0]), 1.0)
        t = oracle.teacher_sparse_row(A, np.array([0, 1]))
        want = [float(Fraction(a, b)) for a, b in case["teacher"]]
        np.testing.assert_allclose(t, want, rtol=0, atol=1e-12, err_msg=case["name"])


@pytest.mark.parametrize("sparse", [True, False])
def test_teacher_sums_to_one_on_rows_with_keys(sparse):
    P = tiny.problem(seg_lens=(52, 20), H=3, topk=6, window=4, seed=10, sparse=sparse)
    for t in range(P.layout.total_q):
        r = oracle.run_row(P, t)
        if r.geom.n_valid:
            assert abs(r.teacher.sum() - 1) < 1e-12
        else:
            assert r.kl == 0.0 and np.all(r.teacher == 0)


@pytest.mark.parametrize("sparse", [True, False])
def test_reduces_to_compressed_only_teacher_without_window_and_sink(sparse):
    """W empty and sink -inf: every Z_h holds only compressed terms, so the paper teacher
    must equal the compressed-only teacher built from whole masked matrices as the
    dsa.py excerpt does (the t-hat equation)."""
    S, ratio, H = 48, 4, 3
    P = tiny.problem(seg_lens=(S,), ratio=ratio, H=H, D=8, topk=5, window=0,
                     sink=[-np.inf] * H, seed=11, sparse=sparse)
    L = P.layout
    n_cmp = L.total_k
    rows = [oracle.run_row(P, t) for t in range(S)]
    causal = np.where(np.arange(n_cmp)[None, :] >= (np.arange(1, S + 1)[:, None] // ratio), -np.inf, 0.0)
    topk_local = np.stack([r.ids for r in rows])   # single segment: global == local
    ref = oracle.compressed_only_teacher(P.q, P.ckv, causal, topk_local, P.scale, sparse)
    for r in rows:
        if r.geom.n_valid == 0:
            assert np.all(ref[r.t] == 0)
            continue
        if sparse:
            got = np.zeros(n_cmp)
            v = r.ids >= 0
            got[r.ids[v]] = r.teacher[v]
        else:
            got = np.zeros(n_cmp)
            got[: r.geom.n_valid] = r.teacher
        np.testing.assert_allclose(got, ref[r.t], rtol=0, atol=1e-12)


def test_single_head_teacher_ignores_sink_and_window():
    """H = 1: Z_1 cancels in the L1 normalisation, t = softmax_C(c)."""
    P1 = tiny.problem(seg_lens=(40,), H=1, topk=5, window=4, sink=[3.0], seed=12)
    P2 = tiny.problem(seg_lens=(40,), H=1, topk=5, window=0, sink=[-np.inf], seed=12)
    for t in _rows_with_keys(P1):
        r1, r2 = oracle.run_row(P1, t), oracle.run_row(P2, t)
        v = r1.ids >= 0
        np.testing.assert_allclose(r1.teacher[v], oracle.predictor(r1.attn.c[0]), rtol=1e-12)
        np.testing.assert_allclose(r1.teacher, r2.teacher, rtol=1e-12, atol=1e-15)


def test_sparse_equals_dense_when_every_visible_key_is_selected():
    Ps = tiny.problem(seg_lens=(40, 24), H=3, topk=64, window=4, seed=13, sparse=True)
    Pd = tiny.problem(seg_lens=(40, 24), H=3, topk=64, window=4, seed=13, sparse=False)
    for t in range(Ps.layout.total_q):
        rs, rd = oracle.run_row(Ps, t), oracle.run_row(Pd, t)
        n = rs.geom.n_valid
        np.testing.assert_allclose(rs.teacher[:n], rd.teacher, rtol=0, atol=1e-12)
        assert abs(rs.kl - rd.kl) < 1e-12


def test_window_or_sink_perturbation_changes_teacher_not_selection():
    """[I5776, "Static reproduction / invariant"]: perturbing only the window values or
    one head's sink changes the teacher (two heads, several keys) while the indexer
    scores and the top-k selection stay bit-identical."""
    base = tiny.problem(seg_lens=(64,), H=2, topk=6, window=5, seed=14)
    sink2 = base.sink.copy(); sink2[0] += 2.0
    pert_sink = tiny.problem(seg_lens=(64,), H=2, topk=6, window=5, seed=14, sink=sink2)
    pert_win = tiny.problem(seg_lens=(64,), H=2, topk=6, window=5, seed=14)
    pert_win.kv = base.kv * 3.0
    moved_s = moved_w = 0
    for t in _rows_with_keys(base, n=20):
        r0 = oracle.run_row(base, t)
        for Pp in (pert_sink, pert_win):
            r1 = oracle.run_row(Pp, t)
            np.testing.assert_array_equal(r0.scores, r1.scores)
            np.testing.assert_array_equal(r0.ids, r1.ids)
        moved_s += np.max(np.abs(oracle.run_row(pert_sink, t).teacher - r0.teacher)) > 1e-6
        moved_w += np.max(np.abs(oracle.run_row(pert_win, t).teacher - r0.teacher)) > 1e-6
    assert moved_s > 0 and moved_w > 0


# ----------------------------------------------------------------------------- KL / loss
def test_kl_golden_values():
    g = json.load(open(os.path.join(GOLDEN, "kl_values.json")))
    for case in g["cases"]:
        t = np.array([float(Fraction(a, b)) for a, b in case["teacher"]])
        p = oracle.predictor([tiny.parse(v) for v in case["pred_logits"]])
        assert abs(oracle.kl_row(t, p) - case["kl"]) < g["tolerance_abs"], case["name"]


def test_kl_matches_scipy_rel_entr_and_vanishes_on_equal_distributions():
    rng = np.random.default_rng(15)
    for _ in range(30):
        n = int(rng.integers(2, 40))
        t = rng.random(n); t /= t.sum()
        p = oracle.predictor(rng.standard_normal(n))
        # the 1e-10 terms move each log by at most 1e-10/x, so the two may differ by
        # at most 1e-10 * sum_j (1 + t_j / p_j)
        bound = 1e-10 * np.sum(1 + t / p) * 1.01
        assert abs(oracle.kl_row(t, p) - scipy.special.rel_entr(t, p).sum()) <= bound
        assert oracle.kl_row(t, p) > -1e-9
        logits = np.log(t) + 3.7
        assert abs(oracle.kl_row(t, oracle.predictor(logits))) < 1e-9


def test_loss_reduction_counts_every_physical_row():
    P = tiny.problem(seg_lens=(20, 12), H=2, topk=3, window=2, seed=16)
    rows, loss = oracle.run_all(P)
    kls = [r.kl for r in rows]
    assert sum(1 for r in rows if r.geom.n_valid == 0) > 0
    assert abs(loss - sum(kls) / P.layout.total_q) < 1e-15
    P.per_token = True
    _, loss_sum = oracle.run_all(P)
    assert abs(loss_sum - sum(kls)) < 1e-12
