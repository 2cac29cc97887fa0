"""Whole-path invariants of the oracle, and planted mistakes that its pins must catch.

The second half plants plausible mistakes in the oracle (on the CPU only, through
monkeypatch) and checks that at least one pin fails for each -- evidence that the pins
constrain the oracle rather than restate it.
"""
import numpy as np
import pytest

import oracle
import oracle.csa_oracle as oc
from tests import test_oracle_attention_teacher_kl as A
from tests import test_oracle_geometry_indexer_topk as G
from tests import tiny


def _slice_problem(P, s):
    """The segment s of a packed problem as a standalone single-sequence problem."""
    L = P.layout
    q0, q1 = int(L.cu_q[s]), int(L.cu_q[s + 1])
    k0, k1 = int(L.cu_k[s]), int(L.cu_k[s + 1])
    Ls = tiny.layout([q1 - q0], L.ratio, off=[int(L.offsets()[s])], cu_k=[0, k1 - k0])
    return oracle.Problem(layout=Ls, q=P.q[q0:q1], kv=P.kv[q0:q1], ckv=P.ckv[k0:k1],
                          q_idx=P.q_idx[q0:q1], k_idx=P.k_idx[k0:k1], weights=P.weights[q0:q1],
                          sink=P.sink, topk=P.topk, window=P.window, scale=P.scale,
                          idx_scale=P.idx_scale, sparse_loss=P.sparse_loss)


@pytest.mark.parametrize("sparse", [True, False])
def test_packed_documents_equal_independent_runs(sparse):
    """[PR8539, item 2] / packed THD: no attention across documents; a packed run equals
    independent per-document runs, with global ids shifted by the segment's key base
    ([PR8539, item 1]: ids are global).  The topk is below every segment's key count so
    the shared k_eff = min(topk, max S_k) is the same in both runs."""
    P = tiny.problem(seg_lens=(36, 48, 28), H=3, topk=5, window=6, seed=21, sparse=sparse)
    L = P.layout
    for s in range(L.num_seqs):
        Ps = _slice_problem(P, s)
        for r in range(Ps.layout.total_q):
            a = oracle.run_row(P, int(L.cu_q[s]) + r)
            b = oracle.run_row(Ps, r)
            np.testing.assert_array_equal(a.scores, b.scores)
            shifted = np.where(b.ids >= 0, b.ids + int(L.cu_k[s]), -1)
            np.testing.assert_array_equal(a.ids, shifted)
            np.testing.assert_allclose(a.attn.out, b.attn.out, rtol=0, atol=1e-14)
            np.testing.assert_allclose(a.teacher, b.teacher, rtol=0, atol=1e-14)
            assert a.kl == pytest.approx(b.kl, abs=1e-14)


def test_batch_of_two_equals_two_single_runs():
    """[PR8539, item 1, test plan]: a micro-batch of 2 must match the same rows run as
    two b=1 calls, with the second batch's ids offset by S_k."""
    P = tiny.problem(seg_lens=(40, 40), H=2, topk=4, window=3, seed=22)
    S_k = 10
    for s in range(2):
        Ps = _slice_problem(P, s)
        for r in range(40):
            a, b = oracle.run_row(P, 40 * s + r), oracle.run_row(Ps, r)
            np.testing.assert_array_equal(a.ids, np.where(b.ids >= 0, b.ids + s * S_k, -1))
            assert a.kl == pytest.approx(b.kl, abs=1e-14)


def test_chunk_with_offset_selects_like_the_full_sequence():
    """[PR8539, item 2 and its test plan]: a query chunk scored against its key prefix
    with offset = chunk start selects exactly the full run's keys (recall 1.0); with
    the offsets removed the selection changes (negative control)."""
    S, c0 = 96, 56
    P = tiny.problem(seg_lens=(S,), H=2, Hi=3, topk=6, window=0, seed=23)
    L_right = tiny.layout([S - c0], 4, off=[c0], cu_k=[0, S // 4])
    L_left = tiny.layout([S - c0], 4, off=[0], cu_k=[0, S // 4])
    changed = 0
    for L in (L_right, L_left):
        Pc = oracle.Problem(layout=L, q=P.q[c0:], kv=P.kv[c0:], ckv=P.ckv, q_idx=P.q_idx[c0:],
                            k_idx=P.k_idx, weights=P.weights[c0:], sink=P.sink, topk=P.topk,
                            window=0, scale=P.scale, idx_scale=P.idx_scale)
        for r in range(S - c0):
            a, b = oracle.run_row(P, c0 + r), oracle.run_row(Pc, r)
            if L is L_right:
                np.testing.assert_array_equal(a.ids, b.ids)
            else:
                changed += not np.array_equal(a.ids, b.ids)
    assert changed > 0


# ----------------------------------------------------------------------------- mutations
def _plant(monkeypatch, name, fn):
    monkeypatch.setattr(oc, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def _fails(pin):
    with pytest.raises(AssertionError):
        pin()


def test_planted_sink_dropped_from_the_denominator(monkeypatch):
    orig = oc.attention_row

    def wrong(q_t, kv, ckv, sink, ids_row, win_rows, scale):
        return orig(q_t, kv, ckv, np.full_like(np.asarray(sink, float), -np.inf), ids_row, win_rows, scale)
    _plant(monkeypatch, "attention_row", wrong)
    _fails(A.test_sink_closed_form)
    _fails(A.test_worked_two_head_example)


def test_planted_compressed_only_teacher(monkeypatch):
    def wrong(attn, ids_row):
        c = attn.c
        p = np.exp(c - oc._logsumexp(c, axis=1)[:, None]).sum(axis=0)
        out = np.zeros(len(ids_row)); out[np.asarray(ids_row) >= 0] = p
        return oc.teacher_from_mass(out)
    _plant(monkeypatch, "teacher_sparse_row", wrong)
    _fails(A.test_worked_two_head_example)


def test_planted_wrong_weight_index(monkeypatch):
    orig = oc.indexer_scores_row

    def wrong(q_idx_t, w_t, k_idx_seg, idx_scale, n_valid):
        w = np.full_like(np.asarray(w_t), np.asarray(w_t)[0])
        return orig(q_idx_t, w, k_idx_seg, idx_scale, n_valid)
    _plant(monkeypatch, "indexer_scores_row", wrong)
    _fails(G.test_scores_are_symmetric_in_heads_and_feature_axes)
    _fails(G.test_exact_family_equals_rational_bruteforce)


def test_planted_transposed_feature_axis(monkeypatch):
    def wrong(q_idx_t, w_t, k_idx_seg, idx_scale, n_valid):
        q = np.asarray(q_idx_t, float)
        k = np.asarray(k_idx_seg, float)
        ws = oc.indexer_weight_scale(w_t, idx_scale).astype(float)
        out = np.full(k.shape[0], -np.inf)
        if n_valid:
            dots = k[:n_valid] @ q[:, ::-1].T     # feature axis reversed on one side
            out[:n_valid] = np.maximum(dots, 0) @ ws
        return out
    _plant(monkeypatch, "indexer_scores_row", wrong)
    _fails(G.test_exact_family_equals_rational_bruteforce)


def test_planted_tie_to_the_higher_index(monkeypatch):
    def wrong(scores_row, n_valid, k_eff, k_base):
        out = np.full(k_eff, -1, dtype=np.int64)
        kt = min(k_eff, n_valid)
        if kt <= 0:
            return out
        vals = np.asarray(scores_row[:n_valid], float)
        order = np.lexsort((-np.arange(n_valid), -vals))
        out[:kt] = np.sort(order[:kt]) + k_base
        return out
    _plant(monkeypatch, "topk_row", wrong)
    with pytest.raises(AssertionError):
        for seed in range(40):
            G.test_topk_matches_subset_bruteforce_with_ties(seed)


def test_planted_tiny_predictor_epsilon(monkeypatch):
    def wrong(teacher, pred):
        t = np.asarray(teacher, float); p = np.asarray(pred, float)
        return float(np.sum(t * (np.log(t + 1e-10) - np.log(np.maximum(p, np.finfo(np.float32).tiny)))))
    _plant(monkeypatch, "kl_row", wrong)
    _fails(A.test_kl_golden_values)


def test_planted_top_left_alignment(monkeypatch):
    def wrong(L, t):
        s = oc.segment_of_row(L.cu_q, t)
        r = t - int(L.cu_q[s])
        s_k = int(L.cu_k[s + 1] - L.cu_k[s])
        n = max(0, min((r + 1) // L.ratio, s_k))
        return oc.RowGeom(s, r, r + 1, n, int(L.cu_k[s]), int(L.cu_q[s]))
    _plant(monkeypatch, "row_geometry", wrong)
    _fails(G.test_chunk_offset_restores_absolute_positions_and_negative_control)


def test_planted_valid_row_divisor(monkeypatch):
    def wrong(kl_rows, total_q, per_token):
        k = np.asarray(kl_rows, float)
        return float(k.sum()) if per_token else float(k.sum() / max(1, np.count_nonzero(k)))
    _plant(monkeypatch, "reduce_loss", wrong)
    _fails(A.test_loss_reduction_counts_every_physical_row)


def test_planted_window_without_the_query_row(monkeypatch):
    def wrong(t, q_start, window):
        lo = max(q_start, t - window)
        return np.arange(lo, t, dtype=np.int64)
    _plant(monkeypatch, "window_rows", wrong)
    _fails(A.test_window_rows_reading)
