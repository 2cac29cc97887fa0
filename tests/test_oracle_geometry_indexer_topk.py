"""CPU pins of the oracle's row geometry, indexer scores and top-k.

Each test checks the oracle against something fixed outside it: the causal mask as the
page writes it (a matrix), exact rational arithmetic, a library matmul, symmetry of the
definition, brute force over subsets, or torch.topk.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import tiny


# ----------------------------------------------------------------------------- geometry
def test_n_valid_matches_the_page_mask_matrix():
    """[I5776, csa.py SBHD excerpt]: mask[b, s, j] = -inf where j >= positions // ratio,
    positions = 1..sq; n_valid(t) must equal the count of unmasked columns."""
    sq, ratio, b = 37, 4, 2
    n_cmp = sq // ratio
    L = tiny.layout([sq] * b, ratio, off=[n_cmp * ratio - sq] * b)
    cols = np.arange(n_cmp)[None, :]
    positions = np.arange(1, sq + 1)[:, None]
    mask = np.where(cols >= positions // ratio, -np.inf, 0.0)
    # with sq not divisible by ratio the default offset (seqlen_k*ratio - seqlen_q) is
    # negative; the page's SBHD mask uses absolute positions, so pass offset 0 for it
    L0 = tiny.layout([sq] * b, ratio, off=[0] * b)
    for t in range(L0.total_q):
        g = oracle.row_geometry(L0, t)
        assert g.n_valid == int(np.sum(mask[g.local] == 0.0))
    # the default offset shifts the alignment by -(sq mod ratio) (bottom-right)
    assert list(oracle.default_offsets(L.cu_q, L.cu_k, ratio)) == [n_cmp * ratio - sq] * b


def test_thd_rows_see_only_their_segment():
    seg = [12, 20, 9]
    L = tiny.layout(seg, 4, off=[0, 0, 0])
    for s, n in enumerate(seg):
        Ls = tiny.layout([n], 4, off=[0])
        for r in range(n):
            g = oracle.row_geometry(L, int(L.cu_q[s]) + r)
            gs = oracle.row_geometry(Ls, r)
            assert (g.seg, g.local, g.n_valid) == (s, r, gs.n_valid)
            assert g.k_base == int(L.cu_k[s])


def test_chunk_offset_restores_absolute_positions_and_negative_control():
    """[PR8539, item 2]: a query chunk scored against its key prefix needs the offset;
    with offset = chunk start each row sees its absolute causal keys; with offset 0
    (top-left) the visible set shrinks (the page's negative control)."""
    S, ratio, c0 = 64, 4, 40
    full = tiny.layout([S], ratio, off=[0])
    chunk_right = tiny.layout([S - c0], ratio, off=[c0], cu_k=[0, S // ratio])
    chunk_left = tiny.layout([S - c0], ratio, off=[0], cu_k=[0, S // ratio])
    changed = 0
    for r in range(S - c0):
        a = oracle.row_geometry(full, c0 + r).n_valid
        assert oracle.row_geometry(chunk_right, r).n_valid == a
        changed += oracle.row_geometry(chunk_left, r).n_valid != a
    assert changed == S - c0


def test_workload_offsets_equal_the_bottom_right_default():
    from deepseek_v4_csa_amd.inputs import WORKLOADS, layout_tensors
    for wl in WORKLOADS:
        cu_q, cu_k, off = layout_tensors(wl, "cpu")
        d = oracle.default_offsets(cu_q.numpy(), cu_k.numpy(), wl.ratio)
        assert d.tolist() == off.tolist()
        assert (oracle.compressed_cu_seqlens(cu_q.numpy(), wl.ratio) == cu_k.numpy()).all()


def test_k_eff():
    L = tiny.layout([1024, 2048, 6144], 4)
    assert oracle.k_eff_of(L, 512) == 512
    assert oracle.k_eff_of(L, 4096) == 1536


# ----------------------------------------------------------------------------- indexer
def test_exact_family_equals_rational_bruteforce():
    """Integer q_idx/k_idx, weights m/16, scale 1/8: the scores are exact rationals; the
    oracle must reproduce an exact Fraction evaluation done with explicit loops."""
    P = tiny.problem(seg_lens=(24, 16), Hi=3, Di=5, integer_idx=True, seed=3)
    L = P.layout
    for t in range(L.total_q):
        g = oracle.row_geometry(L, t)
        k_seg = P.k_idx[g.k_base:int(L.cu_k[g.seg + 1])]
        got = oracle.indexer_scores_row(P.q_idx[t], P.weights[t], k_seg, P.idx_scale, g.n_valid)
        for j in range(len(k_seg)):
            if j >= g.n_valid:
                assert got[j] == -np.inf
                continue
            acc = Fraction(0)
            for h in range(P.q_idx.shape[1]):
                dot = sum(Fraction(int(P.q_idx[t, h, d])) * Fraction(int(k_seg[j, d]))
                          for d in range(P.q_idx.shape[2]))
                ws = Fraction(float(P.weights[t, h])) * Fraction(1, 8)
                acc += ws * max(dot, Fraction(0))
            assert Fraction(got[j]) == acc


def test_single_head_unit_weight_is_relu_of_a_matmul():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 7))
    k = rng.standard_normal((11, 7))
    got = oracle.indexer_scores_row(q, np.ones(1, np.float32), k, 1.0, 9)
    ref = torch.relu(torch.from_numpy(k) @ torch.from_numpy(q[0])).numpy()
    np.testing.assert_allclose(got[:9], ref[:9], rtol=0, atol=1e-15)
    assert np.all(got[9:] == -np.inf)


def test_scores_are_symmetric_in_heads_and_feature_axes():
    """Permuting the indexer heads (q rows together with their weights) or the feature
    axis (q and k together) must not change any score."""
    rng = np.random.default_rng(2)
    q = rng.standard_normal((5, 6))
    w = rng.random(5).astype(np.float32)
    k = rng.standard_normal((10, 6))
    base = oracle.indexer_scores_row(q, w, k, 0.3, 10)
    ph, pd = rng.permutation(5), rng.permutation(6)
    np.testing.assert_allclose(oracle.indexer_scores_row(q[ph], w[ph], k, 0.3, 10), base, rtol=1e-14)
    np.testing.assert_allclose(oracle.indexer_scores_row(q[:, pd], w, k[:, pd], 0.3, 10), base, rtol=1e-14)
    # a head whose weight is 0 contributes nothing; a key whose every head dot is
    # negative scores exactly 0
    w0 = w.copy(); w0[2] = 0
    q2 = q.copy(); q2[2] = 100.0
    np.testing.assert_allclose(oracle.indexer_scores_row(q2, w0, k, 0.3, 10),
                               oracle.indexer_scores_row(q, w0, k, 0.3, 10), rtol=1e-14)
    kneg = -np.abs(k); qpos = np.abs(q)
    assert np.all(oracle.indexer_scores_row(qpos, w, kneg, 0.3, 10) == 0.0)


def test_weight_scale_is_rounded_in_fp32():
    w = np.array([1.0 / 3.0], dtype=np.float32)
    s = 1.0 / np.sqrt(64.0)
    ws = oracle.indexer_weight_scale(w, s)
    assert ws.dtype == np.float32
    assert float(ws[0]) == float(torch.tensor([1.0 / 3.0]).float().mul(torch.tensor(s, dtype=torch.float32))[0])


# ----------------------------------------------------------------------------- top-k
def _bruteforce_topk(vals, k):
    """The unique k-subset S whose members all precede every non-member in the order
    (higher value first, then lower index) -- found by enumerating all subsets."""
    n = len(vals)
    found = []
    for S in itertools.combinations(range(n), k):
        Sset = set(S)
        ok = all((vals[a] > vals[b]) or (vals[a] == vals[b] and a < b)
                 for a in S for b in range(n) if b not in Sset)
        if ok:
            found.append(S)
    assert len(found) == 1
    return list(found[0])


@pytest.mark.parametrize("seed", range(40))
def test_topk_matches_subset_bruteforce_with_ties(seed):
    rng = np.random.default_rng(seed)
    n_total = int(rng.integers(1, 10))
    n_valid = int(rng.integers(0, n_total + 1))
    k_eff = int(rng.integers(1, 6))
    row = rng.integers(0, 4, size=n_total).astype(np.float64)   # many exact ties
    row[n_valid:] = -np.inf
    ids = oracle.topk_row(row, n_valid, k_eff, k_base=100)
    kt = min(k_eff, n_valid)
    assert list(ids[kt:]) == [-1] * (k_eff - kt)
    if kt:
        want = _bruteforce_topk(list(row[:n_valid]), kt)
        assert list(ids[:kt]) == [100 + j for j in sorted(want)]


def test_topk_values_match_torch_topk():
    rng = np.random.default_rng(5)
    for _ in range(50):
        n = int(rng.integers(1, 200))
        k = int(rng.integers(1, 64))
        row = rng.standard_normal(n)
        ids = oracle.topk_row(row, n, k, 0)
        kt = min(n, k)
        ref = torch.topk(torch.from_numpy(row), kt).values.numpy()
        np.testing.assert_array_equal(np.sort(row[ids[:kt]]), np.sort(ref))
        assert np.all(np.diff(ids[:kt]) > 0)


def test_topk_short_and_empty_rows():
    assert list(oracle.topk_row(np.full(4, -np.inf), 0, 3, 7)) == [-1, -1, -1]
    assert list(oracle.topk_row(np.array([0.5, 0.1, -np.inf]), 2, 4, 10)) == [10, 11, -1, -1]
