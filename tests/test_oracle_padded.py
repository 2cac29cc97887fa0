"""Pins of the oracle's padded-THD handling.

[I5776, fused-path excerpt, step 4b]: when CUDA-graph padding makes cu_seqlens_q cover
every physical row, the unpadded boundaries mark each segment's real length; rows past it
are padding, excluded from the loss and its gradients.  [I5776, review comment]: in the
padded-THD fixture with real lengths [9, 11] the real segment losses are weighted by
those lengths and the sum is divided by the physical total_q = 24.

The padded problem is assembled from two independent single-segment problems (plus
padding rows and the keys they compress to), so the pins compare the padded oracle run
with runs that never see a padding mask:
  loss(padded) = (9 loss(seg 0) + 11 loss(seg 1)) / 24          (mean mode)
  loss(padded) = loss(seg 0) + loss(seg 1)                       (per-token mode)
and the backward of the padded run is the single runs' backward scaled by len / 24, with
zero gradient on padding rows and on the keys only padding rows see.  Planted mistakes
(the real-row count as divisor; the mask dropped) must fail the pins.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from tests import tiny

RATIO = 2
REAL = (9, 11)
PHYS_TOTAL = 24


def _alone(seg, seed, sparse):
    L = tiny.layout((seg,), RATIO, off=[0])
    return tiny.problem(L=L, H=3, D=8, Hi=3, Di=6, topk=3, window=3, seed=seed, sparse=sparse)


def _padded(form, sparse, per_token=False):
    """(padded problem, [alone problems], key ranges of the real keys in the padded run)."""
    a = [_alone(REAL[0], 3, sparse), _alone(REAL[1], 4, sparse)]
    n_pad = PHYS_TOTAL - sum(REAL)
    if form == "absorbed":          # padding appended to the last segment
        phys = (REAL[0], REAL[1] + n_pad)
        real = (REAL[0], REAL[1])
    else:                           # a trailing dummy segment of real length 0
        phys = (REAL[0], REAL[1], n_pad)
        real = (REAL[0], REAL[1], 0)
    cu_q = np.concatenate([[0], np.cumsum(phys)]).astype(np.int64)
    cu_k = oracle.compressed_cu_seqlens(cu_q, RATIO)
    cu_real = np.concatenate([[0], np.cumsum(real)]).astype(np.int64)
    L = oracle.Layout(cu_q=cu_q, cu_k=cu_k, ratio=RATIO, off=np.zeros(len(phys), dtype=np.int64),
                      cu_q_real=cu_real)
    rng = np.random.default_rng(99)
    k_real = [REAL[0] // RATIO, REAL[1] // RATIO]
    n_extra_k = int(cu_k[-1]) - sum(k_real)

    def cat(name, extra_rows):
        parts = [getattr(a[0], name), getattr(a[1], name)]
        shape = (extra_rows,) + parts[0].shape[1:]
        extra = rng.standard_normal(shape).astype(parts[0].dtype)
        return np.concatenate(parts + [extra])

    w_pad = rng.random((n_pad, a[0].weights.shape[1])).astype(np.float32)
    P = oracle.Problem(layout=L, q=cat("q", n_pad), kv=cat("kv", n_pad), ckv=cat("ckv", n_extra_k),
                       q_idx=cat("q_idx", n_pad), k_idx=cat("k_idx", n_extra_k),
                       weights=np.concatenate([a[0].weights, a[1].weights, w_pad]),
                       sink=a[0].sink, topk=a[0].topk, window=a[0].window, scale=a[0].scale,
                       idx_scale=a[0].idx_scale, sparse_loss=sparse, per_token=per_token)
    for x in a:
        x.sink = a[0].sink
        x.per_token = per_token
    return P, a, [(0, k_real[0]), (k_real[0], k_real[0] + k_real[1])]


@pytest.mark.parametrize("form", ["absorbed", "dummy"])
@pytest.mark.parametrize("sparse", [True, False])
def test_loss_weights_real_lengths_over_physical_rows(form, sparse):
    P, a, _ = _padded(form, sparse)
    rows, loss = oracle.run_all(P)
    l0, l1 = oracle.run_all(a[0])[1], oracle.run_all(a[1])[1]
    assert loss == pytest.approx((REAL[0] * l0 + REAL[1] * l1) / PHYS_TOTAL, rel=1e-12)
    assert l0 > 0 and l1 > 0
    for r in rows:
        if r.geom.padding:
            assert r.kl == 0.0 and not np.any(r.teacher)
    assert sum(r.geom.padding for r in rows) == PHYS_TOTAL - sum(REAL)


@pytest.mark.parametrize("form", ["absorbed", "dummy"])
def test_per_token_loss_is_the_sum_of_the_real_segments(form):
    P, a, _ = _padded(form, True, per_token=True)
    loss = oracle.run_all(P)[1]
    assert loss == pytest.approx(oracle.run_all(a[0])[1] + oracle.run_all(a[1])[1], rel=1e-12)


def test_real_rows_forward_equals_the_unpadded_runs():
    P, a, kr = _padded("absorbed", True)
    off = 0
    for s in range(2):
        for t in range(REAL[s]):
            rp = oracle.run_row(P, off + t)
            ra = oracle.run_row(a[s], t)
            np.testing.assert_array_equal(rp.ids[rp.ids >= 0] - kr[s][0], ra.ids[ra.ids >= 0])
            np.testing.assert_allclose(rp.attn.out, ra.attn.out, rtol=1e-14, atol=1e-15)
            assert rp.kl == pytest.approx(ra.kl, rel=1e-13, abs=1e-300)
        off += REAL[s]


@pytest.mark.parametrize("sparse", [True, False])
def test_backward_is_the_unpadded_backward_scaled(sparse):
    P, a, kr = _padded("absorbed", sparse)
    dq, dw, dk = oracle.indexer_loss_backward(P)
    off = 0
    for s in range(2):
        f = REAL[s] / PHYS_TOTAL
        dqa, dwa, dka = oracle.indexer_loss_backward(a[s])
        np.testing.assert_allclose(dq[off:off + REAL[s]], f * dqa, rtol=1e-12, atol=1e-16)
        np.testing.assert_allclose(dw[off:off + REAL[s]], f * dwa, rtol=1e-12, atol=1e-16)
        np.testing.assert_allclose(dk[kr[s][0]:kr[s][1]], f * dka, rtol=1e-12, atol=1e-16)
        off += REAL[s]
    assert not dq[sum(REAL):].any() and not dw[sum(REAL):].any()
    assert not dk[kr[1][1]:].any()      # keys compressed from padding rows only
    assert np.abs(dq).max() > 0 and np.abs(dk).max() > 0


def test_planted_real_row_divisor_fails_the_pin(monkeypatch):
    def wrong(kl_rows, total_q, per_token):
        s = float(np.sum(kl_rows))
        return s if per_token else s / float(sum(REAL))
    monkeypatch.setattr(oracle.csa_oracle, "reduce_loss", wrong)
    with pytest.raises(AssertionError):
        test_loss_weights_real_lengths_over_physical_rows("absorbed", True)


def test_planted_mask_dropped_fails_the_pin(monkeypatch):
    real = oracle.csa_oracle.row_geometry

    def no_mask(L, t):
        g = real(L, t)
        g.padding = False
        return g
    monkeypatch.setattr(oracle.csa_oracle, "row_geometry", no_mask)
    with pytest.raises(AssertionError):
        test_loss_weights_real_lengths_over_physical_rows("absorbed", True)
