"""Pins of the oracle's indexer-loss backward (the step after the forward path).

The analytic gradients of ``oracle.indexer_loss_backward`` are checked against
  * central finite differences of the oracle's own forward loss with the teacher and
    the selection held fixed (``indexer_loss_fixed``), a computation that shares none of
    the gradient algebra;
  * float64 autograd of that forward in plain PyTorch CPU ops;
  * the batch-split property of [PR8539]'s test plan: a two-sequence batch gives the
    gradients of two single-sequence runs, scaled for the row-mean loss;
and a planted mistake (the ReLU mask dropped) must fail the finite-difference pin.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from tests import tiny


def _fd(P, rows, which, idx, h):
    arrs = {"q": P.q_idx.copy(), "w": P.weights.astype(np.float64).copy(), "k": P.k_idx.copy()}
    plus = {k: v.copy() for k, v in arrs.items()}
    minus = {k: v.copy() for k, v in arrs.items()}
    plus[which][idx] += h
    minus[which][idx] -= h
    lp = oracle.indexer_loss_fixed(P, rows, plus["q"], plus["w"], plus["k"], exact_ws=True)
    lm = oracle.indexer_loss_fixed(P, rows, minus["q"], minus["w"], minus["k"], exact_ws=True)
    return (lp - lm) / (2 * h)


def _check_fd(P, seed=0, n=10, rel=2e-6):
    rows, _ = oracle.run_all(P)
    dq, dw, dk = oracle.indexer_loss_backward(P, rows)
    rng = np.random.default_rng(seed)
    scale = max(np.abs(dq).max(), np.abs(dw).max(), np.abs(dk).max())
    assert scale > 0
    for which, grad in (("q", dq), ("w", dw), ("k", dk)):
        for _ in range(n):
            idx = tuple(int(rng.integers(0, s)) for s in grad.shape)
            fd = _fd(P, rows, which, idx, 1e-6)
            assert abs(fd - grad[idx]) <= rel * scale + 1e-9 * abs(grad[idx]), (which, idx, fd, grad[idx])


@pytest.mark.parametrize("sparse", [True, False])
def test_backward_matches_finite_differences(sparse):
    P = tiny.problem(seg_lens=(20, 13), ratio=2, Hi=3, Di=5, topk=4, window=3, seed=7, sparse=sparse)
    _check_fd(P, seed=1)


def test_backward_matches_finite_differences_per_token_and_offsets():
    L = tiny.layout((9, 14), ratio=3, off=[2, -1])
    P = tiny.problem(L=L, Hi=2, Di=4, topk=3, window=2, seed=3)
    P.per_token = True
    _check_fd(P, seed=2)


def test_backward_matches_float64_autograd():
    torch = pytest.importorskip("torch")
    P = tiny.problem(seg_lens=(17, 11), ratio=2, Hi=3, Di=6, topk=5, window=4, seed=11)
    rows, _ = oracle.run_all(P)
    dq, dw, dk = oracle.indexer_loss_backward(P, rows)
    L = P.layout
    q = torch.tensor(P.q_idx, dtype=torch.float64, requires_grad=True)
    w = torch.tensor(P.weights.astype(np.float64), requires_grad=True)
    k = torch.tensor(P.k_idx, dtype=torch.float64, requires_grad=True)
    s_idx = float(np.float32(P.idx_scale))
    total = torch.zeros((), dtype=torch.float64)
    for r in rows:
        cols, tch, _ = oracle.loss_support(P, r)
        if cols.size == 0:
            continue
        ks = k[r.geom.k_base + torch.as_tensor(cols)]                   # [n, Di]
        sc = torch.relu(ks @ q[r.t].T) @ (w[r.t] * s_idx)               # [n]
        p = torch.softmax(sc, dim=0)
        t = torch.as_tensor(tch, dtype=torch.float64)
        total = total + (t * (torch.log(t + 1e-10) - torch.log(p + 1e-10))).sum()
    (total / L.total_q).backward()
    # ws rounding: the oracle's dq/dk use fp32(w * s_idx), autograd the exact product
    # (relative 2^-24 per weight, so near-zero sums are compared against the tensor's scale)
    for mine, ref in ((dq, q.grad.numpy()), (dk, k.grad.numpy())):
        np.testing.assert_allclose(mine, ref, rtol=1e-6, atol=1e-6 * np.abs(ref).max())
    np.testing.assert_allclose(dw, w.grad.numpy(), rtol=1e-6, atol=1e-6 * np.abs(dw).max())


def test_batch_of_two_equals_two_single_runs_scaled():
    """[PR8539] test plan: the reference for a two-sequence batch is the same rows run as
    two single-sequence calls, scaled for the row-mean loss."""
    P = tiny.problem(seg_lens=(24, 24), ratio=4, Hi=2, Di=6, topk=3, window=4, seed=5)
    dq, dw, dk = oracle.indexer_loss_backward(P)
    T = P.layout.total_q
    for s in range(2):
        a, b = int(P.layout.cu_q[s]), int(P.layout.cu_q[s + 1])
        ka, kb = int(P.layout.cu_k[s]), int(P.layout.cu_k[s + 1])
        Ls = tiny.layout((b - a,), P.layout.ratio)
        Ps = oracle.Problem(layout=Ls, q=P.q[a:b], kv=P.kv[a:b], ckv=P.ckv[ka:kb], q_idx=P.q_idx[a:b],
                            k_idx=P.k_idx[ka:kb], weights=P.weights[a:b], sink=P.sink, topk=P.topk,
                            window=P.window, scale=P.scale, idx_scale=P.idx_scale, sparse_loss=P.sparse_loss)
        dqs, dws, dks = oracle.indexer_loss_backward(Ps)
        f = (b - a) / T
        np.testing.assert_allclose(dq[a:b], f * dqs, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(dw[a:b], f * dws, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(dk[ka:kb], f * dks, rtol=1e-12, atol=1e-15)


def test_rows_without_visible_keys_have_zero_gradient():
    P = tiny.problem(seg_lens=(16,), ratio=4, Hi=2, Di=4, topk=3, window=2, seed=9)
    dq, dw, _ = oracle.indexer_loss_backward(P)
    for t in range(P.layout.total_q):
        if oracle.row_geometry(P.layout, t).n_valid == 0:
            assert not dq[t].any() and not dw[t].any()


def test_planted_relu_mask_dropped_fails_the_fd_pin(monkeypatch):
    real = oracle.csa_oracle.indexer_grads_row

    def wrong(q_idx_t, w_t, k_idx_seg, idx_scale, cols, g_cols, exact_ws=False):
        q = np.asarray(q_idx_t, dtype=np.float64)
        k = np.asarray(k_idx_seg, dtype=np.float64)[np.asarray(cols)]
        g = np.asarray(g_cols, dtype=np.float64)
        ws = oracle.indexer_weight_scale(w_t, idx_scale).astype(np.float64)
        d = k @ q.T
        dq = ws[:, None] * ((g[:, None] * np.ones_like(d)).T @ k)   # mask dropped
        _, dw, dk = real(q_idx_t, w_t, k_idx_seg, idx_scale, cols, g_cols, exact_ws)
        return dq, dw, dk

    monkeypatch.setattr(oracle.csa_oracle, "indexer_grads_row", wrong)
    P = tiny.problem(seg_lens=(20,), ratio=2, Hi=3, Di=5, topk=4, window=3, seed=4)
    with pytest.raises(AssertionError):
        _check_fd(P, seed=3)
