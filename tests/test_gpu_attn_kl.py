"""GPU parity of csa_sparse_attn_kl_fwd (attention + sparse teacher + KL in one call) and
csa_loss_reduce, through the C ABI.

With selected scores and a shape of the one-wave-per-query attention kernel, the teacher
and the KL are finished in that kernel's epilogue.  Its attention arithmetic is the
stand-alone kernel's, so out, lse, lse_nc and cmass must equal the two-call path bit for
bit; the teacher and KL are the same formulas with another fp64 summation order, so they
are held to the oracle on identical ids (tests/gpu_check.py tolerances: 1e-5 relative) and
to the two-call path within the same bound.  Every other route (full score rows, shapes
without the epilogue) runs the attention and teacher kernels in turn and must equal the two
calls bit for bit.  Layouts: ragged packed documents with rows that see no key, k_eff not a
multiple of 32, fewer than 16 heads, D = 64 and 128, padded THD rows, the full batch-2 x
4096 workload (sampled rows against the oracle, every row against the two calls).
"""
import numpy as np
import pytest
import torch

from deepseek_v4_csa_amd import inputs as I
from tests import gpu_check as C

pytestmark = pytest.mark.gpu


def _ops():
    from deepseek_v4_csa_amd import ops
    ops.load()
    return ops


def _close(a, b, rel=1e-5, abs_=1e-12):
    a = a.double()
    b = b.double()
    return bool(((a - b).abs() <= rel * b.abs() + abs_).all())


def _run_both(inp, fused_scores=True):
    ops = _ops()
    r2 = ops.forward(inp, want_teacher=True, poison=True, fused=fused_scores)
    rk = ops.forward(inp, want_teacher=True, poison=True, fused=fused_scores, attn_kl=True)
    torch.cuda.synchronize()
    return r2, rk


def _scores_for_oracle(inp):
    ops = _ops()
    L = ops.layout_of_inputs(inp)
    s = ops.csa_indexer_score(L, inp.q_idx, inp.k_idx, inp.weights, inp.idx_scale)
    torch.cuda.synchronize()
    return s


def _check(inp, r2, rk, rows, epilogue=True):
    # the attention outputs are the stand-alone kernel's arithmetic
    for k in ("ids", "out", "lse", "lse_nc", "cmass"):
        assert torch.equal(rk[k], r2[k]), k
    if epilogue:
        assert _close(rk["teacher"], r2["teacher"], abs_=1e-9)
        assert _close(rk["kl_row"], r2["kl_row"])
        assert _close(rk["loss"], r2["loss"])
    else:
        for k in ("teacher", "kl_row", "loss"):
            assert torch.equal(rk[k], r2[k]), k
    # the oracle on identical ids (the full score rows give the oracle's score check)
    res = dict(rk)
    res["scores"] = _scores_for_oracle(inp)
    C.check_rows(inp, res, rows, tag=f"attn-kl-{inp.wl.name}", loss_rows=(len(rows) == inp.wl.total_q))


SMALL = {
    # (workload, seed): H <= 16 with a window -> the epilogue route
    "bshd-ragged-h16-d128": (I.scaled_down(I.WORKLOADS[1], (100, 37, 300, 16, 520), topk=40), 11),
    "bshd-h12-d64": (I.scaled_down(I.WORKLOADS[1], (260, 517), topk=72, H=12, D=64, name="attnkl-h12"), 12),
    "bshd-k-small": (I.scaled_down(I.WORKLOADS[1], (384, 129), topk=7, name="attnkl-k7"), 13),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_attn_kl_every_row(gpu_ok, name):
    wl, seed = SMALL[name]
    inp = I.make_inputs(wl, device="cuda", seed=seed)
    r2, rk = _run_both(inp)
    _check(inp, r2, rk, list(range(wl.total_q)))


def test_attn_kl_full_rows_route(gpu_ok):
    """Full score rows (scores_selected = 0): the two kernels in turn, bit-identical."""
    wl = I.scaled_down(I.WORKLOADS[1], (300, 200), topk=40, name="attnkl-full")
    inp = I.make_inputs(wl, device="cuda", seed=5)
    r2, rk = _run_both(inp, fused_scores=False)
    _check(inp, r2, rk, list(range(wl.total_q)), epilogue=False)


def test_attn_kl_other_kernel_route(gpu_ok):
    """More than 16 heads (the workgroup attention kernel): the two kernels in turn."""
    wl = I.scaled_down(I.WORKLOADS[2], (128, 256, 200), topk=24, Hi=16, name="attnkl-h64")
    inp = I.make_inputs(wl, device="cuda", seed=6)
    r2, rk = _run_both(inp)
    _check(inp, r2, rk, list(range(wl.total_q)), epilogue=False)


def test_attn_kl_padded_rows(gpu_ok):
    """Padding rows are attended but left out of the loss: teacher and kl_row 0 there,
    the divisor is the physical row count."""
    wl = I.scaled_down(I.WORKLOADS[1], (512, 300), topk=40)
    inp = I.pad_inputs(I.make_inputs(wl, device="cuda", seed=8), 92)
    r2, rk = _run_both(inp)
    _check(inp, r2, rk, list(range(inp.wl.total_q)))
    real = int(inp.cu_q_real[-1])
    assert bool((rk["kl_row"][real:] == 0).all())
    assert bool((rk["teacher"][real:] == 0).all())
    ops = _ops()
    want = ops.csa_loss_reduce(rk["kl_row"])
    torch.cuda.synchronize()
    assert float(rk["loss"][0]) == float(want[0])
    ref = rk["kl_row"].double().sum().item() / inp.wl.total_q
    assert abs(float(rk["loss"][0]) - ref) <= 1e-6 * abs(ref) + 1e-12


def test_loss_reduce_modes_and_determinism(gpu_ok):
    ops = _ops()
    g = torch.Generator(device="cuda").manual_seed(3)
    for n in (0, 1, 1000, 8192, 70001):
        kl = torch.rand((n,), generator=g, device="cuda", dtype=torch.float32)
        a = ops.csa_loss_reduce(kl)
        b = ops.csa_loss_reduce(kl)
        s = ops.csa_loss_reduce(kl, per_token=True)
        torch.cuda.synchronize()
        ref = kl.double().sum().item()
        assert torch.equal(a, b)
        assert abs(float(s[0]) - ref) <= 1e-6 * abs(ref) + 1e-12, n
        assert abs(float(a[0]) - (ref / n if n else 0.0)) <= 1e-6 * abs(ref / max(n, 1)) + 1e-12, n


def test_attn_kl_full_workload(gpu_ok):
    """bshd-b2-s4096 (the benchmarked call chain): every row against the two calls, sampled
    rows against the oracle, and two runs bitwise equal."""
    wl = I.WORKLOADS[1]
    inp = I.make_inputs(wl, device="cuda")
    r2, rk = _run_both(inp)
    rows = I.sample_rows(wl, 24)
    _check(inp, r2, rk, rows)
    again = _ops().forward(inp, want_teacher=True, poison=True, fused=True, attn_kl=True)
    torch.cuda.synchronize()
    for k in ("teacher", "kl_row", "loss"):
        assert torch.equal(again[k], rk[k]), k
    assert np.isfinite(float(rk["loss"][0]))
