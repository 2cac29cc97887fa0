"""GPU parity of padded THD batches ([I5776] fused-path excerpt, step 4b; review comment on
the padded-THD divisor): padding rows are scored, selected and attended like any row but
left out of the loss (teacher 0, kl_row 0, no gradient), and the mean-mode divisor stays
the physical row count.

Each padded batch is the unpadded one plus padding rows (appended to the last segment,
or a trailing dummy segment of real length 0), so besides the oracle on every row the
real rows must reproduce the unpadded run bit for bit.  Tolerances: tests/gpu_check.py
(forward) and tests/test_gpu_backward.py (backward).
"""
import numpy as np
import pytest
import torch

import oracle
from deepseek_v4_csa_amd import inputs as I
from tests import gpu_check as C
from tests import oracle_bridge as B
from tests.test_gpu_backward import _close, _oracle_rows, nan_workspaces

pytestmark = pytest.mark.gpu

CASES = {
    "thd-small-absorbed": (I.scaled_down(I.WORKLOADS[2], (128, 256, 200, 68), topk=24), 60, False),
    "thd-small-dummy": (I.scaled_down(I.WORKLOADS[2], (128, 256, 200, 68), topk=24), 36, True),
    "bshd-small-absorbed": (I.scaled_down(I.WORKLOADS[1], (512, 300), topk=40), 92, False),
    "dense-small-absorbed": (I.scaled_down(I.WORKLOADS[4], (640,), topk=16), 96, False),
}


def _ops():
    from deepseek_v4_csa_amd import ops
    ops.load()
    return ops


def _fwd(inp):
    res = _ops().forward(inp, want_teacher=True, poison=True)
    torch.cuda.synchronize()
    return res


def _real_rows(inp_pad):
    cu = inp_pad.cu_q.tolist()
    cr = inp_pad.cu_q_real.tolist()
    rows = []
    for s in range(len(cu) - 1):
        rows += range(cu[s], cu[s] + (cr[s + 1] - cr[s]))
    return rows


def _check_against_unpadded(inp, pad, res, resp):
    T_phys = pad.wl.total_q
    real = _real_rows(pad)
    assert real == list(range(inp.wl.total_q))     # padding only at the tail here
    n = inp.wl.total_q
    k_eff = res["ids"].shape[1]
    # forward of real rows: bit-identical (same keys, same arithmetic per row)
    assert torch.equal(resp["ids"][:n, :k_eff], res["ids"])
    assert bool((resp["ids"][:n, k_eff:] == -1).all())
    assert torch.equal(resp["out"][:n], res["out"])
    assert torch.equal(resp["lse"][:n], res["lse"])
    assert torch.equal(resp["kl_row"][:n], res["kl_row"])
    # padding rows: attended like any row, out of the loss
    assert bool((resp["kl_row"][n:] == 0).all())
    assert bool((resp["teacher"][n:] == 0).all())
    assert bool(torch.isfinite(resp["out"][n:].float()).all())
    # loss: the real rows' KL over the physical row count
    want = float(res["kl_row"].double().sum()) / T_phys
    got = float(resp["loss"][0])
    assert abs(got - want) <= 1e-6 * abs(want) + 1e-9, (got, want)


@pytest.mark.parametrize("name", list(CASES))
def test_padded_small_every_row(gpu_ok, name):
    wl, n_pad, dummy = CASES[name]
    inp = I.make_inputs(wl, device="cuda")
    pad = I.pad_inputs(inp, n_pad, dummy=dummy)
    res, resp = _fwd(inp), _fwd(pad)
    rep = C.check_rows(pad, resp, list(range(pad.wl.total_q)), tag=f"padded-{name}", loss_rows=True)
    print(name, dict(rep), flush=True)
    _check_against_unpadded(inp, pad, res, resp)


@pytest.mark.parametrize("name", ["thd-small-absorbed", "thd-small-dummy", "dense-small-absorbed"])
def test_padded_small_backward_every_element(gpu_ok, name):
    ops = _ops()
    wl, n_pad, dummy = CASES[name]
    pad = I.pad_inputs(I.make_inputs(wl, device="cuda"), n_pad, dummy=dummy)
    res = _fwd(pad)
    L = ops.layout_of_inputs(pad)
    g, ws = nan_workspaces(ops, L, pad)
    dq, dw, dk = ops.csa_indexer_loss_bwd(L, pad.wl.sparse_loss, pad.q_idx, pad.k_idx, pad.weights,
                                          pad.idx_scale, res["scores"], res["ids"], res["teacher"],
                                          grad_scores=g, workspace=ws)
    torch.cuda.synchronize()
    P = B.problem_of(pad)
    rows = _oracle_rows(P, res, range(pad.wl.total_q))
    rdq, rdw, rdk = oracle.indexer_loss_backward(P, rows)
    _close(f"{name} dq", B.host(dq), rdq)
    _close(f"{name} dw", B.host(dw), rdw)
    _close(f"{name} dk", B.host(dk), rdk)
    n = wl.total_q
    assert not dq[n:].any() and not dw[n:].any()
    assert not dk[wl.total_k:].any()           # keys compressed from padding rows only


def test_padded_full_thd_workload(gpu_ok):
    """thd-varlen-16k padded by a 1024-row dummy segment: sampled rows against the oracle,
    every real row against the unpadded run."""
    wl = I.WORKLOADS[2]
    inp = I.make_inputs(wl, device="cuda")
    pad = I.pad_inputs(inp, 1024, dummy=True)
    res, resp = _fwd(inp), _fwd(pad)
    rows = sorted(set(I.sample_rows(wl, 24)) | set(range(wl.total_q, wl.total_q + 1024, 97)))
    rep = C.check_rows(pad, resp, rows, tag="thd-varlen-16k-padded")
    print("thd-varlen-16k padded", dict(rep), flush=True)
    _check_against_unpadded(inp, pad, res, resp)
    del res, resp
    torch.cuda.empty_cache()
