"""GPU parity of csa_topk's selected-scores output (sel_scores), through the C ABI.

Slot j of sel_scores must be bit-identical to the score of ids[t, j] gathered from the row
(-inf at -1 slots), for both top-k kernels (one wave per row up to 4096 keys, one
workgroup per row beyond), and the ids must not change when it is requested.  The
teacher/KL reading the selected scores in place (scores_selected = 1) must then equal the
teacher/KL that gathers them from the rows, bit for bit (same values, same arithmetic).
The oracle's own checks of ids, teacher and KL on these layouts are in test_gpu_parity.py.
"""
import pytest
import torch

from deepseek_v4_csa_amd import inputs as I

pytestmark = pytest.mark.gpu


def _ops():
    from deepseek_v4_csa_amd import ops
    ops.load()
    return ops


def _gathered(inp, scores, ids):
    cu_k = inp.cu_k.long()
    T = ids.shape[0]
    seg = torch.searchsorted(inp.cu_q.long(), torch.arange(T, device=ids.device), right=True) - 1
    loc = torch.where(ids >= 0, ids.long() - cu_k[seg][:, None], torch.zeros_like(ids, dtype=torch.long))
    return torch.where(ids >= 0, scores.gather(1, loc), torch.full(ids.shape, -float("inf"), device=ids.device))


CASES = {
    # (workload, seed): rows up to 4096 keys (wave kernel) and beyond (workgroup kernel)
    "thd-short-rows": (I.scaled_down(I.WORKLOADS[2], (128, 256, 200, 68), topk=24), 21),
    "bshd-k-not-multiple-of-32": (I.scaled_down(I.WORKLOADS[1], (700, 333), topk=50), 22),
    "long-rows": (I.scaled_down(I.WORKLOADS[3], (20000, 1200), topk=600, name="topk-sel-long"), 23),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_topk_selected_scores(gpu_ok, name):
    ops = _ops()
    wl, seed = CASES[name]
    inp = I.make_inputs(wl, device="cuda", seed=seed)
    L = ops.layout_of_inputs(inp)
    scores = ops.csa_indexer_score(L, inp.q_idx, inp.k_idx, inp.weights, inp.idx_scale)
    ids0 = ops.csa_topk(L, scores, wl.topk)
    k = ids0.shape[1]
    sel = torch.full((wl.total_q, k), float("nan"), dtype=torch.float32, device="cuda")
    ids1 = ops.csa_topk(L, scores, wl.topk, sel_scores=sel)
    torch.cuda.synchronize()
    assert torch.equal(ids0, ids1)
    assert torch.equal(sel, _gathered(inp, scores, ids1))


@pytest.mark.parametrize("name", ["thd-short-rows", "long-rows"])
def test_teacher_kl_from_topk_selected_scores(gpu_ok, name):
    ops = _ops()
    wl, seed = CASES[name]
    inp = I.make_inputs(wl, device="cuda", seed=seed)
    a = ops.forward(inp, want_teacher=True, poison=True)
    a = {k: (v.clone() if v is not None else None) for k, v in a.items()}
    b = ops.forward(inp, want_teacher=True, poison=True, topk_sel=True)
    torch.cuda.synchronize()
    for key in ("ids", "out", "lse", "lse_nc", "cmass", "teacher", "kl_row", "loss"):
        assert torch.equal(a[key], b[key]), key
