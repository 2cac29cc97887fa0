"""GPU: csa_indexer_loss_bwd_noalloc (the backward for callers that cannot allocate) against
csa_indexer_loss_bwd with caller workspaces, through the C ABI.

Both routes run the same kernels; only where the score gradients and the dk partials live
differs (the library's static device scratch against caller buffers filled with NaN), so
dq_idx, dweights and dk_idx must be equal bit for bit.  The calls run back to back on one
GPU with shrinking inputs (the largest layout the scratch takes, the batch-2 x 4096
workload, then smaller ones), so a stale scratch element read by a later call would show.
A layout needing more scratch than the array holds is rejected before any launch.
"""
import pytest
import torch

from deepseek_v4_csa_amd import inputs as I

pytestmark = pytest.mark.gpu


def _ops():
    from deepseek_v4_csa_amd import ops
    ops.load()
    return ops


def _nan(shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


def _both(inp, fused):
    ops = _ops()
    wl = inp.wl
    res = ops.forward(inp, want_teacher=True, poison=True, fused=fused)
    scores = res["sel"] if fused else res["scores"]
    L = ops.layout_of_inputs(inp)
    g = _nan((wl.total_q, L.max_seqlen_k))
    n = max(ops.csa_indexer_loss_bwd_workspace(L, wl.Hi, wl.Di), 4)
    ws = _nan((n // 4,)).view(torch.uint8)
    a = ops.csa_indexer_loss_bwd(L, wl.sparse_loss, inp.q_idx, inp.k_idx, inp.weights, inp.idx_scale, scores,
                                 res["ids"], res["teacher"], grad_scores=g, workspace=ws, scores_selected=fused)
    out = (_nan(tuple(inp.q_idx.shape)), _nan(tuple(inp.weights.shape)), _nan(tuple(inp.k_idx.shape)))
    b = ops.csa_indexer_loss_bwd_noalloc(L, wl.sparse_loss, inp.q_idx, inp.k_idx, inp.weights, inp.idx_scale,
                                         scores, res["ids"], res["teacher"], *out, scores_selected=fused)
    torch.cuda.synchronize()
    return a, b


CASES = [
    # (workload, fused score + top-k route): largest scratch first, then smaller ones
    (I.WORKLOADS[2], False),                                          # ~114 MiB of scratch
    (I.WORKLOADS[1], True),                                           # batch 2 x 4096, 64 MiB
    (I.scaled_down(I.WORKLOADS[1], (512, 300), topk=40), False),
    (I.scaled_down(I.WORKLOADS[4], (640,), topk=16), False),          # dense loss
    (I.scaled_down(I.WORKLOADS[2], (128, 256, 200, 68), topk=24), False),
]


def test_noalloc_backward_equals_workspace_route(gpu_ok):
    for wl, fused in CASES:
        print("noalloc case", wl.name, "fused" if fused else "two calls", flush=True)
        inp = I.make_inputs(wl, device="cuda")
        a, b = _both(inp, fused)
        for name, x, y in zip(("dq_idx", "dweights", "dk_idx"), a, b):
            assert bool(torch.isfinite(y).all()), (wl.name, name)
            assert torch.equal(x, y), (wl.name, name)
        del inp, a, b
        torch.cuda.empty_cache()


def test_noalloc_rejects_a_layout_beyond_the_scratch(gpu_ok):
    """16,384 rows x 4,096 compressed keys need 256 MiB of score gradients: rejected on the
    host (nothing is launched, so small placeholder tensors do)."""
    ops = _ops()
    L = ops.Layout.from_lengths([16384], [4096], 4)
    t = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device="cuda")
    f = lambda *s: torch.zeros(s, dtype=torch.float32, device="cuda")
    ids = torch.zeros((1, 64), dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError, match="scratch"):
        ops.csa_indexer_loss_bwd_noalloc(L, True, t(1, 16, 64), t(1, 64), f(1, 16), 0.125, f(1, 64), ids,
                                         f(1, 64), f(1, 16, 64), f(1, 16), f(1, 64), scores_selected=True)
