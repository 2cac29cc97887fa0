"""The C-ABI library loads without a GPU, exports every symbol include/csa.h declares,
and rejects host-visible misuse before launching anything (no compute call is made)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:csa_status_t|const char \*|int32_t|int64_t)\s*(csa_\w+)\s*\(", src, re.M)))


@pytest.fixture(scope="module")
def lib():
    import torch  # noqa: F401  (the binding always loads the library after torch)
    from deepseek_v4_csa_amd import ops
    if not os.path.exists(ops.lib_path()):
        pytest.fail("libcsa.so is not built (python -m deepseek_v4_csa_amd.build)")
    return ops.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert set(names) == {"csa_last_error", "csa_k_eff", "csa_indexer_score", "csa_topk",
                          "csa_sparse_attn_fwd", "csa_indexer_teacher_kl", "csa_indexer_loss_bwd",
                          "csa_indexer_loss_bwd_workspace", "csa_cp_plan", "csa_indexer_topk",
                          "csa_sparse_attn_kl_fwd", "csa_loss_reduce", "csa_indexer_loss_bwd_noalloc"}
    from deepseek_v4_csa_amd import ops
    assert set(ops.EXPORTS) == set(names)
    for n in names:
        assert hasattr(lib, n), n


def _layout(ops, **kw):
    d = dict(num_seqs=1, total_q=64, total_k=16, max_seqlen_q=64, max_seqlen_k=16, compress_ratio=4,
             cu_seqlens_q=0x1000, cu_seqlens_k=0x2000, q_causal_offsets=None)
    d.update(kw)
    return ops._CLayout(**d)


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every case below fails validation first


@pytest.mark.parametrize("kw,code", [
    (dict(total_k=0), 1), (dict(num_seqs=0), 1), (dict(compress_ratio=0), 1),
    (dict(max_seqlen_k=0), 1), (dict(cu_seqlens_q=None), 1), (dict(max_seqlen_k=32), 1),
])
def test_layout_misuse_is_rejected(lib, kw, code):
    from deepseek_v4_csa_amd import ops
    L = _layout(ops, **kw)
    st = lib.csa_topk(ctypes.byref(L), FAKE, 16, 4, FAKE, None, None)
    assert st == code
    assert lib.csa_last_error().decode().startswith("csa_topk")


def test_argument_misuse_is_rejected(lib):
    from deepseek_v4_csa_amd import ops
    L = _layout(ops)
    B = ctypes.byref
    assert lib.csa_topk(B(L), FAKE, 16, 0, FAKE, None, None) == 1                      # topk < 1
    assert lib.csa_topk(B(L), FAKE, 8, 4, FAKE, None, None) == 1                       # ld < max_seqlen_k
    assert lib.csa_topk(B(L), None, 16, 4, FAKE, None, None) == 1                      # null scores
    assert lib.csa_indexer_score(B(L), FAKE, FAKE, FAKE, 1, 4, 48, 0.1, FAKE, 16, None) == 2  # Di=48
    assert lib.csa_indexer_score(B(L), FAKE, FAKE, FAKE, 7, 4, 64, 0.1, FAKE, 16, None) == 1  # dtype
    assert lib.csa_sparse_attn_fwd(B(L), FAKE, FAKE, FAKE, FAKE, FAKE, 4, -1, 1, 4, 64, 0.1,
                                   FAKE, FAKE, FAKE, None, None) == 1            # window < 0
    assert lib.csa_sparse_attn_fwd(B(L), FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 1, 4, 96, 0.1,
                                   FAKE, FAKE, FAKE, None, None) == 2            # D = 96
    assert lib.csa_sparse_attn_fwd(B(L), FAKE, FAKE, FAKE, FAKE, FAKE, 32, 8, 1, 4, 64, 0.1,
                                   FAKE, FAKE, FAKE, None, None) == 1            # k_eff > max_seqlen_k
    for bad in (0.0, -0.1, float("inf"), float("nan")):
        assert lib.csa_sparse_attn_fwd(B(L), FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 1, 4, 64, bad,
                                       FAKE, FAKE, FAKE, None, None) == 1        # softmax_scale
        assert "softmax_scale" in lib.csa_last_error().decode()
    assert lib.csa_indexer_teacher_kl(B(L), 1, FAKE, 16, 0, None, 4, FAKE, None, None, None, 1, 4, 64,
                                      0.1, 0, None, 0, FAKE, FAKE, None) == 1    # sparse without ids
    assert lib.csa_indexer_teacher_kl(B(L), 0, FAKE, 16, 1, None, 0, None, FAKE, FAKE, FAKE, 1, 4, 64,
                                      0.1, 0, None, 0, FAKE, FAKE, None) == 1    # dense + selected
    assert "selected" in lib.csa_last_error().decode()
    assert lib.csa_indexer_teacher_kl(B(L), 1, FAKE, 3, 1, FAKE, 4, FAKE, None, None, None, 1, 4, 64,
                                      0.1, 0, None, 0, FAKE, FAKE, None) == 1    # selected ld < k_eff
    assert lib.csa_indexer_teacher_kl(B(L), 0, FAKE, 16, 0, None, 0, None, FAKE, FAKE, FAKE, 0, 4, 64,
                                      0.1, 0, None, 0, FAKE, FAKE, None) == 2    # dense fp32
    assert "dense" in lib.csa_last_error().decode()
    bwd = lib.csa_indexer_loss_bwd
    args = [B(L), 1, FAKE, FAKE, FAKE, 1, 16, 64, 0.1, FAKE, 16, 0, FAKE, 4, FAKE, 4, 1.0, 0, FAKE, 16,
            FAKE, FAKE, FAKE, FAKE, 0, None]
    a = list(args); a[12] = None
    assert bwd(*a) == 1                                                            # sparse without ids
    a = list(args); a[15] = 3
    assert bwd(*a) == 1                                                            # ld_teacher < k_eff
    a = list(args); a[19] = 8
    assert bwd(*a) == 1                                                            # ld_grad < max_seqlen_k
    a = list(args); a[7] = 96
    assert bwd(*a) == 2                                                            # Di = 96
    a = list(args); a[5] = 0
    assert bwd(*a) == 2                                                            # fp32
    a = list(args); a[20] = None
    assert bwd(*a) == 1                                                            # null dq
    a = list(args); a[1] = 0; a[11] = 1
    assert bwd(*a) == 1                                                            # dense + selected
    a = list(args); a[10] = 3; a[11] = 1
    assert bwd(*a) == 1                                                            # selected ld < k_eff
    # a long segment splits dk over token chunks: the workspace must hold the partials
    Lb = _layout(ops, total_q=4096, max_seqlen_q=4096, total_k=1024, max_seqlen_k=1024)
    need = lib.csa_indexer_loss_bwd_workspace(B(Lb), 16, 64)
    assert need == 64 * 1024 * 64 * 4
    # 65,536 tokens, 128 key tiles: 8 chunks would fill the chip, but a chunk holds at most
    # 64 of the 4,096 token blocks, so 64 chunks of partials (Di = 128)
    Ll = _layout(ops, total_q=65536, max_seqlen_q=65536, total_k=16384, max_seqlen_k=16384)
    assert lib.csa_indexer_loss_bwd_workspace(B(Ll), 64, 128) == 64 * 16384 * 128 * 4
    a = list(args); a[0] = B(Lb); a[10] = a[19] = 1024; a[24] = need - 1
    assert bwd(*a) == 1                                                            # workspace too small
    assert "workspace" in lib.csa_last_error().decode()
    a[23] = None; a[24] = need
    assert bwd(*a) == 1                                                            # workspace NULL
    # fused score + top-k
    fz = lib.csa_indexer_topk
    assert fz(B(L), FAKE, FAKE, FAKE, 1, 16, 64, 0.1, 0, FAKE, FAKE, None, None) == 1   # topk < 1
    assert fz(B(L), FAKE, FAKE, FAKE, 1, 16, 64, 0.1, 4, FAKE, None, None, None) == 1   # null sel
    assert fz(B(L), FAKE, FAKE, FAKE, 1, 24, 64, 0.1, 4, FAKE, FAKE, None, None) == 2   # Hi = 24
    assert fz(B(L), FAKE, FAKE, FAKE, 0, 16, 64, 0.1, 4, FAKE, FAKE, None, None) == 2   # fp32
    Lw = _layout(ops, total_q=8192, max_seqlen_q=8192, total_k=2048, max_seqlen_k=2048)
    assert fz(B(Lw), FAKE, FAKE, FAKE, 1, 16, 64, 0.1, 4, FAKE, FAKE, None, None) == 2  # rows too long
    assert "fused" in lib.csa_last_error().decode()
    assert fz(B(Lw), FAKE, FAKE, FAKE, 1, 32, 64, 0.1, 4, FAKE, FAKE, None, None) == 2  # grouped: too long
    # attention + teacher/KL in one call
    akl = lib.csa_sparse_attn_kl_fwd
    args = [B(L), FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 1, 4, 64, 0.1, FAKE, 4, 1, 0,
            FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, FAKE, None]
    a = list(args); a[6] = 0
    assert akl(*a) == 1                                                            # k_eff = 0
    a = list(args); a[19] = None
    assert akl(*a) == 1                                                            # null cmass
    a = list(args); a[12] = None
    assert akl(*a) == 1                                                            # null scores
    a = list(args); a[13] = 3
    assert akl(*a) == 1                                                            # selected ld < k_eff
    a = list(args); a[14] = 0
    assert akl(*a) == 1                                                            # full rows ld < max_seqlen_k
    a = list(args); a[20] = FAKE; a[21] = 3
    assert akl(*a) == 1                                                            # ld_teacher < k_eff
    a = list(args); a[7] = -1
    assert akl(*a) == 1                                                            # window < 0
    a = list(args); a[10] = 96
    assert akl(*a) == 2                                                            # D = 96
    a = list(args); a[11] = -1.0
    assert akl(*a) == 1                                                            # softmax_scale < 0
    assert lib.csa_last_error().decode().startswith("csa_sparse_attn_kl_fwd")
    assert lib.csa_loss_reduce(FAKE, 16, 0, None, None) == 1                      # null loss
    assert lib.csa_loss_reduce(None, 16, 0, FAKE, None) == 1                      # null kl_row
    assert lib.csa_loss_reduce(FAKE, -1, 0, FAKE, None) == 1                      # total_q < 0


def test_backward_workspace_query(lib):
    from deepseek_v4_csa_amd import ops
    B = ctypes.byref
    assert lib.csa_indexer_loss_bwd_workspace(B(_layout(ops)), 16, 64) == 0        # one chunk
    assert lib.csa_indexer_loss_bwd_workspace(B(_layout(ops)), 16, 96) == -1       # no kernel
    assert lib.csa_indexer_loss_bwd_workspace(B(_layout(ops, total_k=0)), 16, 64) == -1


def test_k_eff(lib):
    from deepseek_v4_csa_amd import ops
    L = _layout(ops)
    assert lib.csa_k_eff(ctypes.byref(L), 4) == 4
    assert lib.csa_k_eff(ctypes.byref(L), 400) == 16
    assert lib.csa_k_eff(ctypes.byref(L), -1) == -1


def test_ctypes_layout_matches_the_header(tmp_path):
    """csa_layout_t as the C compiler lays it out (gcc on the header) equals the binding's
    ctypes mirror, field by field."""
    import shutil
    import subprocess
    from deepseek_v4_csa_amd import ops
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    fields = [f for f, _ in ops._CLayout._fields_]
    src = tmp_path / "lay.c"
    body = "".join(f'  printf("%zu ", offsetof(csa_layout_t, {f}));\n' for f in fields)
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "csa.h"\nint main(void) {\n'
                   + body + '  printf("%zu\\n", sizeof(csa_layout_t));\n  return 0;\n}\n')
    exe = tmp_path / "lay"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    want = [getattr(ops._CLayout, f).offset for f in fields] + [ctypes.sizeof(ops._CLayout)]
    assert got == want


CP_CASES = [((4096,), 4, 1, 0), ((4096,), 4, 2, 0), ((4096,), 4, 2, 1), ((1024, 2048), 4, 2, 0),
            ((1024, 2048), 4, 2, 1), ((96, 48, 240), 3, 4, 3), ((40,), 16, 2, 1)]


@pytest.mark.parametrize("docs,ratio,cp,rank", CP_CASES)
def test_cp_plan_matches_the_zigzag_rule(lib, docs, ratio, cp, rank):
    from deepseek_v4_csa_amd import ops
    from tests import cp_rule
    plan = ops.csa_cp_plan(docs, ratio, cp, rank)
    want = cp_rule.share(docs, ratio, cp, rank)
    assert len(plan["off"]) == len(want) == 2 * len(docs)
    for s, (d, a, c, nk, r0, k0) in enumerate(want):
        assert plan["cu_q"][s + 1] - plan["cu_q"][s] == c
        assert plan["cu_k"][s + 1] - plan["cu_k"][s] == nk
        assert (plan["off"][s], plan["q_src"][s], plan["k_src"][s]) == (a, r0, k0)
    assert plan["cu_q"][0] == plan["cu_k"][0] == 0


def test_cp_plan_ranks_cover_every_row_once(lib):
    from deepseek_v4_csa_amd import ops
    docs, cp = (64, 128, 32), 4
    seen = []
    for r in range(cp):
        p = ops.csa_cp_plan(docs, 4, cp, r)
        for s in range(len(p["off"])):
            seen += range(p["q_src"][s], p["q_src"][s] + p["cu_q"][s + 1] - p["cu_q"][s])
    assert sorted(seen) == list(range(sum(docs)))


@pytest.mark.parametrize("args", [((0,), 4, 1, 0), ((4096,), 0, 1, 0), ((4096,), 4, 0, 0),
                                  ((4096,), 4, 2, 2), ((4096,), 4, 2, -1), ((100,), 4, 3, 0)])
def test_cp_plan_rejects_misuse(lib, args):
    from deepseek_v4_csa_amd import ops
    with pytest.raises(RuntimeError, match="csa_cp_plan"):
        ops.csa_cp_plan(*args)
