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
    return sorted(set(re.findall(r"^\s*(?:csa_status_t|const char \*|int32_t)\s*(csa_\w+)\s*\(", src, re.M)))


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
                          "csa_sparse_attn_fwd", "csa_indexer_teacher_kl", "csa_indexer_loss_bwd"}
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
    st = lib.csa_topk(ctypes.byref(L), FAKE, 16, 4, FAKE, None)
    assert st == code
    assert lib.csa_last_error().decode().startswith("csa_topk")


def test_argument_misuse_is_rejected(lib):
    from deepseek_v4_csa_amd import ops
    L = _layout(ops)
    B = ctypes.byref
    assert lib.csa_topk(B(L), FAKE, 16, 0, FAKE, None) == 1                      # topk < 1
    assert lib.csa_topk(B(L), FAKE, 8, 4, FAKE, None) == 1                       # ld < max_seqlen_k
    assert lib.csa_topk(B(L), None, 16, 4, FAKE, None) == 1                      # null scores
    assert lib.csa_indexer_score(B(L), FAKE, FAKE, FAKE, 1, 4, 48, 0.1, FAKE, 16, None) == 2  # Di=48
    assert lib.csa_indexer_score(B(L), FAKE, FAKE, FAKE, 7, 4, 64, 0.1, FAKE, 16, None) == 1  # dtype
    assert lib.csa_sparse_attn_fwd(B(L), FAKE, FAKE, FAKE, FAKE, FAKE, 4, -1, 1, 4, 64, 0.1,
                                   FAKE, FAKE, FAKE, None, None) == 1            # window < 0
    assert lib.csa_sparse_attn_fwd(B(L), FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 1, 4, 96, 0.1,
                                   FAKE, FAKE, FAKE, None, None) == 2            # D = 96
    assert lib.csa_sparse_attn_fwd(B(L), FAKE, FAKE, FAKE, FAKE, FAKE, 32, 8, 1, 4, 64, 0.1,
                                   FAKE, FAKE, FAKE, None, None) == 1            # k_eff > max_seqlen_k
    assert lib.csa_indexer_teacher_kl(B(L), 1, FAKE, 16, None, 4, FAKE, None, None, None, 1, 4, 64,
                                      0.1, 0, None, 0, FAKE, FAKE, None) == 1    # sparse without ids
    assert lib.csa_indexer_teacher_kl(B(L), 0, FAKE, 16, None, 0, None, FAKE, FAKE, FAKE, 0, 4, 64,
                                      0.1, 0, None, 0, FAKE, FAKE, None) == 2    # dense fp32
    assert "dense" in lib.csa_last_error().decode()
    bwd = lib.csa_indexer_loss_bwd
    args = [B(L), 1, FAKE, FAKE, FAKE, 1, 16, 64, 0.1, FAKE, 16, FAKE, 4, FAKE, 4, 1.0, 0, FAKE, 16,
            FAKE, FAKE, FAKE, None]
    a = list(args); a[11] = None
    assert bwd(*a) == 1                                                            # sparse without ids
    a = list(args); a[14] = 3
    assert bwd(*a) == 1                                                            # ld_teacher < k_eff
    a = list(args); a[18] = 8
    assert bwd(*a) == 1                                                            # ld_grad < max_seqlen_k
    a = list(args); a[7] = 96
    assert bwd(*a) == 2                                                            # Di = 96
    a = list(args); a[5] = 0
    assert bwd(*a) == 2                                                            # fp32
    a = list(args); a[19] = None
    assert bwd(*a) == 1                                                            # null dq


def test_k_eff(lib):
    from deepseek_v4_csa_amd import ops
    L = _layout(ops)
    assert lib.csa_k_eff(ctypes.byref(L), 4) == 4
    assert lib.csa_k_eff(ctypes.byref(L), 400) == 16
    assert lib.csa_k_eff(ctypes.byref(L), -1) == -1
