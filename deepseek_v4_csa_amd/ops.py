"""Thin Python binding of libcsa.so (include/csa.h): argument marshalling only.

Every function here has the name of a C entry point, takes torch tensors already on the
GPU, passes their device pointers and the current HIP stream, and raises RuntimeError
with the library's message when the call returns a non-OK status.  No arithmetic of
the method runs in Python; there is no CPU fallback: if the library is missing or the
tensors are not on a GPU the call fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa.so")
_lib = None

CSA_F32, CSA_BF16 = 0, 1


class _CLayout(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("total_q", ctypes.c_int32),
        ("total_k", ctypes.c_int32),
        ("max_seqlen_q", ctypes.c_int32),
        ("max_seqlen_k", ctypes.c_int32),
        ("compress_ratio", ctypes.c_int32),
        ("cu_seqlens_q", ctypes.c_void_p),
        ("cu_seqlens_k", ctypes.c_void_p),
        ("q_causal_offsets", ctypes.c_void_p),
        ("cu_seqlens_q_unpadded", ctypes.c_void_p),
    ]


EXPORTS = ("csa_last_error", "csa_k_eff", "csa_indexer_score", "csa_topk",
           "csa_sparse_attn_fwd", "csa_indexer_teacher_kl", "csa_indexer_loss_bwd", "csa_indexer_loss_bwd_workspace",
           "csa_cp_plan", "csa_indexer_topk", "csa_sparse_attn_kl_fwd", "csa_loss_reduce",
           "csa_indexer_loss_bwd_noalloc")


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libcsa.so (after torch, so the process keeps a single HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run `python -m deepseek_v4_csa_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    LP = ctypes.POINTER(_CLayout)
    lib.csa_last_error.restype = ctypes.c_char_p
    lib.csa_last_error.argtypes = []
    lib.csa_k_eff.restype = I32
    lib.csa_k_eff.argtypes = [LP, I32]
    lib.csa_indexer_score.restype = ctypes.c_int
    lib.csa_indexer_score.argtypes = [LP, P, P, P, ctypes.c_int, I32, I32, F32, P, I64, P]
    lib.csa_topk.restype = ctypes.c_int
    lib.csa_topk.argtypes = [LP, P, I64, I32, P, P, P]
    lib.csa_sparse_attn_fwd.restype = ctypes.c_int
    lib.csa_sparse_attn_fwd.argtypes = [LP, P, P, P, P, P, I32, I32, ctypes.c_int, I32, I32, F32,
                                        P, P, P, P, P]
    lib.csa_indexer_teacher_kl.restype = ctypes.c_int
    lib.csa_indexer_teacher_kl.argtypes = [LP, I32, P, I64, I32, P, I32, P, P, P, P, ctypes.c_int, I32,
                                           I32, F32, I32, P, I64, P, P, P]
    lib.csa_indexer_loss_bwd.restype = ctypes.c_int
    lib.csa_indexer_loss_bwd.argtypes = [LP, I32, P, P, P, ctypes.c_int, I32, I32, F32, P, I64, I32, P,
                                         I32, P, I64, F32, I32, P, I64, P, P, P, P, I64, P]
    lib.csa_indexer_loss_bwd_noalloc.restype = ctypes.c_int
    lib.csa_indexer_loss_bwd_noalloc.argtypes = [LP, I32, P, P, P, ctypes.c_int, I32, I32, F32, P, I64, I32, P,
                                                 I32, P, I64, F32, I32, P, P, P, P]
    lib.csa_indexer_loss_bwd_workspace.restype = I64
    lib.csa_indexer_loss_bwd_workspace.argtypes = [LP, I32, I32]
    lib.csa_indexer_topk.restype = ctypes.c_int
    lib.csa_indexer_topk.argtypes = [LP, P, P, P, ctypes.c_int, I32, I32, F32, I32, P, P, P, P]
    lib.csa_sparse_attn_kl_fwd.restype = ctypes.c_int
    lib.csa_sparse_attn_kl_fwd.argtypes = [LP, P, P, P, P, P, I32, I32, ctypes.c_int, I32, I32, F32, P, I64, I32,
                                           I32, P, P, P, P, P, I64, P, P, P]
    lib.csa_loss_reduce.restype = ctypes.c_int
    lib.csa_loss_reduce.argtypes = [P, I32, I32, P, P]
    lib.csa_cp_plan.restype = ctypes.c_int
    lib.csa_cp_plan.argtypes = [I32, P, I32, I32, I32, P, P, P, P, P, P]
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        msg = load().csa_last_error().decode()
        raise RuntimeError(f"libcsa status {status}: {msg}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise RuntimeError("libcsa takes GPU tensors only")
    if not t.is_contiguous():
        raise RuntimeError("libcsa takes contiguous tensors only")
    return ctypes.c_void_p(t.data_ptr())


def _dtype(t) -> int:
    if t.dtype == torch.bfloat16:
        return CSA_BF16
    if t.dtype == torch.float32:
        return CSA_F32
    raise RuntimeError(f"unsupported dtype {t.dtype}")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


_POISON = [False]


class poisoned_outputs:
    """Within this context every output tensor the functions below allocate is filled
    with NaN (float) or -2 (int32, never a valid id or -1) instead of being left
    uninitialised, so an element a kernel fails to write shows up in a comparison."""

    def __enter__(self):
        self._prev = _POISON[0]
        _POISON[0] = True
        return self

    def __exit__(self, *exc):
        _POISON[0] = self._prev
        return False


def _new(shape, dtype, device):
    if not _POISON[0]:
        return torch.empty(shape, dtype=dtype, device=device)
    fill = -2 if dtype == torch.int32 else float("nan")
    return torch.full(shape, fill, dtype=dtype, device=device)


def _new_like(t):
    return _new(tuple(t.shape), t.dtype, t.device)


@dataclass
class Layout:
    """Packed layout: device int32 cu_seqlens (offsets, unpadded cu_seqlens) plus host sizes."""
    cu_q: torch.Tensor
    cu_k: torch.Tensor
    ratio: int
    total_q: int
    total_k: int
    max_seqlen_q: int
    max_seqlen_k: int
    offsets: torch.Tensor | None = None
    cu_q_real: torch.Tensor | None = None

    @property
    def num_seqs(self) -> int:
        return self.cu_q.numel() - 1

    @classmethod
    def from_lengths(cls, seg_q, seg_k, ratio, device="cuda", offsets=None):
        cq = [0]
        ck = [0]
        for a, b in zip(seg_q, seg_k):
            cq.append(cq[-1] + int(a))
            ck.append(ck[-1] + int(b))
        mk = lambda v: torch.tensor(v, dtype=torch.int32, device=device)
        return cls(mk(cq), mk(ck), int(ratio), cq[-1], ck[-1], max(int(a) for a in seg_q),
                   max(int(b) for b in seg_k), None if offsets is None else mk(list(offsets)))

    def c(self) -> _CLayout:
        return _CLayout(self.num_seqs, int(self.total_q), int(self.total_k), int(self.max_seqlen_q),
                        int(self.max_seqlen_k), int(self.ratio), _ptr(self.cu_q), _ptr(self.cu_k),
                        _ptr(self.offsets) if self.offsets is not None else None,
                        _ptr(self.cu_q_real) if self.cu_q_real is not None else None)


def k_eff(layout: Layout, topk: int) -> int:
    return int(load().csa_k_eff(ctypes.byref(layout.c()), int(topk)))


def csa_indexer_score(layout: Layout, q_idx, k_idx, weights, idx_scale: float, scores=None):
    T, Hi, Di = q_idx.shape
    if scores is None:
        scores = _new((T, layout.max_seqlen_k), torch.float32, q_idx.device)
    _check(load().csa_indexer_score(ctypes.byref(layout.c()), _ptr(q_idx), _ptr(k_idx), _ptr(weights),
                                    _dtype(q_idx), Hi, Di, float(idx_scale), _ptr(scores),
                                    scores.stride(0), _stream()))
    return scores


def csa_topk(layout: Layout, scores, topk: int, ids=None, sel_scores=None):
    """ids [T, k_eff]; with sel_scores (a [T, k_eff] fp32 tensor) also the score of each
    selected id, slot-aligned with ids."""
    ke = k_eff(layout, topk)
    if ids is None:
        ids = _new((scores.shape[0], ke), torch.int32, scores.device)
    _check(load().csa_topk(ctypes.byref(layout.c()), _ptr(scores), scores.stride(0), int(topk),
                           _ptr(ids), _ptr(sel_scores) if sel_scores is not None else None, _stream()))
    return ids


def csa_sparse_attn_fwd(layout: Layout, q, kv, ckv, sink, ids, window: int, softmax_scale: float,
                        out=None, lse=None, lse_nc=None, cmass=None, want_cmass=True):
    T, H, D = q.shape
    k_eff_ = ids.shape[1]
    dev = q.device
    out = _new_like(q) if out is None else out
    lse = _new((T, H), torch.float32, dev) if lse is None else lse
    lse_nc = _new((T, H), torch.float32, dev) if lse_nc is None else lse_nc
    if want_cmass and cmass is None:
        cmass = _new((T, k_eff_), torch.float32, dev)
    _check(load().csa_sparse_attn_fwd(ctypes.byref(layout.c()), _ptr(q), _ptr(kv), _ptr(ckv), _ptr(sink),
                                      _ptr(ids), k_eff_, int(window), _dtype(q), H, D,
                                      float(softmax_scale), _ptr(out), _ptr(lse), _ptr(lse_nc),
                                      _ptr(cmass) if want_cmass else None, _stream()))
    return out, lse, lse_nc, cmass


def csa_sparse_attn_kl_fwd(layout: Layout, q, kv, ckv, sink, ids, window: int, softmax_scale: float, scores,
                           scores_selected: bool, per_token: bool = False, want_teacher: bool = False,
                           out=None, lse=None, lse_nc=None, cmass=None, teacher=None, kl_row=None, loss=None,
                           reduce: bool = True):
    """Attention + sparse-loss teacher + KL + loss in one call:
    (out, lse, lse_nc, cmass, teacher or None, kl_row, loss); reduce=False leaves the loss
    to csa_loss_reduce (loss is then None)."""
    T, H, D = q.shape
    k_eff_ = ids.shape[1]
    dev = q.device
    f32 = torch.float32
    out = _new_like(q) if out is None else out
    lse = _new((T, H), f32, dev) if lse is None else lse
    lse_nc = _new((T, H), f32, dev) if lse_nc is None else lse_nc
    cmass = _new((T, k_eff_), f32, dev) if cmass is None else cmass
    if want_teacher and teacher is None:
        teacher = _new((T, k_eff_), f32, dev)
    kl_row = _new((T,), f32, dev) if kl_row is None else kl_row
    if reduce and loss is None:
        loss = _new((1,), f32, dev)
    if not reduce:
        loss = None
    _check(load().csa_sparse_attn_kl_fwd(
        ctypes.byref(layout.c()), _ptr(q), _ptr(kv), _ptr(ckv), _ptr(sink), _ptr(ids), k_eff_, int(window),
        _dtype(q), H, D, float(softmax_scale), _ptr(scores), scores.stride(0), 1 if scores_selected else 0,
        1 if per_token else 0, _ptr(out), _ptr(lse), _ptr(lse_nc), _ptr(cmass),
        _ptr(teacher) if teacher is not None else None, teacher.stride(0) if teacher is not None else 0,
        _ptr(kl_row), _ptr(loss) if loss is not None else None, _stream()))
    return out, lse, lse_nc, cmass, teacher, kl_row, loss


def csa_loss_reduce(kl_row, per_token: bool = False, loss=None):
    """loss = sum(kl_row) / len(kl_row) (or the sum), reduced on the GPU in a fixed order."""
    loss = _new((1,), torch.float32, kl_row.device) if loss is None else loss
    _check(load().csa_loss_reduce(_ptr(kl_row), int(kl_row.shape[0]), 1 if per_token else 0, _ptr(loss),
                                  _stream()))
    return loss


def csa_indexer_topk(layout: Layout, q_idx, k_idx, weights, idx_scale: float, topk: int, ids=None,
                     sel_scores=None, row_lse=None, want_lse: bool = False):
    """Fused scores + top-k: (ids, sel_scores, row_lse or None); the score matrix is never
    stored."""
    T, Hi, Di = q_idx.shape
    dev = q_idx.device
    k = k_eff(layout, topk)
    ids = _new((T, k), torch.int32, dev) if ids is None else ids
    sel_scores = _new((T, k), torch.float32, dev) if sel_scores is None else sel_scores
    if want_lse and row_lse is None:
        row_lse = _new((T,), torch.float32, dev)
    _check(load().csa_indexer_topk(ctypes.byref(layout.c()), _ptr(q_idx), _ptr(k_idx), _ptr(weights),
                                   _dtype(q_idx), Hi, Di, float(idx_scale), int(topk), _ptr(ids),
                                   _ptr(sel_scores), _ptr(row_lse) if row_lse is not None else None,
                                   _stream()))
    return ids, sel_scores, row_lse


def csa_indexer_teacher_kl(layout: Layout, sparse_loss: bool, scores, ids, cmass, q, ckv, lse_nc,
                           softmax_scale: float, per_token: bool = False, want_teacher: bool = False,
                           teacher=None, kl_row=None, loss=None, scores_selected: bool = False):
    T = scores.shape[0]
    dev = scores.device
    H = q.shape[1] if q is not None else 1
    D = q.shape[2] if q is not None else 1
    k_eff_ = ids.shape[1] if ids is not None else 0
    if want_teacher and teacher is None:
        width = k_eff_ if sparse_loss else layout.max_seqlen_k
        teacher = _new((T, width), torch.float32, dev)
    kl_row = _new((T,), torch.float32, dev) if kl_row is None else kl_row
    loss = _new((1,), torch.float32, dev) if loss is None else loss
    dt = _dtype(q) if q is not None else CSA_BF16
    _check(load().csa_indexer_teacher_kl(
        ctypes.byref(layout.c()), 1 if sparse_loss else 0, _ptr(scores), scores.stride(0),
        1 if scores_selected else 0,
        _ptr(ids) if ids is not None else None, k_eff_, _ptr(cmass) if cmass is not None else None,
        _ptr(q) if q is not None else None, _ptr(ckv) if ckv is not None else None,
        _ptr(lse_nc) if lse_nc is not None else None, dt, H, D, float(softmax_scale),
        1 if per_token else 0, _ptr(teacher) if teacher is not None else None,
        teacher.stride(0) if teacher is not None else 0, _ptr(kl_row), _ptr(loss), _stream()))
    return teacher, kl_row, loss


def csa_indexer_loss_bwd(layout: Layout, sparse_loss: bool, q_idx, k_idx, weights, idx_scale: float,
                         scores, ids, teacher, grad_loss: float = 1.0, per_token: bool = False,
                         grad_scores=None, dq_idx=None, dweights=None, dk_idx=None, workspace=None,
                         scores_selected: bool = False):
    """Indexer-loss gradients (fp32) for q_idx, weights and k_idx; the teacher and the
    selection (ids) of the forward are held fixed.  workspace: a uint8 device tensor of at
    least csa_indexer_loss_bwd_workspace bytes (allocated here if None)."""
    T, Hi, Di = q_idx.shape
    dev = q_idx.device
    k_eff_ = ids.shape[1] if ids is not None else 0
    if grad_scores is None:
        grad_scores = _new((T, layout.max_seqlen_k), torch.float32, dev)
    dq_idx = _new((T, Hi, Di), torch.float32, dev) if dq_idx is None else dq_idx
    dweights = _new((T, Hi), torch.float32, dev) if dweights is None else dweights
    dk_idx = _new(tuple(k_idx.shape), torch.float32, dev) if dk_idx is None else dk_idx
    if workspace is None:
        n = csa_indexer_loss_bwd_workspace(layout, Hi, Di)
        workspace = torch.empty((max(n, 1),), dtype=torch.uint8, device=dev)
    _check(load().csa_indexer_loss_bwd(
        ctypes.byref(layout.c()), 1 if sparse_loss else 0, _ptr(q_idx), _ptr(k_idx), _ptr(weights),
        _dtype(q_idx), Hi, Di, float(idx_scale), _ptr(scores), scores.stride(0), 1 if scores_selected else 0,
        _ptr(ids) if ids is not None else None, k_eff_, _ptr(teacher), teacher.stride(0),
        float(grad_loss), 1 if per_token else 0, _ptr(grad_scores), grad_scores.stride(0),
        _ptr(dq_idx), _ptr(dweights), _ptr(dk_idx), _ptr(workspace), workspace.numel(), _stream()))
    return dq_idx, dweights, dk_idx


def csa_indexer_loss_bwd_noalloc(layout: Layout, sparse_loss: bool, q_idx, k_idx, weights, idx_scale: float,
                                 scores, ids, teacher, dq_idx, dweights, dk_idx, grad_loss: float = 1.0,
                                 per_token: bool = False, scores_selected: bool = False):
    """csa_indexer_loss_bwd with the library's static device scratch in place of the
    grad_scores and workspace buffers: the C call allocates nothing, so the outputs
    (fp32 dq_idx [T, Hi, Di], dweights [T, Hi], dk_idx [T_k, Di]) are the caller's."""
    T, Hi, Di = q_idx.shape
    k_eff_ = ids.shape[1] if ids is not None else 0
    _check(load().csa_indexer_loss_bwd_noalloc(
        ctypes.byref(layout.c()), 1 if sparse_loss else 0, _ptr(q_idx), _ptr(k_idx), _ptr(weights),
        _dtype(q_idx), Hi, Di, float(idx_scale), _ptr(scores), scores.stride(0), 1 if scores_selected else 0,
        _ptr(ids) if ids is not None else None, k_eff_, _ptr(teacher), teacher.stride(0),
        float(grad_loss), 1 if per_token else 0, _ptr(dq_idx), _ptr(dweights), _ptr(dk_idx), _stream()))
    return dq_idx, dweights, dk_idx


def csa_indexer_loss_bwd_workspace(layout: Layout, Hi: int, Di: int) -> int:
    """Bytes of device workspace csa_indexer_loss_bwd needs (host-only query)."""
    n = int(load().csa_indexer_loss_bwd_workspace(ctypes.byref(layout.c()), int(Hi), int(Di)))
    if n < 0:
        raise RuntimeError(f"libcsa: {load().csa_last_error().decode()}")
    return n


def csa_cp_plan(doc_lens, ratio: int, cp_size: int, cp_rank: int) -> dict:
    """Host-only: the packed layout of one rank's CP share (lists of Python ints:
    cu_q, cu_k, off, q_src, k_src)."""
    lib = load()
    n = len(doc_lens)
    arr = lambda m: (ctypes.c_int32 * m)()
    dl = (ctypes.c_int32 * n)(*[int(x) for x in doc_lens])
    ns = ctypes.c_int32(0)
    cu_q, cu_k, off, q_src, k_src = arr(2 * n + 1), arr(2 * n + 1), arr(2 * n), arr(2 * n), arr(2 * n)
    _check(lib.csa_cp_plan(n, dl, int(ratio), int(cp_size), int(cp_rank), ctypes.byref(ns), cu_q,
                           cu_k, off, q_src, k_src))
    m = ns.value
    return dict(cu_q=list(cu_q[:m + 1]), cu_k=list(cu_k[:m + 1]), off=list(off[:m]),
                q_src=list(q_src[:m]), k_src=list(k_src[:m]))


def layout_of_inputs(inp) -> Layout:
    """Layout of a deepseek_v4_csa_amd.inputs.Inputs (device tensors already built)."""
    wl = inp.wl
    return Layout(inp.cu_q, inp.cu_k, wl.ratio, wl.total_q, wl.total_k, wl.max_seqlen_q,
                  wl.max_seqlen_k, inp.offsets, inp.cu_q_real)


def forward(inp, want_teacher=False, fused=False, attn_kl=False, topk_sel=False, poison=False):
    """The whole path on one Inputs, on the current stream: the four calls, or with
    fused=True (sparse loss) csa_indexer_topk in place of the score and top-k calls, the
    teacher/KL then reading the selected scores (no score matrix: scores is None), and
    with attn_kl=True (sparse loss) csa_sparse_attn_kl_fwd in place of the attention and
    teacher/KL calls.  topk_sel=True (sparse loss, two score calls): csa_topk also writes
    the selected scores and the teacher/KL reads those instead of gathering from the rows.
    poison=True: the outputs start as NaN / -2 (see poisoned_outputs)."""
    if poison:
        with poisoned_outputs():
            return forward(inp, want_teacher, fused, attn_kl, topk_sel)
    wl = inp.wl
    L = layout_of_inputs(inp)
    sel = row_lse = scores = None
    if fused:
        if not wl.sparse_loss:
            raise RuntimeError("the fused score + top-k path serves the sparse loss")
        ids, sel, row_lse = csa_indexer_topk(L, inp.q_idx, inp.k_idx, inp.weights, inp.idx_scale, wl.topk,
                                             want_lse=True)
    else:
        scores = csa_indexer_score(L, inp.q_idx, inp.k_idx, inp.weights, inp.idx_scale)
        if topk_sel and wl.sparse_loss:
            sel = _new((wl.total_q, k_eff(L, wl.topk)), torch.float32, scores.device)
        ids = csa_topk(L, scores, wl.topk, sel_scores=sel)
    selected = sel is not None
    if attn_kl:
        if not wl.sparse_loss:
            raise RuntimeError("the attention + teacher/KL call serves the sparse loss")
        out, lse, lse_nc, cmass, teacher, kl_row, loss = csa_sparse_attn_kl_fwd(
            L, inp.q, inp.kv, inp.ckv, inp.sink, ids, wl.window, inp.scale, sel if selected else scores,
            scores_selected=selected, want_teacher=want_teacher)
        return dict(scores=scores, ids=ids, out=out, lse=lse, lse_nc=lse_nc, cmass=cmass,
                    teacher=teacher, kl_row=kl_row, loss=loss, sel=sel, row_lse=row_lse)
    out, lse, lse_nc, cmass = csa_sparse_attn_fwd(L, inp.q, inp.kv, inp.ckv, inp.sink, ids, wl.window,
                                                  inp.scale, want_cmass=wl.sparse_loss)
    teacher, kl_row, loss = csa_indexer_teacher_kl(L, wl.sparse_loss, sel if selected else scores, ids, cmass,
                                                   inp.q, inp.ckv, lse_nc, inp.scale, want_teacher=want_teacher,
                                                   scores_selected=selected)
    return dict(scores=scores, ids=ids, out=out, lse=lse, lse_nc=lse_nc, cmass=cmass,
                teacher=teacher, kl_row=kl_row, loss=loss, sel=sel, row_lse=row_lse)


class Prepared:
    """The four calls of one forward step with every ctypes argument built once.

    Marshalling only: the same C entry points with the same arguments as the functions
    above, but the pointers, strides, layout struct and stream handle are converted a
    single time, so a host loop can enqueue steps far faster than the GPU runs them.
    The tensors given here must stay alive and in place while the object is used.
    """

    def __init__(self, layout: Layout, inp, scores, ids, out, lse, lse_nc, cmass, kl_row, loss,
                 sparse_loss: bool, topk: int, window: int, teacher=None, sel=None):
        lib = load()
        self._lib = lib
        self._L = layout.c()
        Lp = ctypes.byref(self._L)
        st = _stream()
        T, Hi, Di = inp.q_idx.shape
        _, H, D = inp.q.shape
        k_eff_ = ids.shape[1]
        self._keep = (inp, scores, ids, out, lse, lse_nc, cmass, kl_row, loss, teacher, sel)
        if scores is not None:
            self.args_score = (Lp, _ptr(inp.q_idx), _ptr(inp.k_idx), _ptr(inp.weights), _dtype(inp.q_idx),
                               Hi, Di, ctypes.c_float(inp.idx_scale), _ptr(scores),
                               ctypes.c_int64(scores.stride(0)), st)
            # with sel, the top-k call also writes the selected scores
            self.args_topk = (Lp, _ptr(scores), ctypes.c_int64(scores.stride(0)), int(topk), _ptr(ids),
                              _ptr(sel) if sel is not None else None, st)
        if sel is not None:   # the teacher/KL reads the selected scores (fused call or top-k's)
            self.args_fused = (Lp, _ptr(inp.q_idx), _ptr(inp.k_idx), _ptr(inp.weights), _dtype(inp.q_idx),
                               Hi, Di, ctypes.c_float(inp.idx_scale), int(topk), _ptr(ids), _ptr(sel), None, st)
        tkl_scores = sel if sel is not None else scores
        self.args_attn = (Lp, _ptr(inp.q), _ptr(inp.kv), _ptr(inp.ckv), _ptr(inp.sink), _ptr(ids), k_eff_,
                          int(window), _dtype(inp.q), H, D, ctypes.c_float(inp.scale), _ptr(out), _ptr(lse),
                          _ptr(lse_nc), _ptr(cmass) if cmass is not None else None, st)
        self.args_tkl = (Lp, 1 if sparse_loss else 0, _ptr(tkl_scores), ctypes.c_int64(tkl_scores.stride(0)),
                         1 if sel is not None else 0, _ptr(ids), k_eff_, _ptr(cmass) if cmass is not None else None, _ptr(inp.q),
                         _ptr(inp.ckv), _ptr(lse_nc), _dtype(inp.q), H, D, ctypes.c_float(inp.scale), 0,
                         _ptr(teacher) if teacher is not None else None,
                         ctypes.c_int64(teacher.stride(0) if teacher is not None else 0),
                         _ptr(kl_row), _ptr(loss), st)
        if sparse_loss and cmass is not None:
            self.args_attn_kl = (Lp, _ptr(inp.q), _ptr(inp.kv), _ptr(inp.ckv), _ptr(inp.sink), _ptr(ids), k_eff_,
                                 int(window), _dtype(inp.q), H, D, ctypes.c_float(inp.scale), _ptr(tkl_scores),
                                 ctypes.c_int64(tkl_scores.stride(0)), 1 if sel is not None else 0, 0,
                                 _ptr(out), _ptr(lse), _ptr(lse_nc), _ptr(cmass),
                                 _ptr(teacher) if teacher is not None else None,
                                 ctypes.c_int64(teacher.stride(0) if teacher is not None else 0),
                                 _ptr(kl_row), None, st)
            self.args_loss = (_ptr(kl_row), T, 0, _ptr(loss), st)

    def csa_sparse_attn_kl_fwd(self):
        """attention + teacher + KL (kl_row only; csa_loss_reduce then gives the loss)"""
        _check(self._lib.csa_sparse_attn_kl_fwd(*self.args_attn_kl))

    def csa_loss_reduce(self):
        _check(self._lib.csa_loss_reduce(*self.args_loss))

    def csa_indexer_score(self):
        _check(self._lib.csa_indexer_score(*self.args_score))

    def csa_topk(self):
        _check(self._lib.csa_topk(*self.args_topk))

    def csa_indexer_topk(self):
        _check(self._lib.csa_indexer_topk(*self.args_fused))

    def csa_sparse_attn_fwd(self):
        _check(self._lib.csa_sparse_attn_fwd(*self.args_attn))

    def csa_indexer_teacher_kl(self):
        _check(self._lib.csa_indexer_teacher_kl(*self.args_tkl))
