"""Seeded synthetic inputs for the CSA forward path.

This module holds the workload definitions and the random draws only -- no step of the
method's arithmetic -- so that the HIP path and the CPU oracle can be fed identical
values without sharing any computation.  It depends on torch alone.

Workloads (shapes and distributions of the five CSA forward configurations):
  tiny-fp32   b=1, S=256, ratio 4, H=4 x D=64, Hi=4 x Di=32, topk 16, window 32, fp32
  bshd-b2     b=2, S=4096, ratio 4, H=16 x D=128, Hi=16 x Di=64, topk 256, window 128
  thd-varlen  documents 1024/2048/3072/4096/6144, ratio 4, H=64 x D=192, Hi=32 x Di=64,
              topk 512, window 128
  long-64k    b=1, S=65536, ratio 4, H=128 x D=512, Hi=64 x Di=128, topk 2048, window 128
  dense-32k   b=1, S=32768, ratio 16, H=64 x D=128, Hi=32 x Di=64, topk 1024, window 256,
              dense loss, sink ~ N(0, 4), original KV rows scaled by 2
Draws (in this order, fp32, then cast): q, kv, ckv, q_idx, k_idx ~ N(0,1)/sqrt(D);
weights ~ U(0,1); sink ~ N(0, sink_var).  seed = 20260000 + workload index.

The "exact" family replaces q_idx, k_idx by integers in [-3, 3], the weights by m/16
(m in 0..15) and the indexer scale by 1/8: every indexer score is then an integer
multiple of 2^-7 below 2^24 * 2^-7, so it is exact in fp32 in any summation order.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

SEED_BASE = 20260000
_CHUNK_ROWS = 4096  # rows per draw for the big tensors (fixes the stream layout)


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    seg_lens: tuple
    ratio: int
    H: int
    D: int
    Hi: int
    Di: int
    topk: int
    window: int
    sparse_loss: bool
    dtype: str               # "f32" or "bf16" for q, kv, ckv, q_idx, k_idx
    sink_var: float = 1.0
    kv_scale: float = 1.0

    @property
    def total_q(self) -> int:
        return int(sum(self.seg_lens))

    @property
    def total_k(self) -> int:
        return int(sum(s // self.ratio for s in self.seg_lens))

    @property
    def max_seqlen_q(self) -> int:
        return int(max(self.seg_lens))

    @property
    def max_seqlen_k(self) -> int:
        return int(max(s // self.ratio for s in self.seg_lens))

    @property
    def k_eff(self) -> int:
        return min(self.topk, self.max_seqlen_k)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def idx_scale(self) -> float:
        return 1.0 / math.sqrt(self.Di)

    def describe(self) -> dict:
        return dict(workload=self.name, segments=list(self.seg_lens), compress_ratio=self.ratio,
                    heads=self.H, head_dim=self.D, indexer_heads=self.Hi, indexer_dim=self.Di,
                    topk=self.topk, window=self.window,
                    loss="sparse" if self.sparse_loss else "dense", total_q=self.total_q,
                    total_k=self.total_k)


WORKLOADS = [
    Workload(0, "tiny-fp32", (256,), 4, 4, 64, 4, 32, 16, 32, True, "f32"),
    Workload(1, "bshd-b2-s4096", (4096, 4096), 4, 16, 128, 16, 64, 256, 128, True, "bf16"),
    Workload(2, "thd-varlen-16k", (1024, 2048, 3072, 4096, 6144), 4, 64, 192, 32, 64, 512, 128, True, "bf16"),
    Workload(3, "long-64k", (65536,), 4, 128, 512, 64, 128, 2048, 128, True, "bf16"),
    Workload(4, "dense-32k", (32768,), 16, 64, 128, 32, 64, 1024, 256, False, "bf16", 4.0, 2.0),
]


def scaled_down(w: Workload, seg_lens, name=None, **kw) -> Workload:
    """Same head shapes and distributions with other segment lengths (for small cases)."""
    d = dict(w.__dict__)
    d.update(seg_lens=tuple(seg_lens), name=name or f"{w.name}-small", **kw)
    return Workload(**d)


@dataclass
class Inputs:
    wl: Workload
    cu_q: torch.Tensor      # int32 [B+1]
    cu_k: torch.Tensor      # int32 [B+1]
    offsets: torch.Tensor   # int32 [B]
    q: torch.Tensor         # [T, H, D]
    kv: torch.Tensor        # [T, D]
    ckv: torch.Tensor       # [T_k, D]
    q_idx: torch.Tensor     # [T, Hi, Di]
    k_idx: torch.Tensor     # [T_k, Di]
    weights: torch.Tensor   # fp32 [T, Hi]
    sink: torch.Tensor      # fp32 [H]
    idx_scale: float
    scale: float
    family: str = "gauss"
    extra: dict = field(default_factory=dict)
    cu_q_real: torch.Tensor | None = None   # int32 [B+1] real boundaries of a padded batch


def _randn(gen, shape, device, std, dtype):
    """Draw N(0, std^2) in fp32 in row chunks of the leading axis, then cast."""
    out = torch.empty(shape, dtype=dtype, device=device)
    for r0 in range(0, shape[0], _CHUNK_ROWS):
        r1 = min(shape[0], r0 + _CHUNK_ROWS)
        x = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=gen, device=device, dtype=torch.float32)
        out[r0:r1] = (x * std).to(dtype)
    return out


def _randint(gen, shape, lo, hi, device, dtype):
    out = torch.empty(shape, dtype=dtype, device=device)
    for r0 in range(0, shape[0], _CHUNK_ROWS):
        r1 = min(shape[0], r0 + _CHUNK_ROWS)
        x = torch.randint(lo, hi, (r1 - r0,) + tuple(shape[1:]), generator=gen, device=device)
        out[r0:r1] = x.to(dtype)
    return out


def layout_tensors(wl: Workload, device):
    """cu_q, cu_k (compressed lengths seg_len // ratio) and per-segment offsets.
    Every workload's segment lengths are multiples of the ratio, so the bottom-right
    offsets are all 0; they are passed explicitly."""
    seg = list(wl.seg_lens)
    cu_q = [0]
    cu_k = [0]
    for s in seg:
        cu_q.append(cu_q[-1] + s)
        cu_k.append(cu_k[-1] + s // wl.ratio)
    mk = lambda v: torch.tensor(v, dtype=torch.int32, device=device)
    return mk(cu_q), mk(cu_k), mk([0] * len(seg))


def make_inputs(wl: Workload, device="cpu", family="gauss", seed=None) -> Inputs:
    seed = SEED_BASE + wl.index if seed is None else seed
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    dt = wl.torch_dtype
    T, Tk = wl.total_q, wl.total_k
    sd = 1.0 / math.sqrt(wl.D)
    cu_q, cu_k, off = layout_tensors(wl, device)
    q = _randn(gen, (T, wl.H, wl.D), device, sd, dt)
    kv = _randn(gen, (T, wl.D), device, sd * wl.kv_scale, dt)
    ckv = _randn(gen, (Tk, wl.D), device, sd, dt)
    if family == "gauss":
        q_idx = _randn(gen, (T, wl.Hi, wl.Di), device, sd, dt)
        k_idx = _randn(gen, (Tk, wl.Di), device, sd, dt)
        weights = torch.rand((T, wl.Hi), generator=gen, device=device, dtype=torch.float32)
        idx_scale = wl.idx_scale
    elif family == "exact":
        q_idx = _randint(gen, (T, wl.Hi, wl.Di), -3, 4, device, dt)
        k_idx = _randint(gen, (Tk, wl.Di), -3, 4, device, dt)
        weights = _randint(gen, (T, wl.Hi), 0, 16, device, torch.float32) / 16.0
        idx_scale = 0.125
    else:
        raise ValueError(family)
    sink = torch.randn((wl.H,), generator=gen, device=device, dtype=torch.float32) * math.sqrt(wl.sink_var)
    return Inputs(wl, cu_q, cu_k, off, q, kv, ckv, q_idx, k_idx, weights, sink,
                  float(idx_scale), float(wl.scale), family)


def sample_rows(wl: Workload, n: int, seed: int = 7) -> list:
    """A seeded row sample that always holds the first ratio+1 rows and the last row of
    every segment, topped up with uniform rows (sorted, unique)."""
    rows = set()
    start = 0
    for s in wl.seg_lens:
        rows.update(range(start, min(start + wl.ratio + 1, start + s)))
        rows.add(start + s - 1)
        start += s
    g = torch.Generator()
    g.manual_seed(seed)
    extra = torch.randperm(wl.total_q, generator=g).tolist()
    for t in extra:
        if len(rows) >= n:
            break
        rows.add(int(t))
    return sorted(rows)


def uniform_rows(total: int, n: int, seed: int = 11) -> list:
    """A seeded uniform sample of n distinct rows (for timing the oracle)."""
    g = torch.Generator()
    g.manual_seed(seed)
    perm = torch.randperm(total, generator=g)[: min(n, total)]
    return sorted(perm.tolist())


def pad_inputs(inp: Inputs, n_pad: int, dummy: bool = False, seed: int = 4242) -> Inputs:
    """The same batch padded to a static shape with n_pad padding rows: appended to the
    last segment (dummy=False) or as a trailing dummy segment of real length 0.  The real
    rows and keys are the input's own; padding rows (and the compressed keys the padded
    segment gains) are fresh draws from the same distributions.  cu_q_real keeps the
    real boundaries."""
    wl = inp.wl
    segs = list(wl.seg_lens)
    if dummy:
        segs.append(int(n_pad))
    else:
        segs[-1] += int(n_pad)
    pw = scaled_down(wl, segs, name=f"{wl.name}-pad{n_pad}{'-dummy' if dummy else ''}")
    dev = inp.q.device
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    dt = wl.torch_dtype
    sd = 1.0 / math.sqrt(wl.D)
    extra_k = pw.total_k - wl.total_k
    q = torch.cat([inp.q, _randn(gen, (n_pad, wl.H, wl.D), dev, sd, dt)])
    kv = torch.cat([inp.kv, _randn(gen, (n_pad, wl.D), dev, sd * wl.kv_scale, dt)])
    ckv = torch.cat([inp.ckv, _randn(gen, (extra_k, wl.D), dev, sd, dt)])
    q_idx = torch.cat([inp.q_idx, _randn(gen, (n_pad, wl.Hi, wl.Di), dev, sd, dt)])
    k_idx = torch.cat([inp.k_idx, _randn(gen, (extra_k, wl.Di), dev, sd, dt)])
    weights = torch.cat([inp.weights, torch.rand((n_pad, wl.Hi), generator=gen, device=dev,
                                                 dtype=torch.float32)])
    cu_q, cu_k, off = layout_tensors(pw, dev)
    real = inp.cu_q.tolist() + ([inp.cu_q[-1].item()] if dummy else [])
    cu_real = torch.tensor(real, dtype=torch.int32, device=dev)
    return Inputs(pw, cu_q, cu_k, off, q, kv, ckv, q_idx, k_idx, weights, inp.sink,
                  inp.idx_scale, inp.scale, inp.family, cu_q_real=cu_real)
