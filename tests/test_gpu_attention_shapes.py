"""GPU parity of csa_sparse_attn_fwd on every attention kernel route (through the C ABI).

The workloads exercise one head shape each; this file covers the shapes in between, so
that every kernel the launcher can pick is checked against the oracle's attention_row:
  persistent gather kernel   bf16, H <= 16, D in {64, 128}, 1 <= k_eff <= 256, window > 0
  gather kernel              bf16, H <= 16, D in {64, 128}, 1 <= k_eff <= 256, window = 0
  workgroup kernel           other bf16 shapes with D in {64, 128, 192, 256}: H up to
                             128 (not a multiple of 16 too), k_eff up to 4096
  wide workgroup kernel      bf16, D = 512, any H up to 128 (P.V split over the output
                             columns, P shared through LDS)
  register-staged kernel     fp32 inputs
The ids are drawn directly (ascending distinct visible keys of the row's segment with
random -1 holes, -1 padding past the visible count), so the selection is not involved;
k_eff is not a multiple of 32 in most cases.  Tolerances as in tests/gpu_check.py: out
2e-2 absolute and within the rounding bound beta * sum_r P_hr |V_rd| (bf16 or fp32),
lse / lse_nc / cmass 1e-5 relative.  The outputs start as NaN, so an element a kernel
leaves unwritten fails.
"""
import zlib
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import oracle
from tests import gpu_check as C
from tests.oracle_bridge import host

pytestmark = pytest.mark.gpu

# (name, dtype, H, D, k_eff, window, segment lengths)
CASES = [
    ("pipe-h16-d128", torch.bfloat16, 16, 128, 200, 48, (300, 900)),
    ("pipe-h5-d64", torch.bfloat16, 5, 64, 33, 7, (97, 400)),
    ("dma-h16-d128-nowin", torch.bfloat16, 16, 128, 256, 0, (300, 1100)),
    ("wg-h16-d128-k600", torch.bfloat16, 16, 128, 600, 64, (300, 2600)),
    ("wg-h20-d64", torch.bfloat16, 20, 64, 300, 40, (150, 1300)),
    ("wg-h40-d192", torch.bfloat16, 40, 192, 77, 33, (97, 500)),
    ("wg-h64-d256-nowin", torch.bfloat16, 64, 256, 520, 0, (64, 2200)),
    ("wide-h128-d512", torch.bfloat16, 128, 512, 130, 64, (200, 700)),
    ("wide-h128-d512-k600", torch.bfloat16, 128, 512, 600, 64, (300, 2600)),
    ("wide-h112-d512", torch.bfloat16, 112, 512, 300, 130, (150, 1300)),
    ("wide-h40-d512-nowin", torch.bfloat16, 40, 512, 77, 0, (97, 500)),
    ("wide-h8-d512-k1", torch.bfloat16, 8, 512, 1, 1, (40, 90)),
    # 125 compressed chunks: key masks of chunks 64 and up, and the three-tile ring (four
    # 32 KiB tiles no longer fit the LDS beside 4,000 staged ids)
    ("wide-h16-d512-k4000", torch.bfloat16, 16, 512, 4000, 64, (16400,)),
    ("wg-h33-d128-k1", torch.bfloat16, 33, 128, 1, 1, (40, 90)),
    ("f32-h4-d64", torch.float32, 4, 64, 16, 32, (100, 256)),
    ("f32-h20-d128", torch.float32, 20, 128, 300, 40, (150, 1300)),
]
RATIO = 4


def _ops():
    from deepseek_v4_csa_amd import ops
    ops.load()
    return ops


def _draw_ids(Lo, T, k_eff, rng):
    ids = np.full((T, k_eff), -1, dtype=np.int32)
    for t in range(T):
        g = oracle.row_geometry(Lo, t)
        n = min(k_eff, g.n_valid)
        if n == 0:
            continue
        pick = np.sort(rng.choice(g.n_valid, size=n, replace=False)) + g.k_base
        holes = rng.random(n) < 0.1
        pick[holes] = -1
        ids[t, :n] = pick
    return ids


def _rows_to_check(cu_q, rng, per_seg=16):
    rows = set()
    for s in range(len(cu_q) - 1):
        a, b = int(cu_q[s]), int(cu_q[s + 1])
        rows.update(range(a, min(b, a + 6)))
        rows.update(range(max(a, b - 6), b))
        if b - a > 12:
            rows.update(int(x) for x in rng.choice(np.arange(a, b), size=min(per_seg, b - a), replace=False))
    return sorted(rows)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_attention_route_against_oracle(gpu_ok, case):
    name, dt, H, D, k_eff, window, seg_q = case
    ops = _ops()
    seg_k = [s // RATIO for s in seg_q]
    T, Tk = sum(seg_q), sum(seg_k)
    L = ops.Layout.from_lengths(list(seg_q), seg_k, RATIO)
    cu_q = L.cu_q.cpu().numpy()
    Lo = oracle.Layout(cu_q=cu_q, cu_k=L.cu_k.cpu().numpy(), ratio=RATIO, off=None)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(int(rng.integers(1 << 30)))
    rnd = lambda *s: (torch.randn(*s, generator=gen, device="cuda") / D ** 0.5).to(dt)
    q, kv, ckv = rnd(T, H, D), rnd(T, D), rnd(Tk, D)
    sink = torch.randn(H, generator=gen, device="cuda")
    ids_h = _draw_ids(Lo, T, k_eff, rng)
    ids = torch.from_numpy(ids_h).cuda()
    scale = D ** -0.5
    with ops.poisoned_outputs():
        out, lse, lse_nc, cm = ops.csa_sparse_attn_fwd(L, q, kv, ckv, sink, ids, window, scale)
    torch.cuda.synchronize()
    q_h, kv_h, ckv_h, sink_h = host(q), host(kv), host(ckv), host(sink)
    g_out, g_lse, g_lnc, g_cm = host(out), host(lse), host(lse_nc), host(cm)
    worst = {}
    Pv = SimpleNamespace(kv=kv_h, ckv=ckv_h, window=window)
    for t in _rows_to_check(cu_q, rng):
        g = oracle.row_geometry(Lo, t)
        A = oracle.attention_row(q_h[t], kv_h, ckv_h, sink_h, ids_h[t], oracle.window_rows(t, g.q_start, window),
                                 scale)
        err = np.abs(g_out[t] - A.out)
        e = float(err.max())
        assert e <= C.TOL_OUT, (name, t, "out", e)
        scl, nrow = C.value_scale(Pv, t, g, A, ids_h[t])
        bnd = C.out_bound(scl, nrow, dt == torch.float32)
        assert np.all(err <= bnd), (name, t, "out above its rounding bound", float(np.max(err / bnd)))
        worst["out"] = max(worst.get("out", 0.0), e)
        worst["out_over_bound"] = max(worst.get("out_over_bound", 0.0), float(np.max(err / bnd)))
        for nm, gv, ov in (("lse", g_lse[t], A.lse), ("lse_nc", g_lnc[t], A.lse_nc)):
            fin = np.isfinite(ov)
            assert np.array_equal(np.isfinite(gv), fin), (name, t, nm)
            err = np.abs(gv[fin] - ov[fin])
            assert np.all(err <= C.REL * np.abs(ov[fin]) + 1e-6), (name, t, nm, err.max())
        err = np.abs(g_cm[t] - A.cmass)
        assert np.all(err <= C.REL * np.abs(A.cmass) + 1e-9), (name, t, "cmass", err.max())
        assert np.all(g_cm[t][ids_h[t] < 0] == 0), (name, t, "cmass at -1 slots")
    # every row's outputs are written (NaN-filled before the call)
    assert bool(torch.isfinite(lse).all() and torch.isfinite(lse_nc).all() and torch.isfinite(cm).all())
    assert bool(torch.isfinite(out.float()).all())
    print(name, {k: float(v) for k, v in worst.items()}, flush=True)
    C.record(f"attn-{name}", worst)
