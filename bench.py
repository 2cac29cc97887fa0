"""Throughput of the CSA forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload bshd-b2-s4096]

One step = the four calls of the path (indexer scores, top-k, window+top-k sparse
attention with sink and teacher masses, teacher + KL + loss) over one batch of seeded
synthetic inputs already resident in HBM.  Prints one JSON line: query tokens/s over K
timed steps, the roofline of the dominant kernel (HIP events on the launch stream,
around every launch inside the timed region) and the CPU oracle timed on a bounded
row sample of the same workload (cpu_baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
FP32_MFMA_PEAK_TFLOPS = 157.3


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="bshd-b2-s4096")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def geometry(wl):
    """Host-side per-row counts for the algorithmic work model (n_valid, K_t, window)."""
    import numpy as np
    n_valid, kt, nwin = [], [], []
    for L in wl.seg_lens:
        s_k = L // wl.ratio
        r = np.arange(L)
        nv = np.minimum((r + 1) // wl.ratio, s_k)
        n_valid.append(nv)
        kt.append(np.minimum(nv, wl.k_eff))
        nwin.append(np.minimum(r + 1, wl.window))
    cat = lambda x: np.concatenate(x).astype(np.int64)
    return cat(n_valid), cat(kt), cat(nwin)


def work_model(wl):
    nv, kt, nw = geometry(wl)
    eb = 4 if wl.dtype == "f32" else 2
    T, H, D = wl.total_q, wl.H, wl.D
    P = int(nv.sum())
    G = int(kt.sum() + nw.sum())
    return {
        "indexer_flop": 2 * wl.Hi * wl.Di * P,
        "topk_bytes": 4 * P + 4 * T * wl.k_eff,
        "attn_bytes": G * D * eb + 2 * T * H * D * eb + 8 * T * H + 8 * T * wl.k_eff,
        "attn_flop": 4 * H * D * G,
        "teacher_bytes": (12 * T * wl.k_eff + 4 * T) if wl.sparse_loss else (4 * P + 4 * T * H + 4 * T),
        "gathered_rows": G,
        "causal_pairs": P,
    }


def traffic_of(wl_name, kernel):
    """HBM bytes per launch of ``kernel`` from the committed counter table of the
    workload (FETCH_SIZE / WRITE_SIZE scaled by a copy of known size), if it was taken
    on the current source of the kernel; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"csa_path_{wl_name}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path)).get("kernels", {}).get(kernel)
    if not d:
        return None
    sha = hashlib.sha256(open(os.path.join(ROOT, d["source"]), "rb").read()).hexdigest()
    if d.get("source_sha256") != sha:
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(inp, seconds):
    """The CPU oracle (as it stands) on a seeded uniform sample of rows of the workload."""
    import numpy as np
    import torch
    import oracle
    from deepseek_v4_csa_amd.inputs import uniform_rows
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    wl = inp.wl
    h = lambda x: x.detach().to("cpu", torch.float64).numpy()
    L = oracle.Layout(cu_q=inp.cu_q.cpu().numpy(), cu_k=inp.cu_k.cpu().numpy(), ratio=wl.ratio,
                      off=inp.offsets.cpu().numpy())
    P = oracle.Problem(layout=L, q=h(inp.q), kv=h(inp.kv), ckv=h(inp.ckv), q_idx=h(inp.q_idx),
                       k_idx=h(inp.k_idx), weights=h(inp.weights), sink=h(inp.sink), topk=wl.topk,
                       window=wl.window, scale=inp.scale, idx_scale=inp.idx_scale,
                       sparse_loss=wl.sparse_loss)
    order = uniform_rows(wl.total_q, wl.total_q, seed=11)
    rng = np.random.default_rng(11)
    rng.shuffle(order)
    t0 = time.perf_counter()
    done = 0
    for t in order:
        oracle.run_row(P, int(t))
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "query tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} uniformly drawn rows of {wl.total_q} ({wl.name}), every step of the path "
                      f"per row in NumPy float64, {el:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import torch
    from deepseek_v4_csa_amd import inputs as I
    from deepseek_v4_csa_amd import ops

    ops.load()
    wl = next(w for w in I.WORKLOADS if w.name == args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = I.make_inputs(wl, device="cuda")
    L = ops.layout_of_inputs(inp)
    T = wl.total_q
    k_eff = ops.k_eff(L, wl.topk)
    scores = torch.empty((T, wl.max_seqlen_k), dtype=torch.float32, device=dev)
    ids = torch.empty((T, k_eff), dtype=torch.int32, device=dev)
    out = torch.empty_like(inp.q)
    lse = torch.empty((T, wl.H), dtype=torch.float32, device=dev)
    lse_nc = torch.empty_like(lse)
    cmass = torch.empty((T, k_eff), dtype=torch.float32, device=dev) if wl.sparse_loss else None
    kl_row = torch.empty((T,), dtype=torch.float32, device=dev)
    loss = torch.empty((1,), dtype=torch.float32, device=dev)

    names = ("indexer_score", "topk", "sparse_attn", "teacher_kl")
    # every ctypes argument is marshalled once, so the host enqueues far ahead of the GPU
    P = ops.Prepared(L, inp, scores, ids, out, lse, lse_nc, cmass, kl_row, loss,
                     wl.sparse_loss, wl.topk, wl.window)

    def step(ev=None):
        P.csa_indexer_score()
        P.csa_topk()
        if ev: ev[0].record()
        P.csa_sparse_attn_fwd()
        if ev: ev[1].record()
        P.csa_indexer_teacher_kl()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: K whole steps; HIP events (on the launch stream) bracket only the
    # attention launch, whose duration gives the roofline figure
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    att_ms = sum(ev[0].elapsed_time(ev[1]) for ev in events) / args.steps

    # per-call breakdown from a separate, untimed pass with events between all calls
    nb = min(args.steps, 50)
    bev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(nb)]
    calls = (P.csa_indexer_score, P.csa_topk, P.csa_sparse_attn_fwd, P.csa_indexer_teacher_kl)
    for ev in bev:
        ev[0].record()
        for i, f in enumerate(calls):
            f()
            ev[i + 1].record()
    torch.cuda.synchronize()
    per_kernel_ms = {n: sum(ev[i].elapsed_time(ev[i + 1]) for ev in bev) / nb for i, n in enumerate(names)}
    value = T * args.steps / elapsed
    wm = work_model(wl)

    roof = {"kernel": "sparse_attn", "bound": "hbm",
            "achieved": wm["attn_bytes"] / (att_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "traffic": traffic_of(wl.name, "sparse_attn")}
    roof["frac"] = roof["achieved"] / roof["peak"]
    idx_peak = FP32_MFMA_PEAK_TFLOPS if wl.dtype == "f32" else BF16_MFMA_PEAK_TFLOPS
    kernels = {
        "indexer_score": {"us": per_kernel_ms["indexer_score"] * 1e3,
                          "tflops": wm["indexer_flop"] / (per_kernel_ms["indexer_score"] * 1e-3) / 1e12,
                          "frac_mfma_peak": wm["indexer_flop"] / (per_kernel_ms["indexer_score"] * 1e-3) / 1e12 / idx_peak},
        "topk": {"us": per_kernel_ms["topk"] * 1e3,
                 "gbs": wm["topk_bytes"] / (per_kernel_ms["topk"] * 1e-3) / 1e9},
        "sparse_attn": {"us": att_ms * 1e3, "gbs_gather_model": roof["achieved"],
                        "tflops": wm["attn_flop"] / (att_ms * 1e-3) / 1e12},
        "teacher_kl": {"us": per_kernel_ms["teacher_kl"] * 1e3,
                       "gbs": wm["teacher_bytes"] / (per_kernel_ms["teacher_kl"] * 1e-3) / 1e9},
    }
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args.cpu_seconds)
    line = {
        "metric": "query tokens/s for indexer+topk+CSA attn+teacher/KL; % MFMA / HBM peak",
        "value": value, "unit": "query tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": elapsed / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32" if wl.dtype == "f32" else "bf16",
        "data": "synthetic",
        "config": {**wl.describe(), "parallelism": "none (1 GPU)"},
        "roofline": roof, "cpu_baseline": cpu, "kernels": kernels,
        "loss": float(loss[0]),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
