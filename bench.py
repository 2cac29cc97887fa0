"""Throughput of the CSA forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long-64k]
                    [--row path|backward|cp-share]

One step = the four calls of the path (indexer scores, top-k, window+top-k sparse
attention with sink and teacher masses, teacher + KL + loss) over one batch of seeded
synthetic inputs already resident in HBM.  The default workload is the largest one that
fits one GPU: one 65,536-token sequence, 128 heads over a shared 512-wide latent KV, 64
indexer heads x 128, top-2048 of 16,384 compressed keys, window 128.  Prints one JSON
line: query tokens/s over K timed steps, the roofline of the dominant kernel (HIP events
on the launch stream, around the attention launch inside the timed region) and the CPU
oracle timed on a bounded row sample of the same workload (cpu_baseline).

The steps after the path are measured the same way, one JSON line each:
  --row backward   one step = csa_indexer_loss_bwd (score gradients, dq_idx/dweights,
                   dk_idx) after one forward, on the same workload;
  --row cp-share   one step = csa_indexer_score + csa_topk on one rank's share of
                   context-parallel scoring (csa_cp_plan): the 65,536-token sequence at
                   CP = 8, rank 0 (chunks 0 and 15, 8,192 rows, key prefixes cropped at
                   the chunk ends).

Measurement tools (the profiles' summaries are made with these):
  python bench.py copy-probe
        a plain 1 GiB device copy, three times: profiled beside the path, it calibrates
        the FETCH_SIZE / WRITE_SIZE counters (a copy's bytes are known exactly);
  python bench.py prof-summary stats <stats_dir> <out.txt> --cmd "<command>"
  python bench.py prof-summary traffic <workload> <fetch_dir> <write_dir> \
        <copy_fetch_dir> <copy_write_dir> <out_prefix> --cmd "<command>"
  python bench.py prof-summary counters <workload> <counter_dir> <out.txt> --cmd "<command>"
        rocprofv3 CSV output (run_kernel_stats.csv of --kernel-trace --stats;
        run_counter_collection.csv of one --pmc FETCH_SIZE or WRITE_SIZE pass) turned
        into the short summaries of profiles/ and the per-kernel HBM traffic table that
        the JSON line's roofline.traffic reads; a --pmc pass of the SQ counters into the
        per-kernel LDS bank-conflict ratio and MFMA busy fraction.
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
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long-64k")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--row", default="path", choices=("path", "backward", "cp-share"))
    ap.add_argument("--unfused", action="store_true",
                    help="path: score and top-k as two calls (the score matrix stored) even where "
                         "the fused call applies")
    ap.add_argument("--one-call-attn", action="store_true",
                    help="path: the one-call attention + teacher/KL kernel (csa_sparse_attn_kl_fwd, then "
                         "csa_loss_reduce) where it applies, instead of csa_sparse_attn_fwd + "
                         "csa_indexer_teacher_kl (the default: on bshd-b2-s4096 the two calls' kernels "
                         "take 82 us against 88 us, since the fp64 predictor and log-ratios of the KL "
                         "cost the one-wave-per-query kernel more than the teacher kernel)")
    ap.add_argument("--cp", type=int, default=8, help="cp-share: CP size")
    ap.add_argument("--rank", type=int, default=0, help="cp-share: rank")
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
    """HBM bytes per call of ``kernel`` (every kernel the call launches) from the committed
    counter table of the workload (FETCH_SIZE / WRITE_SIZE scaled by a copy of known size),
    if it was taken on the current sources of those kernels; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"csa_path_{wl_name}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path)).get("kernels", {}).get(kernel)
    if not d or not d.get("sources"):
        return None
    for src, want in d["sources"].items():
        if hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest() != want:
            return None
    return d.get("hbm_bytes_per_launch")


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(inp, seconds):
    """The CPU oracle (as it stands) on a seeded uniform sample of rows of the workload.
    Only the sampled rows of the per-row tensors (q, q_idx, weights) are copied to the
    host; the key/value tensors are copied whole.  Uniform rows carry the average work of
    a row, so rows/s is the oracle's query tokens/s on the whole workload."""
    import numpy as np
    import oracle
    from deepseek_v4_csa_amd.inputs import uniform_rows
    wl = inp.wl
    # enough rows for the time target on every workload, at most ~1.6 GB of fp64 q rows
    # on the host (long-64k: 3,051 rows of 512 KiB)
    n = min(wl.total_q, 4096, max(256, int(1.6e9 / (wl.H * wl.D * 8))))
    order = uniform_rows(wl.total_q, n, seed=11)
    P = _oracle_problem(inp, order)
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
    return {"value": done / el, "unit": "query tokens/s", "cores": int(_threads()), "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"{done} uniformly drawn rows of {wl.total_q} ({wl.name}), every step of the path "
                      f"per row in NumPy float64, {el:.1f} s"}


def _threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def _oracle_problem(inp, rows=None):
    """oracle.Problem over host copies of the inputs (only `rows` of the per-row tensors
    when given, as a dict-backed row map)."""
    import numpy as np
    import torch
    import oracle
    wl = inp.wl
    h = lambda x: x.detach().to("cpu", torch.float64).numpy()

    class Rows:
        def __init__(self, full):
            idx = torch.tensor(sorted(rows), device=full.device)
            self.pos = {r: i for i, r in enumerate(sorted(rows))}
            self.v = h(full.index_select(0, idx))

        def __getitem__(self, t):
            return self.v[self.pos[int(t)]]

    pr = (lambda x: h(x)) if rows is None else Rows
    L = oracle.Layout(cu_q=inp.cu_q.cpu().numpy(), cu_k=inp.cu_k.cpu().numpy(), ratio=wl.ratio,
                      off=inp.offsets.cpu().numpy())
    return oracle.Problem(layout=L, q=pr(inp.q), kv=h(inp.kv), ckv=h(inp.ckv), q_idx=pr(inp.q_idx),
                          k_idx=h(inp.k_idx), weights=pr(inp.weights), sink=h(inp.sink), topk=wl.topk,
                          window=wl.window, scale=inp.scale, idx_scale=inp.idx_scale,
                          sparse_loss=wl.sparse_loss)


def _line(metric, value, args, ms, dtype, config, roof, cpu, extra):
    d = {"metric": metric, "value": value, "unit": "query tokens/s", "n_gpus": 1, "steps": args.steps,
         "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
         "vs_baseline": None, "dtype": dtype, "data": "synthetic", "config": config,
         "roofline": roof, "cpu_baseline": cpu}
    d.update(extra)
    print(json.dumps(d))


def _roof(kernel, flop, nbytes, sec, mfma_peak):
    """The binding resource is the one with the larger ideal time."""
    t_mfma = flop / (mfma_peak * 1e12)
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    if t_hbm >= t_mfma:
        r = {"kernel": kernel, "bound": "hbm", "achieved": nbytes / sec / 1e9, "peak": HBM_PEAK_GBS,
             "unit": "GB/s"}
    else:
        r = {"kernel": kernel, "bound": "mfma", "achieved": flop / sec / 1e12, "peak": mfma_peak,
             "unit": "TFLOP/s"}
    r["frac"] = r["achieved"] / r["peak"]
    r["traffic"] = None
    r["algorithmic"] = {"flop": flop, "bytes": nbytes}
    return r


def bench_backward(args):
    """Indexer-loss backward (the step after the path) on the workload."""
    import numpy as np
    import torch
    from deepseek_v4_csa_amd import inputs as I
    from deepseek_v4_csa_amd import ops
    wl = next(w for w in I.WORKLOADS if w.name == args.workload)
    dev = torch.device("cuda:0")
    inp = I.make_inputs(wl, device="cuda")
    res = ops.forward(inp, want_teacher=True)
    L = ops.layout_of_inputs(inp)
    T = wl.total_q
    g = torch.empty((T, wl.max_seqlen_k), dtype=torch.float32, device=dev)
    dq = torch.empty(tuple(inp.q_idx.shape), dtype=torch.float32, device=dev)
    dw = torch.empty(tuple(inp.weights.shape), dtype=torch.float32, device=dev)
    dk = torch.empty(tuple(inp.k_idx.shape), dtype=torch.float32, device=dev)
    ws = torch.empty((max(ops.csa_indexer_loss_bwd_workspace(L, wl.Hi, wl.Di), 1),), dtype=torch.uint8,
                     device=dev)
    call = lambda: ops.csa_indexer_loss_bwd(L, wl.sparse_loss, inp.q_idx, inp.k_idx, inp.weights,
                                            inp.idx_scale, res["scores"], res["ids"], res["teacher"],
                                            grad_scores=g, dq_idx=dq, dweights=dw, dk_idx=dk, workspace=ws)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for k in range(args.steps):
        ev[k][0].record()
        call()
        ev[k][1].record()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    call_ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    nv, kt, _ = geometry(wl)
    S = int(kt.sum()) if wl.sparse_loss else int(nv.sum())      # support pairs
    P = int(nv.sum())
    flop = 6 * wl.Hi * wl.Di * S          # d recomputed once, dq and dk contractions
    nbytes = (2 * T * wl.Hi * wl.Di + 2 * wl.total_k * wl.Di + 4 * T * wl.Hi
              + (12 * T * wl.k_eff if wl.sparse_loss else 8 * P)
              + 4 * T * wl.Hi * wl.Di + 4 * T * wl.Hi + 4 * wl.total_k * wl.Di)
    roof = _roof("csa_indexer_loss_bwd (score gradients, dq/dweights, dk, dk reduce)", flop, nbytes,
                 call_ms * 1e-3, BF16_MFMA_PEAK_TFLOPS)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        rows = I.uniform_rows(T, 4096, seed=13)
        P_ = _oracle_problem(inp, rows)
        Lo = P_.layout
        t1 = time.perf_counter()
        done = 0
        for t in rows:
            r = oracle.run_row(P_, int(t))
            cols, tch, prd = oracle.loss_support(P_, r)
            if cols.size:
                gs = oracle.kl_grad_scores(tch, prd) / T
                ge = r.geom
                oracle.indexer_grads_row(P_.q_idx[t], P_.weights[t],
                                         P_.k_idx[ge.k_base:int(Lo.cu_k[ge.seg + 1])], P_.idx_scale, cols, gs)
            done += 1
            if time.perf_counter() - t1 >= args.cpu_seconds:
                break
        e1 = time.perf_counter() - t1
        cpu = {"value": done / e1, "unit": "query tokens/s", "cores": int(_threads()), "kind": "oracle",
               "sample": f"{done} uniformly drawn rows of {T} ({wl.name}): each row's forward (for the "
                         f"teacher) and its indexer gradients in NumPy float64, {e1:.1f} s"}
    _line("query tokens/s through the indexer-loss backward (dq_idx, dweights, dk_idx)", T * args.steps / el,
          args, el / args.steps * 1e3, "bf16", {**wl.describe(), "row": "indexer-loss backward",
                                                 "support_pairs": S, "parallelism": "none (1 GPU)"},
          roof, cpu, {"call_us": call_ms * 1e3})


def bench_cp_share(args):
    """One rank's share of CP scoring (indexer + top-k) of the 65,536-token sequence."""
    import numpy as np
    import torch
    from deepseek_v4_csa_amd import inputs as I
    from deepseek_v4_csa_amd import ops
    base = I.WORKLOADS[3]
    dev = torch.device("cuda:0")
    plan = ops.csa_cp_plan(list(base.seg_lens), base.ratio, args.cp, args.rank)
    nseg = len(plan["off"])
    seg_q = [plan["cu_q"][s + 1] - plan["cu_q"][s] for s in range(nseg)]
    seg_k = [plan["cu_k"][s + 1] - plan["cu_k"][s] for s in range(nseg)]
    # the rank's own rows and the sequence's keys, drawn like the workload's indexer inputs
    gen = torch.Generator(device="cuda")
    gen.manual_seed(I.SEED_BASE + 300 + args.rank)
    sd = 1.0 / np.sqrt(base.D)
    Ts = sum(seg_q)
    q_idx = (torch.randn((Ts, base.Hi, base.Di), generator=gen, device=dev) * sd).to(torch.bfloat16)
    weights = torch.rand((Ts, base.Hi), generator=gen, device=dev)
    k_all = (torch.randn((base.total_k, base.Di), generator=gen, device=dev) * sd).to(torch.bfloat16)
    kidx = torch.cat([torch.arange(plan["k_src"][s], plan["k_src"][s] + seg_k[s], device=dev)
                      for s in range(nseg)])
    k_idx = k_all.index_select(0, kidx).contiguous()
    L = ops.Layout.from_lengths(seg_q, seg_k, base.ratio, offsets=plan["off"])
    k_eff = ops.k_eff(L, base.topk)
    scores = torch.empty((Ts, L.max_seqlen_k), dtype=torch.float32, device=dev)
    ids = torch.empty((Ts, k_eff), dtype=torch.int32, device=dev)
    idx_scale = 1.0 / np.sqrt(base.Di)

    def step(ev=None):
        if ev: ev[0].record()
        ops.csa_indexer_score(L, q_idx, k_idx, weights, idx_scale, scores=scores)
        if ev: ev[1].record()
        ops.csa_topk(L, scores, base.topk, ids=ids)
        if ev: ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(ev[k])
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    idx_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    topk_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    # causal pairs of the share: row at absolute position i sees floor(i / ratio) keys
    P = 0
    for s in range(nseg):
        i = np.arange(plan["off"][s] + 1, plan["off"][s] + seg_q[s] + 1)
        P += int(np.minimum(i // base.ratio, seg_k[s]).sum())
    flop = 2 * base.Hi * base.Di * P
    roof = _roof("indexer_score", flop, 2 * Ts * base.Hi * base.Di + 2 * sum(seg_k) * base.Di + 4 * P,
                 idx_ms * 1e-3, BF16_MFMA_PEAK_TFLOPS)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        qh = q_idx.to("cpu", torch.float64).numpy()
        wh = weights.cpu().numpy()
        kh = k_idx.to("cpu", torch.float64).numpy()
        cu_k = plan["cu_k"]
        rng = np.random.default_rng(17)
        order = rng.permutation(Ts)
        t1 = time.perf_counter()
        done = 0
        starts = np.asarray(plan["cu_q"])
        for t in order:
            s = int(np.searchsorted(starts, t, side="right") - 1)
            nvv = min((plan["off"][s] + (t - starts[s]) + 1) // base.ratio, seg_k[s])
            sc = oracle.indexer_scores_row(qh[t], wh[t], kh[cu_k[s]:cu_k[s + 1]], idx_scale, nvv)
            oracle.topk_row(sc, nvv, k_eff, cu_k[s])
            done += 1
            if time.perf_counter() - t1 >= args.cpu_seconds:
                break
        e1 = time.perf_counter() - t1
        cpu = {"value": done / e1, "unit": "query tokens/s", "cores": int(_threads()), "kind": "oracle",
               "sample": f"{done} uniformly drawn rows of the {Ts}-row share: indexer scores and top-k "
                         f"per row in NumPy float64, {e1:.1f} s"}
    _line("query tokens/s of one rank's CP scoring share (indexer + top-k)", Ts * args.steps / el, args,
          el / args.steps * 1e3, "bf16",
          {"workload": f"{base.name}-cp{args.cp}-rank{args.rank}", "sequence": base.seg_lens[0],
           "cp_size": args.cp, "rank": args.rank, "share_rows": Ts, "segments": seg_q,
           "key_prefixes": seg_k, "offsets": plan["off"], "indexer_heads": base.Hi,
           "indexer_dim": base.Di, "topk": base.topk, "compress_ratio": base.ratio,
           "parallelism": "one rank's share on 1 GPU"},
          roof, cpu, {"kernels": {"indexer_score": {"us": idx_ms * 1e3,
                                                    "tflops": flop / (idx_ms * 1e-3) / 1e12},
                                  "topk": {"us": topk_ms * 1e3,
                                           "gbs": (4 * P + 4 * Ts * k_eff) / (topk_ms * 1e-3) / 1e9}}})


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import torch
    from deepseek_v4_csa_amd import ops
    ops.load()
    torch.cuda.set_device(0)
    if args.row == "backward":
        return bench_backward(args)
    if args.row == "cp-share":
        return bench_cp_share(args)
    from deepseek_v4_csa_amd import inputs as I

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

    # the fused score + top-k call where it applies (sparse loss, supported shape): the
    # score matrix is never stored and the teacher/KL reads the selected scores
    fused = wl.sparse_loss and not args.unfused
    sel = None
    if fused:
        sel = torch.empty((T, k_eff), dtype=torch.float32, device=dev)
        try:
            ops.csa_indexer_topk(L, inp.q_idx, inp.k_idx, inp.weights, inp.idx_scale, wl.topk, ids=ids,
                                 sel_scores=sel)
        except RuntimeError:
            fused, sel = False, None
    if fused:
        scores = None
    # sparse loss on shapes the one-wave-per-query kernel takes (bf16, H <= 16, D of 64 or
    # 128, a window, k_eff <= 256, the selected scores of the fused top-k): attention,
    # teacher and KL in one call, the loss reduced by its own call
    attn_kl = (wl.sparse_loss and args.one_call_attn and sel is not None and wl.dtype != "f32"
               and wl.H <= 16 and wl.D in (64, 128) and wl.window > 0 and k_eff <= 256)
    att_name = "sparse_attn_kl" if attn_kl else "sparse_attn"
    names = (("indexer_topk",) if fused else ("indexer_score", "topk")) + \
        ((att_name, "loss_reduce") if attn_kl else (att_name, "teacher_kl"))
    # every ctypes argument is marshalled once, so the host enqueues far ahead of the GPU
    P = ops.Prepared(L, inp, scores, ids, out, lse, lse_nc, cmass, kl_row, loss,
                     wl.sparse_loss, wl.topk, wl.window, sel=sel)
    att_call = P.csa_sparse_attn_kl_fwd if attn_kl else P.csa_sparse_attn_fwd
    tail_call = P.csa_loss_reduce if attn_kl else P.csa_indexer_teacher_kl

    def step(ev=None):
        if fused:
            P.csa_indexer_topk()
        else:
            P.csa_indexer_score()
            P.csa_topk()
        if ev: ev[0].record()
        att_call()
        if ev: ev[1].record()
        tail_call()

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
    calls = ((P.csa_indexer_topk,) if fused else (P.csa_indexer_score, P.csa_topk)) + (att_call, tail_call)
    bev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(nb)]
    for ev in bev:
        ev[0].record()
        for i, f in enumerate(calls):
            f()
            ev[i + 1].record()
    torch.cuda.synchronize()
    per_kernel_ms = {n: sum(ev[i].elapsed_time(ev[i + 1]) for ev in bev) / nb for i, n in enumerate(names)}
    value = T * args.steps / elapsed
    wm = work_model(wl)

    # The attention's roofline: algorithmic bytes on the gather model (each query's
    # window and selected KV rows counted once per query, plus q, out and the per-row
    # statistics; with the teacher/KL finished in its epilogue also the selected scores it
    # reads and kl_row) against the HBM peak, and its algorithmic FLOP (4 H D per gathered
    # row) against the MFMA peak; the binding resource is the one with the larger ideal
    # time.  The unique KV rows are small enough for the caches, so the DRAM bytes the
    # counters see (traffic) stay below the gather-model bytes.
    att_bytes = wm["attn_bytes"] + ((4 * T * k_eff + 4 * T) if attn_kl else 0)
    mfma_peak = FP32_MFMA_PEAK_TFLOPS if wl.dtype == "f32" else BF16_MFMA_PEAK_TFLOPS
    att_sec = att_ms * 1e-3
    hbm = {"achieved": att_bytes / att_sec / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    mfma = {"achieved": wm["attn_flop"] / att_sec / 1e12, "peak": mfma_peak, "unit": "TFLOP/s"}
    hbm_bound = att_bytes / (HBM_PEAK_GBS * 1e9) >= wm["attn_flop"] / (mfma_peak * 1e12)
    roof = {"kernel": att_name, "bound": "hbm" if hbm_bound else "mfma", **(hbm if hbm_bound else mfma),
            "traffic": traffic_of(wl.name, att_name)}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["model"] = "gather: every query's window and selected KV rows counted once, plus q, out and row statistics"
    roof["algorithmic"] = {"bytes": att_bytes, "flop": wm["attn_flop"]}
    roof["frac_mfma"] = mfma["achieved"] / mfma["peak"]
    roof["frac_hbm_gather"] = hbm["achieved"] / hbm["peak"]
    if roof["traffic"] is not None:
        roof["frac_hbm_counters"] = roof["traffic"] / att_sec / 1e9 / HBM_PEAK_GBS
    idx_peak = mfma_peak
    kernels = {}
    if fused:
        kernels["indexer_topk"] = {
            "us": per_kernel_ms["indexer_topk"] * 1e3,
            "tflops": wm["indexer_flop"] / (per_kernel_ms["indexer_topk"] * 1e-3) / 1e12,
            "frac_mfma_peak": wm["indexer_flop"] / (per_kernel_ms["indexer_topk"] * 1e-3) / 1e12 / idx_peak}
    else:
        kernels["indexer_score"] = {
            "us": per_kernel_ms["indexer_score"] * 1e3,
            "tflops": wm["indexer_flop"] / (per_kernel_ms["indexer_score"] * 1e-3) / 1e12,
            "frac_mfma_peak": wm["indexer_flop"] / (per_kernel_ms["indexer_score"] * 1e-3) / 1e12 / idx_peak}
        kernels["topk"] = {"us": per_kernel_ms["topk"] * 1e3,
                           "gbs": wm["topk_bytes"] / (per_kernel_ms["topk"] * 1e-3) / 1e9}
    kernels[att_name] = {"us": att_ms * 1e3, "gbs_gather_model": hbm["achieved"], "tflops": mfma["achieved"],
                         "frac_mfma_peak": roof["frac_mfma"]}
    if attn_kl:
        kernels["loss_reduce"] = {"us": per_kernel_ms["loss_reduce"] * 1e3}
    else:
        kernels["teacher_kl"] = {"us": per_kernel_ms["teacher_kl"] * 1e3,
                                 "gbs": wm["teacher_bytes"] / (per_kernel_ms["teacher_kl"] * 1e-3) / 1e9}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args.cpu_seconds)
    line = {
        "metric": "query tokens/s for indexer+topk+CSA attn+teacher/KL; % MFMA / HBM peak",
        "value": value, "unit": "query tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": elapsed / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32" if wl.dtype == "f32" else "bf16",
        "data": "synthetic",
        "config": {**wl.describe(), "parallelism": "none (1 GPU)",
                   "score_path": "fused score + top-k (no score matrix)" if fused else "score and top-k calls",
                   "attention_path": "attention + teacher/KL in one call" if attn_kl
                   else "attention and teacher/KL calls"},
        "roofline": roof, "cpu_baseline": cpu, "kernels": kernels,
        "loss": float(loss[0]),
    }
    print(json.dumps(line))


# ------------------------------------------------------------------ measurement tools
COPY_BYTES = 1 << 30
KSRC = os.path.join(ROOT, "deepseek_v4_csa_amd", "csrc", "kernels")
# kernel family -> (name prefix in the trace, source file)
FAMILIES = {
    "indexer_topk": ("csa::indexer_score_lds_kernel", "indexer_score.hip"),
    "indexer_score": ("csa::indexer_score", "indexer_score.hip"),
    "topk": ("csa::topk", "topk.hip"),
    "sparse_attn": ("csa::sparse_attn", "sparse_attn.hip"),
    "sparse_attn_kl": ("csa::sparse_attn_pipe_kernel", "sparse_attn.hip"),
    "teacher_kl": ("csa::teacher_kl", "teacher_kl.hip"),
    "loss_reduce": ("csa::loss_reduce", "teacher_kl.hip"),
}


def copy_probe():
    """A plain device copy of COPY_BYTES, three times (counter calibration)."""
    import torch
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {COPY_BYTES} bytes x3")


def _short(name: str) -> str:
    import re
    name = re.sub(r"^void ", "", name)
    return re.sub(r"\(.*", "", name)


def _source_of(name: str, fam: str) -> str:
    if "sparse_attn_wide_lse" in name:
        return "sparse_attn_wide_lse.hip"
    if "sparse_attn_wide" in name:
        return "sparse_attn_wide.hip"
    return FAMILIES[fam][1]


def _family_of(name: str):
    # the attention kernel that also finishes the teacher and KL (csa_sparse_attn_kl_fwd)
    if "csa::sparse_attn_pipe_kernel" in name and ", true>" in name:
        return "sparse_attn_kl"
    # the fused score + top-k instance of the paired-block indexer kernel
    if "csa::indexer_score_lds_kernel" in name and ", true," in name:
        return "indexer_topk"
    for fam, (prefix, _) in FAMILIES.items():
        if fam != "indexer_topk" and prefix in name:
            return fam
    return None


def _sha256(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def prof_stats(stats_dir: str, out: str, cmd: str) -> None:
    import csv
    rows = list(csv.DictReader(open(os.path.join(stats_dir, "run_kernel_stats.csv"))))
    lines = ["# rocprofv3 kernel statistics", f"# command: {cmd}", "",
             f"{'kernel':<58} {'calls':>6} {'avg us':>9} {'min us':>9} {'max us':>9} {'% time':>7}"]
    for r in rows:
        lines.append(f"{_short(r['Name'])[:58]:<58} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>9.2f} "
                     f"{float(r['MinNs']) / 1e3:>9.2f} {float(r['MaxNs']) / 1e3:>9.2f} {float(r['Percentage']):>7.2f}")
    open(out, "w").write("\n".join(lines) + "\n")


def _counter_means(d: str, counter: str):
    import collections
    import csv
    acc = collections.defaultdict(list)
    for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
        if r["Counter_Name"] == counter:
            acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}


def _copy_scale(d: str, counter: str) -> float:
    """Bytes per counter unit, from the plain copy kernel of copy-probe."""
    means, _ = _counter_means(d, counter)
    copies = {k: v for k, v in means.items() if "copyBuffer" in k}
    if len(copies) != 1:
        raise SystemExit(f"{d}: expected one copy kernel, found {list(copies)}")
    return COPY_BYTES / next(iter(copies.values()))


def prof_traffic(wl: str, fdir: str, wdir: str, cfdir: str, cwdir: str, prefix: str, cmd: str) -> None:
    fs, ws = _copy_scale(cfdir, "FETCH_SIZE"), _copy_scale(cwdir, "WRITE_SIZE")
    fm, fn = _counter_means(fdir, "FETCH_SIZE")
    wm, _ = _counter_means(wdir, "WRITE_SIZE")
    table = {}
    lines = [f"# HBM traffic per launch, workload {wl}", f"# command: {cmd}",
             f"# scale: FETCH_SIZE x {fs:.4f} B/unit, WRITE_SIZE x {ws:.4f} B/unit "
             f"(copy of {COPY_BYTES} B)", "",
             f"{'kernel':<50} {'n':>4} {'FETCH KiB':>11} {'WRITE KiB':>11} {'read MB':>9} {'write MB':>9}"]
    for name, fv in sorted(fm.items()):
        fam = _family_of(name)
        if fam is None:
            continue
        wv = wm.get(name, 0.0)
        rd, wr = fv * fs, wv * ws
        src = os.path.join(KSRC, _source_of(name, fam))
        # one call may launch several kernels of the family (the D = 512 attention: the lse
        # kernel, then the output kernel): their bytes add up per call
        e = table.setdefault(fam, {"kernels": [], "read_bytes": 0.0, "write_bytes": 0.0,
                                   "hbm_bytes_per_launch": 0.0, "sources": {}})
        e["kernels"].append({"kernel": _short(name), "dispatches": fn[name], "fetch_counter": fv,
                             "write_counter": wv, "read_bytes": rd, "write_bytes": wr})
        e["read_bytes"] += rd
        e["write_bytes"] += wr
        e["hbm_bytes_per_launch"] += rd + wr
        e["sources"][os.path.relpath(src, ROOT)] = _sha256(src)
        lines.append(f"{_short(name)[:50]:<50} {fn[name]:>4} {fv:>11.1f} {wv:>11.1f} {rd / 1e6:>9.2f} {wr / 1e6:>9.2f}")
    doc = {"workload": wl, "command": cmd, "fetch_scale": fs, "write_scale": ws, "kernels": table}
    json.dump(doc, open(prefix + ".json", "w"), indent=1)
    open(prefix + ".txt", "w").write("\n".join(lines) + "\n")


# SQ counters of the counter summaries; the MFMA busy fraction is
# SQ_VALU_MFMA_BUSY_CYCLES / (4 SQ_BUSY_CU_CYCLES) (busy cycles summed over the 4 SIMDs of
# every CU against the busy cycles summed over the CUs)
SQ_COUNTERS = ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES",
               "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_WAIT_INST_LDS")


def prof_counters(wl: str, cdir: str, out: str, cmd: str) -> None:
    """Per-kernel means per dispatch of the SQ counters of one --pmc pass, with the LDS
    bank-conflict ratio and the MFMA busy fraction."""
    means = {c: _counter_means(cdir, c) for c in SQ_COUNTERS}
    names = sorted({k for m, _ in means.values() for k in m if _family_of(k)})
    lines = [f"# SQ counters per launch, workload {wl}", f"# command: {cmd}",
             "# lds_conflict = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE;"
             " mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (4 SQ_BUSY_CU_CYCLES)", ""]
    for k in names:
        v = {c: means[c][0].get(k, 0.0) for c in SQ_COUNTERS}
        n = max(means[c][1].get(k, 0) for c in SQ_COUNTERS)
        conf = v["SQ_LDS_BANK_CONFLICT"] / v["SQ_LDS_IDX_ACTIVE"] if v["SQ_LDS_IDX_ACTIVE"] else 0.0
        busy = v["SQ_VALU_MFMA_BUSY_CYCLES"] / (4 * v["SQ_BUSY_CU_CYCLES"]) if v["SQ_BUSY_CU_CYCLES"] else 0.0
        lines.append(f"{_short(k)}  (dispatches {n})")
        lines.append(f"    lds_conflict {conf:.4f}   mfma_busy {busy:.3f}")
        lines.append("    " + "  ".join(f"{c[3:]}={v[c]:.4g}" for c in SQ_COUNTERS))
    open(out, "w").write("\n".join(lines) + "\n")


def tools_main(argv):
    ap = argparse.ArgumentParser(prog="bench.py")
    sub = ap.add_subparsers(dest="tool", required=True)
    sub.add_parser("copy-probe")
    ps = sub.add_parser("prof-summary")
    pm = ps.add_subparsers(dest="mode", required=True)
    s = pm.add_parser("stats")
    s.add_argument("stats_dir")
    s.add_argument("out")
    s.add_argument("--cmd", required=True)
    t = pm.add_parser("traffic")
    for a in ("workload", "fetch_dir", "write_dir", "copy_fetch_dir", "copy_write_dir", "out_prefix"):
        t.add_argument(a)
    t.add_argument("--cmd", required=True)
    c = pm.add_parser("counters")
    for a_ in ("workload", "counter_dir", "out"):
        c.add_argument(a_)
    c.add_argument("--cmd", required=True)
    a = ap.parse_args(argv)
    if a.tool == "copy-probe":
        copy_probe()
    elif a.mode == "stats":
        prof_stats(a.stats_dir, a.out, a.cmd)
    elif a.mode == "counters":
        prof_counters(a.workload, a.counter_dir, a.out, a.cmd)
    else:
        prof_traffic(a.workload, a.fetch_dir, a.write_dir, a.copy_fetch_dir, a.copy_write_dir, a.out_prefix,
                     a.cmd)


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] in ("copy-probe", "prof-summary"):
        tools_main(sys.argv[1:])
    else:
        main()
