"""Turn rocprofv3 CSV output of ``bench.py`` into the short text summaries kept in
``profiles/`` and the per-kernel HBM traffic table that ``bench.py`` reports.

    python -m deepseek_v4_csa_amd.prof_summary stats  <stats_dir> <out.txt> --cmd "<command>"
    python -m deepseek_v4_csa_amd.prof_summary traffic <workload> <fetch_dir> <write_dir> \\
        <copy_fetch_dir> <copy_write_dir> <out_prefix> --cmd "<command>"

``stats_dir`` holds ``run_kernel_stats.csv`` (``rocprofv3 --kernel-trace --stats
--output-format csv -o run``); the counter directories hold ``run_counter_collection.csv``
of one ``--pmc FETCH_SIZE`` or ``--pmc WRITE_SIZE`` pass each, of the bench and of
``copy_probe.py``.  The copy moves a known number of bytes, so bytes / counter is the
scale that turns each counter into HBM bytes (reported beside the result).
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re

from . import copy_probe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KSRC = os.path.join(ROOT, "deepseek_v4_csa_amd", "csrc", "kernels")

# kernel family -> (name prefix in the trace, source file)
FAMILIES = {
    "indexer_score": ("csa::indexer_score", "indexer_score.hip"),
    "topk": ("csa::topk", "topk.hip"),
    "sparse_attn": ("csa::sparse_attn", "sparse_attn.hip"),
    "sparse_attn_kl": ("csa::sparse_attn_pipe_kernel", "sparse_attn.hip"),
    "teacher_kl": ("csa::teacher_kl", "teacher_kl.hip"),
    "loss_reduce": ("csa::loss_reduce", "teacher_kl.hip"),
}


def short(name: str) -> str:
    name = re.sub(r"^void ", "", name)
    return re.sub(r"\(.*", "", name)


def family_of(name: str):
    # the attention kernel that also finishes the teacher and KL (csa_sparse_attn_kl_fwd)
    if "csa::sparse_attn_pipe_kernel" in name and ", true>" in name:
        return "sparse_attn_kl"
    for fam, (prefix, _) in FAMILIES.items():
        if prefix in name:
            return fam
    return None


def sha256(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def stats(stats_dir: str, out: str, cmd: str) -> None:
    rows = list(csv.DictReader(open(os.path.join(stats_dir, "run_kernel_stats.csv"))))
    lines = [f"# rocprofv3 kernel statistics", f"# command: {cmd}", "",
             f"{'kernel':<58} {'calls':>6} {'avg us':>9} {'min us':>9} {'max us':>9} {'% time':>7}"]
    for r in rows:
        lines.append(f"{short(r['Name'])[:58]:<58} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>9.2f} "
                     f"{float(r['MinNs']) / 1e3:>9.2f} {float(r['MaxNs']) / 1e3:>9.2f} {float(r['Percentage']):>7.2f}")
    open(out, "w").write("\n".join(lines) + "\n")


def counter_means(d: str, counter: str):
    acc = collections.defaultdict(list)
    for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
        if r["Counter_Name"] == counter:
            acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}


def copy_scale(d: str, counter: str) -> float:
    """Bytes per counter unit, from the plain copy kernel of copy_probe.py."""
    means, _ = counter_means(d, counter)
    copies = {k: v for k, v in means.items() if "copyBuffer" in k}
    if len(copies) != 1:
        raise SystemExit(f"{d}: expected one copy kernel, found {list(copies)}")
    return copy_probe.N_BYTES / next(iter(copies.values()))


def traffic(wl: str, fdir: str, wdir: str, cfdir: str, cwdir: str, prefix: str, cmd: str) -> None:
    fs, ws = copy_scale(cfdir, "FETCH_SIZE"), copy_scale(cwdir, "WRITE_SIZE")
    fm, fn = counter_means(fdir, "FETCH_SIZE")
    wm, _ = counter_means(wdir, "WRITE_SIZE")
    table = {}
    lines = [f"# HBM traffic per launch, workload {wl}", f"# command: {cmd}",
             f"# scale: FETCH_SIZE x {fs:.4f} B/unit, WRITE_SIZE x {ws:.4f} B/unit "
             f"(copy of {copy_probe.N_BYTES} B)", "",
             f"{'kernel':<50} {'n':>4} {'FETCH KiB':>11} {'WRITE KiB':>11} {'read MB':>9} {'write MB':>9}"]
    for name, fv in sorted(fm.items()):
        fam = family_of(name)
        if fam is None:
            continue
        wv = wm.get(name, 0.0)
        rd, wr = fv * fs, wv * ws
        src = os.path.join(KSRC, FAMILIES[fam][1])
        table[fam] = {"kernel": short(name), "dispatches": fn[name], "fetch_counter": fv, "write_counter": wv,
                      "read_bytes": rd, "write_bytes": wr, "hbm_bytes_per_launch": rd + wr,
                      "source": os.path.relpath(src, ROOT), "source_sha256": sha256(src)}
        lines.append(f"{short(name)[:50]:<50} {fn[name]:>4} {fv:>11.1f} {wv:>11.1f} {rd / 1e6:>9.2f} {wr / 1e6:>9.2f}")
    doc = {"workload": wl, "command": cmd, "fetch_scale": fs, "write_scale": ws, "kernels": table}
    json.dump(doc, open(prefix + ".json", "w"), indent=1)
    open(prefix + ".txt", "w").write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    s = sub.add_parser("stats")
    s.add_argument("stats_dir")
    s.add_argument("out")
    s.add_argument("--cmd", required=True)
    t = sub.add_parser("traffic")
    for a in ("workload", "fetch_dir", "write_dir", "copy_fetch_dir", "copy_write_dir", "out_prefix"):
        t.add_argument(a)
    t.add_argument("--cmd", required=True)
    a = ap.parse_args()
    if a.mode == "stats":
        stats(a.stats_dir, a.out, a.cmd)
    else:
        traffic(a.workload, a.fetch_dir, a.write_dir, a.copy_fetch_dir, a.copy_write_dir, a.out_prefix, a.cmd)


if __name__ == "__main__":
    main()
