"""Build libcsa.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m deepseek_v4_csa_amd.build        # or: python deepseek_v4_csa_amd/build.py

Each source is compiled by hipcc to an object under _build/, then linked into
deepseek_v4_csa_amd/libcsa.so.  Always rebuilds (the sources are small).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcsa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = [
    os.path.join(CSRC, "csa_api.cpp"),
    os.path.join(CSRC, "kernels", "indexer_score.hip"),
    os.path.join(CSRC, "kernels", "topk.hip"),
    os.path.join(CSRC, "kernels", "sparse_attn.hip"),
    os.path.join(CSRC, "kernels", "sparse_attn_wide.hip"),
    os.path.join(CSRC, "kernels", "sparse_attn_wide_lse.hip"),
    os.path.join(CSRC, "kernels", "teacher_kl.hip"),
    os.path.join(CSRC, "kernels", "indexer_bwd.hip"),
]

# packed-fp32 VALU ops are disabled for every device pass; the host pass warns that it
# does not know the feature, which is harmless
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-result",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]
# MFMA results in VGPRs (the kernels keep at most 256 registers per lane), except in the
# wide attention kernel, whose single wave per SIMD keeps its output accumulators in AGPRs
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
AGPR_SOURCES = {"sparse_attn_wide.hip"}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    extra = [] if os.path.basename(src) in AGPR_SOURCES else VGPR_FORM
    cmd = [HIPCC, *FLAGS, *extra, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
