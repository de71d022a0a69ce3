"""Builds the SparsePR HIP library (libsparsepr.so) in-tree for gfx950 with hipcc.

Usage: python -m free_block_sparse_response_amd.build [--jobs N]
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libsparsepr.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["plan_kernels.hip", "attn_kernels.hip", "ridge_kernels.hip", "sparsepr_api.hip",
           "static_workspace.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
         # keep the compiler from forming packed fp32 vector ops
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source extras. The attention kernels see no NaN inputs (masked scores are -inf, never
# NaN), so fmax needs no quieting of its operands and maps to bare v_max3_f32.
EXTRA = {"attn_kernels.hip": ["-fno-honor-nans"]}


def _compile(src):
    obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    return obj, msgs


def build(jobs=4, verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    if verbose:
        for _, m in results:
            if m.strip():
                print(m)
    objs = [o for o, _ in results]
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    jobs = int(sys.argv[sys.argv.index("--jobs") + 1]) if "--jobs" in sys.argv else 4
    print(build(jobs=jobs, verbose=True))
