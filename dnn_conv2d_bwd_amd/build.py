"""Build libcbd.so (planner, C ABI and gfx950 kernels) in-tree with hipcc.

    python dnn_conv2d_bwd_amd/build.py

Objects go to _build/ at the repository root; the shared library lands next
to this file so it travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libcbd.so")
OBJDIR = os.path.join(ROOT, "_build", "cbd")

SOURCES = [
    "cbd_plan.cpp",
    "cbd_api.cpp",
    "cbd_noalloc.hip",
    "kern_igemm_generic.hip",
    "kern_igemm_nhwc_bf16.hip",
    "kern_grouped_direct.hip",
    "kern_grouped_rows.hip",
    "kern_grouped_pipe.hip",
    "kern_grouped_mfma.hip",
    "kern_grouped_wide.hip",
    "kern_zero_fill.hip",
    "kern_nchw_rows.hip",
]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-x", "hip",
    "-Wall", "-Wno-unused-result",
    # Packed-f32 VALU instructions are kept out of every kernel.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Per-source extra flags.  The large-tile, generic and grouped-MFMA kernels take their
# tensors (and sizes) as leading scalar parameters, preloaded into SGPRs at
# wave launch (code objects keep a fallback that loads them for firmware
# without preloading).
EXTRA = {
    "kern_igemm_nhwc_bf16.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=16"],
    "kern_igemm_generic.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=16"],
    "kern_grouped_mfma.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=16"],
}


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = min(len(SOURCES), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
