"""Build libmoe.so (HIP for gfx950) in-tree.

    python -m quantized_moe_expert_softmax_amd.build

Every source is compiled with hipcc for gfx950 only, correctly rounded fp32
divides (the HIP default; never fast-math) and packed fp32 VALU instructions
disabled, then linked into ``libmoe.so`` next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe.so")
SOURCES = ["mv_q8_0.hip", "mv_q4_0.hip", "mv_q5_1.hip", "mv_q4_k.hip", "mv_q5_k.hip", "mv_q3_k.hip",
           "mv_nvfp4.hip",
           "mfma.hip", "thin.hip",
           "route.hip", "matvec.hip", "table.hip", "probe.hip", "capi.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libmoe")


COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-x", "hip",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-fast-math", "-ffp-contract=fast-honor-pragmas", "-Wall", "-Wno-unused-function",
          "-Wno-unused-command-line-argument", "-I", os.path.join(HERE, "..", "include")]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-8000:]}")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source and link libmoe.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-8000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
