"""Build libmla.so in-tree with hipcc for gfx950.

Usage: python mla_decode_decoupled_amd/build.py [--debug]
(run by path: importing the package first would load the library being replaced)
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libmla.so")
SOURCES = ["api.hip", "generic.hip", "decode_fast.hip", "proj_fast.hip", "proj_gemm.hip", "linear.hip", "prefill_explicit.hip"]

# Packed-FP32 instructions (v_pk_*_f32) are switched off for every device pass: the compiler
# otherwise forms them from plain float code, and the kernels are validated without them.
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmla)")


def build(debug: bool = False, verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, "-I", os.path.join(PKG_DIR, os.pardir, "include"), "-o", tmp, *srcs]
    if debug:
        cmd = [c for c in cmd if c != "-O3"] + ["-O1", "-g"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that noise.
    noise = "packed-fp32-ops"
    err = "\n".join(line for line in res.stderr.splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    path = build(debug="--debug" in sys.argv, verbose=True)
    print(path)
