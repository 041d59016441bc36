"""Build libmla.so in-tree with hipcc for gfx950.

Usage: python mla_decode_decoupled_amd/build.py [--debug] [--sanitize]
(run by path: importing the package first would load the library being replaced)
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libmla.so")
SOURCES = ["api.hip", "generic.hip", "decode_fast.hip", "proj_fast.hip", "proj_gemm.hip", "linear.hip", "prefill_explicit.hip"]
# the ceiling microbenchmarks (MFMA issue, HBM streaming) are a library of their own
CEIL_LIB_PATH = os.path.join(PKG_DIR, "libmla_ceilings.so")
CEIL_SOURCES = ["ceilings.hip"]
# a copy of libmla whose host code (argument checks, planning, launch set-up) runs under AddressSanitizer
# and UndefinedBehaviorSanitizer; the device code is built as usual. Loaded only by the CPU test that
# runs the C-ABI checks against it (tests/test_abi_sanitized.py), with the sanitizer runtime preloaded.
ASAN_LIB_PATH = os.path.join(PKG_DIR, "libmla_asan.so")
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libasan"]
# a copy of libmla whose attention kernels also record per-workgroup phase stamps
# (include/mla_stamps.h); loaded only by bench.py --phase-stamps
STAMPS_LIB_PATH = os.path.join(PKG_DIR, "libmla_stamps.so")
STAMPS_FLAGS = ["-DMLA_PHASE_STAMPS"]

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


def build(debug: bool = False, verbose: bool = False, sanitize: bool = False) -> str:
    """Build libmla.so, libmla_ceilings.so and the phase-stamp build libmla_stamps.so; with sanitize,
    also the host-sanitized libmla_asan.so."""
    _build_one(SOURCES, LIB_PATH, debug, verbose)
    _build_one(CEIL_SOURCES, CEIL_LIB_PATH, debug, verbose)
    _build_one(SOURCES, STAMPS_LIB_PATH, debug, verbose, STAMPS_FLAGS)
    if sanitize:
        _build_one(SOURCES, ASAN_LIB_PATH, debug, verbose, SANITIZE_FLAGS)
    return LIB_PATH


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (preloaded for libmla_asan.so)."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the compiler's shared AddressSanitizer runtime was not found")
    return path


def _run(cmd, verbose: bool) -> None:
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


def _build_one(sources, lib_path: str, debug: bool, verbose: bool, extra=()) -> str:
    """Compile the sources to objects in parallel, then link the library."""
    flags = [*HIP_FLAGS, *extra, "-I", os.path.join(PKG_DIR, os.pardir, "include")]
    if debug:
        flags = [f for f in flags if f != "-O3"] + ["-O1", "-g"]
    compile_flags = [f for f in flags if f != "-shared"]
    obj_dir = lib_path + ".objs"
    os.makedirs(obj_dir, exist_ok=True)
    objs = [os.path.join(obj_dir, os.path.splitext(s)[0] + ".o") for s in sources]
    cmds = [[hipcc(), *compile_flags, "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(sources, objs)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as pool:
        for f in [pool.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = lib_path + ".tmp"
    _run([hipcc(), *flags, "-o", tmp, *objs], verbose)
    os.replace(tmp, lib_path)
    shutil.rmtree(obj_dir, ignore_errors=True)
    return lib_path


if __name__ == "__main__":
    path = build(debug="--debug" in sys.argv, verbose=True, sanitize="--sanitize" in sys.argv)
    print(path)
