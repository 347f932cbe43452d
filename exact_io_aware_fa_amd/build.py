"""Build libfa.so in-tree with hipcc for gfx950.

    python -m exact_io_aware_fa_amd.build

Every source is compiled on every call (objects under _build/), then linked
into exact_io_aware_fa_amd/libfa.so; the same sources built with
FA_DEBUG_SYNC give libfa_debug.so, which the race-check tests compare with
it.  No GPU is needed: hipcc cross-compiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")
DEBUG_LIB = os.path.join(PKG, "libfa_debug.so")   # FA_DEBUG_SYNC build: the race check's reference
ARCH = "gfx950"
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HIP_SOURCES = ["fa_prefill_bf16.hip", "fa_prefill_f32.hip", "fa_decode.hip", "fa_bwd_bf16.hip"]
HOST_SOURCES = ["fa_api.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-result"]
# Packed fp32 VALU instructions stay disabled for all device code.
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def _compile(src: str, extra: list[str], build_dir: str = BUILD) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [hipcc()] + COMMON + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def build(verbose: bool = False, out: str = LIB, defines: tuple = ()) -> str:
    """Compile and link the library into `out`; `defines` (NAME=VALUE strings)
    override tuning constants of the kernels."""
    build_dir = BUILD if out == LIB else out + ".objs"
    os.makedirs(build_dir, exist_ok=True)
    dflags = ["-D" + d for d in defines]
    host = ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include")]
    jobs = [(s, DEVICE + dflags) for s in HIP_SOURCES] + [(s, host + dflags) for s in HOST_SOURCES]
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], j[1], build_dir), jobs))
    LIB_OUT = out
    tmp = LIB_OUT + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, LIB_OUT)
    if verbose:
        print("built", LIB_OUT)
    return LIB_OUT


def build_debug(verbose: bool = False) -> str:
    """The same library with FA_DEBUG_SYNC: every copy and barrier drained in
    order; its results must match libfa.so's bit for bit."""
    return build(verbose=verbose, out=DEBUG_LIB, defines=("FA_DEBUG_SYNC=1",))


if __name__ == "__main__":
    build(verbose=True)
    build_debug(verbose=True)
    sys.exit(0)
