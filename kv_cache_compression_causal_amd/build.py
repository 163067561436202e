"""Build liblt.so (the HIP kernels + C ABI) for gfx950 with hipcc.

Run as ``python -m kv_cache_compression_causal_amd.build``.  Objects go to
``_build/`` at the repository root; the shared library lands next to this
file so that it ships with the source tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblt.so")
# The same sources built with LT_POISON_LDS: every kernel fills its LDS with
# NaN before first use (a check for reads of unwritten LDS; tests compare it
# with liblt.so bit for bit).  Not the product library.
LIB_DEBUG = os.path.join(PKG, "liblt_debug.so")
ARCH = "gfx950"

SOURCES = ["attn_bf16.hip", "attn_f32.hip", "decode.hip", "compact.hip", "probe.hip", "lt_api.cpp",
           "lazy_queue.cpp"]

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _compile(src: str, debug: bool = False) -> str:
    objdir = os.path.join(OBJDIR, "debug") if debug else OBJDIR
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [_hipcc()] + HIPCC_FLAGS + (["-DLT_POISON_LDS"] if debug else []) + lang + ["-c", path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj


def _build_one(debug: bool, verbose: bool) -> str:
    out = LIB_DEBUG if debug else LIB
    os.makedirs(os.path.join(OBJDIR, "debug") if debug else OBJDIR, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, debug), SOURCES))
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def build(verbose: bool = False, debug: bool = True) -> str:
    """Compile every source (always) and link liblt.so, and (debug=True) the
    LDS-poisoning liblt_debug.so beside it; returns the liblt.so path."""
    lib = _build_one(False, verbose)
    if debug:
        _build_one(True, verbose)
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
