"""Builds libdiffattn.so in-tree with hipcc for gfx950.

Every HIP translation unit under csrc/ is compiled to an object file in
``_build/`` (in parallel) and linked into ``libdiffattn.so`` next to this file.
``build(debug=True)`` builds the same sources with DIFFATTN_DEBUG_BARRIERS (an extra
workgroup barrier at every step of the kernels' main loops) into ``_build/debug/`` and
``libdiffattn_debug.so``; its results must equal the normal build's bit for bit.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdiffattn.so")
LIB_DEBUG = os.path.join(PKG, "libdiffattn_debug.so")
# Marker ranges around the entry points (rocprofiler-sdk's roctx).
LINK_LIBS = ["-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx", "-Wl,-rpath,/opt/rocm/lib"]

SOURCES = ["api.cpp", "lambda.hip", "fwd_fp32.hip", "fwd_bf16.hip", "decode.hip", "bwd.hip",
           "append.hip", "gemm.hip", "scratch.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed float32 ops (v_pk_*_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]

# Kernel sources: no NaN inputs are supported, so max/min need no canonicalisation of
# MFMA results. The host-side argument checks (api.cpp) keep IEEE NaN semantics so that
# their finiteness tests are not folded away.
KERNEL_FLAGS = ["-fno-honor-nans"]

# Per-file extra flags.
FILE_FLAGS = {s: KERNEL_FLAGS for s in SOURCES if s.endswith(".hip")}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def _compile(src: str, extra, outdir: str) -> str:
    obj = os.path.join(outdir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc()] + HIPCC_FLAGS + FILE_FLAGS.get(src, []) + list(extra) + \
        ["-I", INCLUDE, "-I", CSRC] + lang + \
        ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(extra_flags=(), debug: bool = False) -> str:
    """Compile every source and link libdiffattn.so (or, with debug, the debug-barrier
    build libdiffattn_debug.so); returns the library path."""
    outdir = os.path.join(BUILD, "debug") if debug else BUILD
    lib = LIB_DEBUG if debug else LIB
    flags = list(extra_flags) + (["-DDIFFATTN_DEBUG_BARRIERS"] if debug else [])
    os.makedirs(outdir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, flags, outdir), SOURCES))
    tmp = lib + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs + LINK_LIBS
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    args = sys.argv[1:]
    debug = "--debug" in args
    print(build([a for a in args if a != "--debug"], debug=debug))
