"""Build libfa2.so (the C-ABI attention library) in-tree with hipcc for gfx950.

Usage: ``python -m tiled_attention_fwd_amd.build`` (or ``build()`` from
Python).  Sources are compiled in parallel into ``_build/`` and linked into
``tiled_attention_fwd_amd/libfa2.so``; the link goes through a temporary
file so a half-written library is never loaded.
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
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa2.so")
SOURCES = ["fa2_api.cpp", "fa2_fwd.hip", "fa2_bwd.hip", "fa2_decode.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    cand = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return cand if os.path.exists(cand) else (shutil.which("hipcc") or "hipcc")


def compile_flags() -> list:
    return [
        "-x", "hip", "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
        "-munsafe-fp-atomics",
        # packed fp32 VALU forms stay off: the compiler must not emit them.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # No NaN ever reaches the kernels' arithmetic (masked scores are -inf,
        # which this keeps): without it every fmaxf on an MFMA result first
        # canonicalises its inputs, one extra VALU op per element.
        "-fno-honor-nans",
        "-I", INCLUDE, "-I", CSRC,
        "-Wno-unused-command-line-argument",
    ]


def _compile(src: str, extra: list) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + compile_flags() + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr[-8000:]))
    return obj


def build(extra_flags: list | None = None, verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libfa2.so; return its path."""
    extra = list(extra_flags or [])
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr[-8000:]))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(sys.argv[1:], verbose=True)
