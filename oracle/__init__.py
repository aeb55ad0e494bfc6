"""fp64 CPU oracle for softmax attention (forward and backward).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers.  The GPU library and its
Python binding never import this package, and this package imports nothing
from them.

The arithmetic lives in ``oracle.c`` (plain C, fp64, full N x N matrices); this
module only builds it with gcc, loads it with ctypes and marshals numpy arrays.
What it computes, and which passage each step follows, is written at the top
of ``oracle.c``: the plain definition of softmax attention that the article
"Revolutionizing Web-Based AI: How a Plain JavaScript Prototype Paved the Way
for High-Performance WebGPU Flash Attention 2" (section "Translating to WGSL
and Optimizing Passes") says FlashAttention-2 evaluates blockwise.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle C source into a shared library (gcc, OpenMP)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.run(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, src, "-lm"],
            check=True,
        )
        os.replace(tmp, out)
    return out


class Oracle:
    """ctypes view of one compiled oracle library (the default one, or a
    variant the mutation tests build from an edited copy of the source)."""

    def __init__(self, lib_path: str = _LIB):
        if lib_path == _LIB and not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(lib_path)
        dp = ctypes.POINTER(ctypes.c_double)
        L = ctypes.c_long
        lib.oracle_fwd_f64.argtypes = [dp, dp, dp, dp, dp, L, L, L, L, ctypes.c_double, ctypes.c_int]
        lib.oracle_fwd_f64.restype = ctypes.c_int
        lib.oracle_bwd_f64.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, L, L, L, L,
                                       ctypes.c_double, ctypes.c_int]
        lib.oracle_bwd_f64.restype = ctypes.c_int
        lib.oracle_decode_f64.argtypes = [dp, dp, dp, dp, dp, L, L, L, L, L, ctypes.c_double, ctypes.c_int]
        lib.oracle_decode_f64.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        self.lib = lib

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())

    def fwd(self, q, k, v, scale: float, causal: bool):
        """Return (O, LSE) in fp64 for q [B, H, N, d] and k, v [B, H_kv, N, d]
        (numpy or CPU torch); H_kv divides H (H_kv < H: grouped-query
        attention, see _expand_kv)."""
        q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
        B, H, N, d = _shape(q)
        k, v = _expand_kv(k, H), _expand_kv(v, H)
        if k.shape != q.shape or v.shape != q.shape:
            raise ValueError("q, k, v shapes differ")
        o = np.empty_like(q)
        lse = np.empty((B, H, N), dtype=np.float64)
        rc = self.lib.oracle_fwd_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                     B, H, N, d, float(scale), int(bool(causal)))
        if rc != 0:
            raise RuntimeError("oracle_fwd_f64 failed with code %d" % rc)
        return o, lse

    def bwd(self, q, k, v, dO, scale: float, causal: bool, return_delta: bool = False):
        """Return (dQ, dK, dV[, D]) in fp64 for the loss L = sum(O * dO); with
        k, v of H_kv < H heads, dK and dV are [B, H_kv, N, d]."""
        q, k, v, dO = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dO)
        B, H, N, d = _shape(q)
        H_kv = k.shape[1] if k.ndim == 4 else H
        k, v = _expand_kv(k, H), _expand_kv(v, H)
        for t in (k, v, dO):
            if t.shape != q.shape:
                raise ValueError("input shapes differ")
        dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
        delta = np.empty((B, H, N), dtype=np.float64)
        rc = self.lib.oracle_bwd_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(dq), _ptr(dk),
                                     _ptr(dv), _ptr(delta), B, H, N, d, float(scale),
                                     int(bool(causal)))
        if rc != 0:
            raise RuntimeError("oracle_bwd_f64 failed with code %d" % rc)
        dk, dv = _reduce_kv(dk, H_kv), _reduce_kv(dv, H_kv)
        if return_delta:
            return dq, dk, dv, delta
        return dq, dk, dv

    def decode(self, q, k, v, scale: float, causal: bool):
        """Return (O, LSE) in fp64 for N_q queries q [B, H, N_q, d] against a
        cache k, v [B, H_kv, N_k, d] (H_kv divides H); causal places the
        queries at the last N_q positions (see oracle_decode_f64)."""
        q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
        B, H, Nq, d = _shape(q)
        k, v = _expand_kv(k, H), _expand_kv(v, H)
        Nk = k.shape[2]
        if k.shape != (B, H, Nk, d) or v.shape != k.shape:
            raise ValueError("k, v must be [B, H_kv, N_k, d] with q's B and d")
        o = np.empty_like(q)
        lse = np.empty((B, H, Nq), dtype=np.float64)
        rc = self.lib.oracle_decode_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                        B, H, Nq, Nk, d, float(scale), int(bool(causal)))
        if rc != 0:
            raise RuntimeError("oracle_decode_f64 failed with code %d" % rc)
        return o, lse


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def fwd(q, k, v, scale: float, causal: bool):
    """(O, LSE) from the default oracle library."""
    return default().fwd(q, k, v, scale, causal)


def bwd(q, k, v, dO, scale: float, causal: bool, return_delta: bool = False):
    """(dQ, dK, dV[, D]) from the default oracle library."""
    return default().bwd(q, k, v, dO, scale, causal, return_delta)


def decode(q, k, v, scale: float, causal: bool):
    """(O, LSE) of N_q queries against an N_k cache, from the default oracle."""
    return default().decode(q, k, v, scale, causal)


def _expand_kv(t: np.ndarray, H: int) -> np.ndarray:
    """Grouped-query attention (named, not defined, in the article's section
    "Next Frontiers in WebGPU ML", "Broader Opset Support"), read as: query
    head h uses key/value head h // (H / H_kv), i.e. consecutive groups of
    H / H_kv query heads share one K, V head.  It is exactly multi-head
    attention on K and V with each head repeated H / H_kv times."""
    if t.ndim != 4:
        raise ValueError("expected [B, H, N, d] arrays, got shape %r" % (t.shape,))
    H_kv = t.shape[1]
    if H_kv == H:
        return t
    if H_kv <= 0 or H % H_kv != 0:
        raise ValueError("key/value heads (%d) must divide query heads (%d)" % (H_kv, H))
    return np.ascontiguousarray(np.repeat(t, H // H_kv, axis=1))


def _reduce_kv(g: np.ndarray, H_kv: int) -> np.ndarray:
    """Gradient of a K or V head shared by a group: the sum over the group's
    repeated copies (chain rule through the repeat in _expand_kv)."""
    B, H, N, d = g.shape
    if H_kv == H:
        return g
    return np.ascontiguousarray(g.reshape(B, H_kv, H // H_kv, N, d).sum(axis=2))


def _as_f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch CPU tensor
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _shape(q):
    if q.ndim != 4:
        raise ValueError("expected [B, H, N, d] arrays, got shape %r" % (q.shape,))
    return q.shape
