"""Seeded synthetic inputs for attention forward and backward.

This module holds no attention arithmetic: it only draws random tensors.  The
GPU path, the oracle, the tests and the benchmark all take their inputs from
here, so both sides see bit-identical values.

The five workloads are the shapes named for this method: a tiny and a small
causal fp32 case, the fp32 shape whose N x N score tensor is the 67 MB the
article "Revolutionizing Web-Based AI: How a Plain JavaScript Prototype Paved
the Way for High-Performance WebGPU Flash Attention 2" (section "Memory
Bandwidth Optimization") says is no longer moved per layer and step, the
large bf16 causal case, and a ragged non-causal bf16 stress case whose Q and K
are scaled by 8 so the online-softmax maximum is rescaled often; a sixth is
the large case with grouped-query attention (2 key/value heads).

Recipe (identical for every workload): a CPU ``torch.Generator`` seeded with
the workload's seed draws ``torch.randn`` tensors of shape [B, H, N, d] in
float32, in the order q, k, v, dO.  Where ``qk_mult`` is not 1 (a power of two,
so exact), q and k are multiplied by it.  bf16 workloads then round every
tensor to bfloat16 (round to nearest even), f16 workloads to IEEE half
precision (round to nearest even).  Grouped-query cases (``H_kv``
key/value heads below H) draw k and v with shape [B, H_kv, N, d].  The oracle receives the same
tensors converted to float64, so input rounding is never counted as error.

Decoding workloads (``DecodeWorkload``: N_q new queries against a cache of
N_k keys) follow the same recipe with q [B, H, N_q, d] and k, v
[B, H_kv, N_k, d], drawn in the order q, k, v.
"""
from __future__ import annotations

import dataclasses
import math

import torch


TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "f32", "bf16" or "f16"
    causal: bool
    seed: int
    qk_mult: float = 1.0
    H_kv: int = 0  # key/value heads; 0 means H (plain multi-head attention)

    @property
    def kv_heads(self) -> int:
        return self.H_kv or self.H

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self) -> torch.dtype:
        return TORCH_DTYPES[self.dtype]

    def shape(self):
        return (self.B, self.H, self.N, self.d)

    def describe(self) -> str:
        return "%s B%d H%d%s N%d d%d %s %s" % (
            self.name, self.B, self.H, "" if self.kv_heads == self.H else "/kv%d" % self.kv_heads, self.N,
            self.d, self.dtype, "causal" if self.causal else "non-causal")


WORKLOADS = {
    1: Workload("tiny_causal_f32", 1, 2, 64, 16, "f32", True, 1),
    2: Workload("small_causal_f32", 4, 4, 256, 32, "f32", True, 2),
    3: Workload("mega_class_causal_f32", 8, 8, 512, 64, "f32", True, 3),
    4: Workload("large_causal_bf16", 4, 16, 4096, 128, "bf16", True, 4),
    5: Workload("ragged_noncausal_bf16", 16, 12, 1000, 64, "bf16", False, 5, 8.0),
    # Grouped-query variant of workload 4: 16 query heads over 2 key/value
    # heads (groups of 8).
    6: Workload("large_causal_gqa_bf16", 4, 16, 4096, 128, "bf16", True, 6, 1.0, 2),
    # Workload 4 in IEEE half precision.
    7: Workload("large_causal_f16", 4, 16, 4096, 128, "f16", True, 7),
}


def make_inputs(w: Workload, seed: int | None = None, device: str | torch.device = "cpu"):
    """Return (q, k, v, dO) for workload ``w`` on ``device`` in its dtype."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else int(seed))
    shp = w.shape()
    kv_shp = (w.B, w.kv_heads, w.N, w.d)
    q = torch.randn(shp, generator=g, dtype=torch.float32)
    k = torch.randn(kv_shp, generator=g, dtype=torch.float32)
    v = torch.randn(kv_shp, generator=g, dtype=torch.float32)
    dO = torch.randn(shp, generator=g, dtype=torch.float32)
    if w.qk_mult != 1.0:
        q = q * w.qk_mult
        k = k * w.qk_mult
    out = []
    for t in (q, k, v, dO):
        t = t.to(w.torch_dtype).contiguous()
        if str(device) != "cpu":
            t = t.to(device)
        out.append(t)
    return tuple(out)


def custom(B: int, H: int, N: int, d: int, dtype: str, causal: bool, seed: int,
           qk_mult: float = 1.0, name: str = "custom", H_kv: int = 0) -> Workload:
    """A workload outside the named five (edge-case shapes in the tests)."""
    return Workload(name, B, H, N, d, dtype, causal, seed, qk_mult, H_kv)


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    H: int
    H_kv: int
    N_q: int
    N_k: int
    d: int
    dtype: str
    causal: bool
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self) -> torch.dtype:
        return TORCH_DTYPES[self.dtype]

    def describe(self) -> str:
        return "%s B%d H%d/kv%d Nq%d Nk%d d%d %s %s" % (
            self.name, self.B, self.H, self.H_kv, self.N_q, self.N_k, self.d, self.dtype,
            "causal" if self.causal else "non-causal")


# One new token per sequence for 16 sequences of a 64-query-head model with 8
# key/value heads and a 16 K cache (a 1 GiB bf16 cache: far larger than the
# device's caches, so every pass reads it from HBM).
DECODE_WORKLOADS = {
    "decode_gqa_bf16": DecodeWorkload("decode_gqa_bf16", 16, 64, 8, 1, 16384, 128, "bf16", False, 7),
}


def make_decode_inputs(w: DecodeWorkload, seed: int | None = None, device: str | torch.device = "cpu"):
    """Return (q, k, v) for decoding workload ``w`` on ``device`` in its dtype."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else int(seed))
    q = torch.randn((w.B, w.H, w.N_q, w.d), generator=g, dtype=torch.float32)
    k = torch.randn((w.B, w.H_kv, w.N_k, w.d), generator=g, dtype=torch.float32)
    v = torch.randn((w.B, w.H_kv, w.N_k, w.d), generator=g, dtype=torch.float32)
    out = []
    for t in (q, k, v):
        t = t.to(w.torch_dtype).contiguous()
        if str(device) != "cpu":
            t = t.to(device)
        out.append(t)
    return tuple(out)


@dataclasses.dataclass(frozen=True)
class VarlenWorkload:
    """A packed ragged batch: sequences of the given lengths, one after the
    other along the token axis of every head ([H, T, d] tensors), with T rows
    per head (T >= the total length; rows past it belong to no sequence)."""
    name: str
    lengths: tuple
    H: int
    H_kv: int
    d: int
    dtype: str
    causal: bool
    seed: int
    qk_mult: float = 1.0
    T: int = 0  # 0: the total length

    @property
    def total(self) -> int:
        return self.T or sum(self.lengths)

    @property
    def max_seqlen(self) -> int:
        return max(self.lengths) if self.lengths else 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self) -> torch.dtype:
        return TORCH_DTYPES[self.dtype]

    def cu_seqlens(self) -> list:
        cu = [0]
        for n in self.lengths:
            cu.append(cu[-1] + n)
        return cu

    def describe(self) -> str:
        return "%s %d seqs (max %d, T %d) H%d/kv%d d%d %s %s" % (
            self.name, len(self.lengths), self.max_seqlen, self.total, self.H, self.H_kv, self.d, self.dtype,
            "causal" if self.causal else "non-causal")


def varlen_lengths(count: int, lo: int, hi: int, seed: int) -> tuple:
    """Sequence lengths drawn uniformly from [lo, hi] by a seeded CPU generator."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return tuple(int(x) for x in torch.randint(lo, hi + 1, (count,), generator=g))


# 16 sequences of 512 .. 4096 tokens (seeded), 16 heads, d = 128, causal
# bf16: the large workload's head shape with a length mix instead of one N.
VARLEN_WORKLOADS = {
    "varlen_causal_bf16": VarlenWorkload("varlen_causal_bf16", varlen_lengths(16, 512, 4096, 8), 16, 16, 128,
                                         "bf16", True, 8),
}


def make_varlen_inputs(w: VarlenWorkload, seed: int | None = None, device: str | torch.device = "cpu"):
    """Return (q, k, v, dO, cu_seqlens) for a packed workload: q, dO [H, T, d],
    k, v [H_kv, T, d] in its dtype, cu_seqlens int32 [B + 1]."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else int(seed))
    T = w.total
    q = torch.randn((w.H, T, w.d), generator=g, dtype=torch.float32)
    k = torch.randn((w.H_kv, T, w.d), generator=g, dtype=torch.float32)
    v = torch.randn((w.H_kv, T, w.d), generator=g, dtype=torch.float32)
    dO = torch.randn((w.H, T, w.d), generator=g, dtype=torch.float32)
    if w.qk_mult != 1.0:
        q = q * w.qk_mult
        k = k * w.qk_mult
    out = []
    for t in (q, k, v, dO):
        t = t.to(w.torch_dtype).contiguous()
        if str(device) != "cpu":
            t = t.to(device)
        out.append(t)
    cu = torch.tensor(w.cu_seqlens(), dtype=torch.int32)
    if str(device) != "cpu":
        cu = cu.to(device)
    out.append(cu)
    return tuple(out)
