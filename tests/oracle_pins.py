"""Checks that pin the fp64 oracle to facts outside itself.

Each ``pin_*`` function takes an oracle object (``oracle.Oracle``: the shipped
library or a deliberately broken copy built by the mutation tests) and raises
AssertionError when the oracle disagrees with:

* a library routine that is independent of it (torch's float64
  ``scaled_dot_product_attention`` and autograd, ``torch.logsumexp``);
* closed forms of special cases (Q = 0 gives uniform weights, N = 1, two
  keys reduce softmax to the logistic function, causal row 0 sees one key);
* invariants of softmax attention (weights sum to one, key-shift invariance
  of the logits, permutation equivariance without a mask);
* central finite differences of the scalar loss L = sum(O * dO), which pins
  the backward to the forward.

The article "Revolutionizing Web-Based AI: How a Plain JavaScript Prototype
Paved the Way for High-Performance WebGPU Flash Attention 2" (section "The
JavaScript-First Methodology") describes the same discipline for its own
reference: check the online-softmax state and the gradients before any
shader is trusted.  The article prints no worked example with values, so no
pin here reproduces a printed number.
"""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F


def rel_err(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    denom = float(np.max(np.abs(b))) if b.size else 0.0
    with np.errstate(invalid="ignore"):  # inf - inf from a broken oracle: reported as inf below
        diff = float(np.max(np.abs(a - b))) if a.size else 0.0
    if not np.isfinite(diff):
        return float("inf")
    if denom == 0.0:
        return diff
    return diff / denom


def randn(shape, seed, mult=1.0):
    g = np.random.default_rng(seed)
    return g.standard_normal(shape) * mult


# --------------------------------------------------------------------------
# library routine: torch float64 SDPA + autograd, torch.logsumexp
# --------------------------------------------------------------------------
def torch_reference(q, k, v, dO, scale, causal):
    qt = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    vt = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    gqa = kt.shape[1] != qt.shape[1]
    o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=scale, enable_gqa=gqa)
    (o * torch.tensor(dO, dtype=torch.float64)).sum().backward()
    with torch.no_grad():
        kx = kt.repeat_interleave(qt.shape[1] // kt.shape[1], dim=1) if gqa else kt
        logits = scale * torch.matmul(qt, kx.transpose(-1, -2).contiguous())
        if causal:
            n = q.shape[-2]
            mask = torch.ones(n, n, dtype=torch.bool).triu(1)
            logits = logits.masked_fill(mask, float("-inf"))
        lse = torch.logsumexp(logits, dim=-1)
    return (o.detach().numpy(), lse.numpy(), qt.grad.numpy(), kt.grad.numpy(),
            vt.grad.numpy())


def pin_torch(orc, q, k, v, dO, scale, causal, tol=1e-10):
    o_ref, lse_ref, dq_ref, dk_ref, dv_ref = torch_reference(q, k, v, dO, scale, causal)
    o, lse = orc.fwd(q, k, v, scale, causal)
    dq, dk, dv = orc.bwd(q, k, v, dO, scale, causal)
    errs = {
        "O": rel_err(o, o_ref), "LSE": rel_err(lse, lse_ref), "dQ": rel_err(dq, dq_ref),
        "dK": rel_err(dk, dk_ref), "dV": rel_err(dv, dv_ref),
    }
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, "oracle vs torch float64 SDPA: %r (tol %g)" % (bad, tol)
    return errs


# --------------------------------------------------------------------------
# closed forms and special cases
# --------------------------------------------------------------------------
def pin_uniform_v(orc, seed=11, causal=True):
    """Every V row equal to one vector u: each output row is u, because the
    attention weights of a row sum to one."""
    B, H, N, d = 2, 3, 37, 8
    q, k = randn((B, H, N, d), seed), randn((B, H, N, d), seed + 1)
    u = randn((B, H, 1, d), seed + 2)
    v = np.broadcast_to(u, (B, H, N, d)).copy()
    o, _ = orc.fwd(q, k, v, 1.0 / math.sqrt(d), causal)
    err = rel_err(o, v)
    assert err < 1e-12, "rows of P do not sum to 1: O differs from the common V row by %g" % err


def pin_direct_lse(orc, seed=12, causal=True):
    """LSE equals ln(sum_j exp(S_ij)) taken without the max shift (safe at
    these magnitudes): pins the natural-log convention and the scaling."""
    B, H, N, d = 1, 2, 29, 16
    scale = 0.3
    q, k, v = (randn((B, H, N, d), seed + t) for t in range(3))
    _, lse = orc.fwd(q, k, v, scale, causal)
    S = scale * np.einsum("bhid,bhjd->bhij", q, k)
    E = np.exp(S)
    if causal:
        E = E * np.tril(np.ones((N, N)))
    direct = np.log(E.sum(axis=-1))
    err = rel_err(lse, direct)
    assert err < 1e-12, "LSE differs from the direct log-sum-exp by %g" % err


def pin_causal_row0(orc, seed=13):
    """Causal row 0 attends to key 0 only: O_0 = V_0 and LSE_0 = S_00."""
    B, H, N, d = 2, 2, 19, 8
    scale = 0.25
    q, k, v = (randn((B, H, N, d), seed + t) for t in range(3))
    o, lse = orc.fwd(q, k, v, scale, True)
    assert np.array_equal(o[:, :, 0, :], v[:, :, 0, :]), "causal row 0 is not V_0"
    s00 = scale * np.sum(q[:, :, 0, :] * k[:, :, 0, :], axis=-1)
    assert rel_err(lse[:, :, 0], s00) < 1e-14, "causal LSE_0 is not S_00"


def pin_q_zero(orc, seed=14):
    """Q = 0 makes every weight of a row equal: O_i is the mean of the
    visible V rows, LSE_i = ln(number of visible keys), and dK = 0."""
    B, H, N, d = 1, 2, 23, 4
    q = np.zeros((B, H, N, d))
    k, v, dO = (randn((B, H, N, d), seed + t) for t in range(3))
    for causal in (True, False):
        o, lse = orc.fwd(q, k, v, 0.5, causal)
        _, dk, _ = orc.bwd(q, k, v, dO, 0.5, causal)
        counts = np.arange(1, N + 1) if causal else np.full(N, N)
        if causal:
            mean = np.cumsum(v, axis=2) / counts[None, None, :, None]
        else:
            mean = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
        assert rel_err(o, mean) < 1e-12, "Q=0: O is not the mean of visible V rows"
        assert rel_err(lse, np.broadcast_to(np.log(counts), lse.shape)) < 1e-14, \
            "Q=0: LSE is not ln(count)"
        assert np.max(np.abs(dk)) == 0.0, "Q=0: dK must be exactly zero"


def pin_single_key(orc, seed=15):
    """N = 1: O = V, LSE = S_00, dQ = dK = 0 (a one-key softmax is constant),
    dV = dO."""
    B, H, N, d = 3, 2, 1, 8
    q, k, v, dO = (randn((B, H, N, d), seed + t) for t in range(4))
    for causal in (True, False):
        o, lse = orc.fwd(q, k, v, 0.7, causal)
        dq, dk, dv = orc.bwd(q, k, v, dO, 0.7, causal)
        assert np.array_equal(o, v)
        assert rel_err(lse, 0.7 * np.sum(q * k, axis=-1)) < 1e-14
        assert np.max(np.abs(dq)) == 0.0 and np.max(np.abs(dk)) == 0.0
        assert np.array_equal(dv, dO)


def pin_two_keys(orc, seed=16):
    """Two keys, no mask: the weight of key 0 is the logistic function of
    S_i0 - S_i1, and the gradients take the logistic-derivative form
    dS_i0 = -dS_i1 = p0 p1 (dP_i0 - dP_i1)."""
    B, H, N, d = 1, 3, 2, 5
    scale = 0.4
    q, k, v, dO = (randn((B, H, N, d), seed + t) for t in range(4))
    o, lse = orc.fwd(q, k, v, scale, False)
    dq, dk, dv = orc.bwd(q, k, v, dO, scale, False)
    s0 = scale * np.sum(q * k[:, :, 0:1, :], axis=-1)  # [B,H,N]
    s1 = scale * np.sum(q * k[:, :, 1:2, :], axis=-1)
    p0 = 1.0 / (1.0 + np.exp(s1 - s0))
    p1 = 1.0 - p0
    o_cf = p0[..., None] * v[:, :, 0:1, :] + p1[..., None] * v[:, :, 1:2, :]
    lse_cf = s0 + np.log1p(np.exp(s1 - s0))
    assert rel_err(o, o_cf) < 1e-13, "two keys: O differs from the logistic form"
    assert rel_err(lse, lse_cf) < 1e-13, "two keys: LSE differs from the logistic form"
    dp0 = np.sum(dO * v[:, :, 0:1, :], axis=-1)
    dp1 = np.sum(dO * v[:, :, 1:2, :], axis=-1)
    g = p0 * p1 * (dp0 - dp1)  # dS_i0; dS_i1 = -g
    dq_cf = scale * g[..., None] * (k[:, :, 0:1, :] - k[:, :, 1:2, :])
    dk0 = scale * np.sum(g[..., None] * q, axis=2)
    dv0 = np.sum(p0[..., None] * dO, axis=2)
    dv1 = np.sum(p1[..., None] * dO, axis=2)
    assert rel_err(dq, dq_cf) < 1e-12, "two keys: dQ differs from the logistic form"
    assert rel_err(dk[:, :, 0, :], dk0) < 1e-12 and rel_err(dk[:, :, 1, :], -dk0) < 1e-12, \
        "two keys: dK differs from the logistic form"
    assert rel_err(dv[:, :, 0, :], dv0) < 1e-12 and rel_err(dv[:, :, 1, :], dv1) < 1e-12, \
        "two keys: dV differs from the logistic form"


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------
def pin_invariants(orc, seed=17, causal=True, N=41, d=8):
    """Per (b, h): sum_j dK_j = 0 (adding one vector to every key shifts a
    row's logits by a constant, which softmax ignores), sum_j dV_j = sum_i dO_i
    (rows of P sum to one), and D_i = sum_j P_ij dP_ij equals rowsum(dO * O)."""
    B, H = 2, 2
    q, k, v, dO = (randn((B, H, N, d), seed + t) for t in range(4))
    o, _ = orc.fwd(q, k, v, 0.35, causal)
    dq, dk, dv, delta = orc.bwd(q, k, v, dO, 0.35, causal, return_delta=True)
    sk = np.abs(dk.sum(axis=2)).max() / max(np.abs(dk).max(), 1e-300)
    assert sk < 1e-12, "sum_j dK_j is not zero (relative %g)" % sk
    assert rel_err(dv.sum(axis=2), dO.sum(axis=2)) < 1e-12, "sum_j dV_j != sum_i dO_i"
    assert rel_err(delta, np.sum(dO * o, axis=-1)) < 1e-12, "D != rowsum(dO * O)"


def pin_permutation(orc, seed=18):
    """Without a mask, permuting the rows of K and V together leaves O and
    LSE unchanged, and permutes dK and dV the same way."""
    B, H, N, d = 1, 2, 17, 8
    q, k, v, dO = (randn((B, H, N, d), seed + t) for t in range(4))
    perm = np.random.default_rng(seed).permutation(N)
    o, lse = orc.fwd(q, k, v, 0.3, False)
    o2, lse2 = orc.fwd(q, k[:, :, perm], v[:, :, perm], 0.3, False)
    assert rel_err(o2, o) < 1e-13 and rel_err(lse2, lse) < 1e-13
    _, dk, dv = orc.bwd(q, k, v, dO, 0.3, False)
    _, dk2, dv2 = orc.bwd(q, k[:, :, perm], v[:, :, perm], dO, 0.3, False)
    assert rel_err(dk2, dk[:, :, perm]) < 1e-12 and rel_err(dv2, dv[:, :, perm]) < 1e-12


# --------------------------------------------------------------------------
# finite differences
# --------------------------------------------------------------------------
def pin_finite_diff(orc, shape=(1, 1, 6, 3), causal=True, seed=19, sample=None, tol=1e-6):
    """Central differences (h = 1e-6) of L = sum(O * dO) against dQ, dK, dV.
    ``sample``: None checks every element, else that many seeded elements per
    tensor."""
    q, k, v, dO = (randn(shape, seed + t) for t in range(4))
    scale = 1.0 / math.sqrt(shape[-1])
    grads = orc.bwd(q, k, v, dO, scale, causal)
    h = 1e-6
    rng = np.random.default_rng(seed)

    def loss(qq, kk, vv):
        o, _ = orc.fwd(qq, kk, vv, scale, causal)
        return float(np.sum(o * dO))

    worst = 0.0
    for which, g in enumerate(grads):
        base = [q, k, v]
        n = g.size
        idx = range(n) if sample is None else rng.choice(n, size=min(sample, n), replace=False)
        num = np.empty(len(idx))
        ana = np.empty(len(idx))
        for t, flat in enumerate(idx):
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which].flat[flat] += h
            minus[which].flat[flat] -= h
            num[t] = (loss(*plus) - loss(*minus)) / (2 * h)
            ana[t] = g.flat[flat]
        err = rel_err(ana, num)
        worst = max(worst, err)
        assert err < tol, "finite differences disagree with %s (rel %g)" % ("dQ dK dV".split()[which], err)
    return worst


# --------------------------------------------------------------------------
# grouped-query attention (the article's "Next Frontiers in WebGPU ML",
# "Broader Opset Support", names it; query head h reads K, V head h // G)
# --------------------------------------------------------------------------
def pin_gqa_torch(orc):
    """GQA (H=4 over 2 K/V heads, causal) and MQA (H=3 over 1, unmasked)
    against torch float64 SDPA with enable_gqa and autograd."""
    q, g = randn((2, 4, 19, 8), 40), randn((2, 4, 19, 8), 41)
    k, v = randn((2, 2, 19, 8), 42), randn((2, 2, 19, 8), 43)
    pin_torch(orc, q, k, v, g, 0.35, True)
    q, g = randn((1, 3, 12, 4), 44), randn((1, 3, 12, 4), 45)
    k, v = randn((1, 1, 12, 4), 46), randn((1, 1, 12, 4), 47)
    pin_torch(orc, q, k, v, g, 0.5, False)


def pin_gqa_shared_heads(orc, seed=48, H=3, N=9, d=4):
    """MQA with every query head equal and every dO head equal: each output
    head is the single-head result, and the shared K, V receive the sum of
    the heads' gradients, i.e. H times the single-head dK, dV."""
    q1, g1 = randn((1, 1, N, d), seed), randn((1, 1, N, d), seed + 1)
    k, v = randn((1, 1, N, d), seed + 2), randn((1, 1, N, d), seed + 3)
    q, g = np.repeat(q1, H, axis=1), np.repeat(g1, H, axis=1)
    o1, l1 = orc.fwd(q1, k, v, 0.4, True)
    dq1, dk1, dv1 = orc.bwd(q1, k, v, g1, 0.4, True)
    o, lse = orc.fwd(q, k, v, 0.4, True)
    dq, dk, dv = orc.bwd(q, k, v, g, 0.4, True)
    assert dk.shape == k.shape and dv.shape == v.shape
    for h in range(H):
        assert rel_err(o[:, h:h + 1], o1) < 1e-14 and rel_err(lse[:, h:h + 1], l1) < 1e-14
        assert rel_err(dq[:, h:h + 1], dq1) < 1e-14
    assert rel_err(dk, H * dk1) < 1e-13 and rel_err(dv, H * dv1) < 1e-13


# --------------------------------------------------------------------------
# decoding: N_q new queries against an N_k cache (the article's "Next
# Frontiers in WebGPU ML", "Broader Opset Support", names flash-decoding);
# causal places the queries at the last N_q positions of the sequence
# --------------------------------------------------------------------------
def torch_decode_reference(q, k, v, scale, causal):
    """(O, LSE) from torch float64 SDPA with an explicit boolean mask that
    keeps key j for query i when j <= N_k - N_q + i."""
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64) for x in (q, k, v))
    Nq, Nk = qt.shape[2], kt.shape[2]
    gqa = kt.shape[1] != qt.shape[1]
    mask = None
    if causal:
        i = torch.arange(Nq).unsqueeze(1)
        j = torch.arange(Nk).unsqueeze(0)
        mask = j <= i + (Nk - Nq)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale, enable_gqa=gqa)
    kx = kt.repeat_interleave(qt.shape[1] // kt.shape[1], dim=1) if gqa else kt
    logits = scale * torch.matmul(qt, kx.transpose(-1, -2).contiguous())
    if causal:
        logits = logits.masked_fill(~mask, float("-inf"))
    return o.numpy(), torch.logsumexp(logits, dim=-1).numpy()


def pin_decode_torch(orc):
    """Single query, a few queries (causal and not) and grouped heads against
    torch float64 SDPA with the bottom-right mask written out."""
    for (B, H, Hkv, Nq, Nk, d, causal, sd) in [(1, 2, 2, 1, 37, 8, True, 50), (2, 2, 2, 5, 40, 8, True, 51),
                                               (1, 3, 3, 7, 23, 4, False, 52), (2, 4, 2, 3, 29, 8, True, 53),
                                               (1, 4, 1, 16, 16, 8, True, 54)]:
        q = randn((B, H, Nq, d), sd)
        k, v = randn((B, Hkv, Nk, d), sd + 100), randn((B, Hkv, Nk, d), sd + 200)
        o, lse = orc.decode(q, k, v, 0.45, causal)
        o_t, lse_t = torch_decode_reference(q, k, v, 0.45, causal)
        assert rel_err(o, o_t) < 1e-12, ("O", Nq, Nk, causal)
        assert rel_err(lse, lse_t) < 1e-12, ("LSE", Nq, Nk, causal)


def pin_decode_suffix(orc, seed=55, N=24, Nq=6, d=4):
    """The last N_q rows of causal attention over a whole sequence are the
    decode of those N_q queries against the sequence's keys."""
    q, k, v = randn((1, 2, N, d), seed), randn((1, 2, N, d), seed + 1), randn((1, 2, N, d), seed + 2)
    o_full, lse_full = orc.fwd(q, k, v, 0.5, True)
    o, lse = orc.decode(q[:, :, N - Nq:], k, v, 0.5, True)
    assert rel_err(o, o_full[:, :, N - Nq:]) < 1e-13
    assert rel_err(lse, lse_full[:, :, N - Nq:]) < 1e-13


def pin_decode_merge(orc, seed=56, Nq=3, Nk=31, cut=12, d=5):
    """Attention over a cache split in two parts equals the LSE-weighted
    merge of the attention over each part (the identity split-KV decoding
    rests on): O = (e^L1 O1 + e^L2 O2) / (e^L1 + e^L2), LSE = log(e^L1 + e^L2)."""
    q = randn((1, 2, Nq, d), seed)
    k, v = randn((1, 2, Nk, d), seed + 1), randn((1, 2, Nk, d), seed + 2)
    o, lse = orc.decode(q, k, v, 0.6, False)
    o1, l1 = orc.decode(q, k[:, :, :cut], v[:, :, :cut], 0.6, False)
    o2, l2 = orc.decode(q, k[:, :, cut:], v[:, :, cut:], 0.6, False)
    lm = np.logaddexp(l1, l2)
    w1, w2 = np.exp(l1 - lm)[..., None], np.exp(l2 - lm)[..., None]
    assert rel_err(lse, lm) < 1e-13
    assert rel_err(o, w1 * o1 + w2 * o2) < 1e-13


def pin_decode_q_zero(orc, seed=57, Nq=4, Nk=10, d=3):
    """Q = 0: uniform weights over the visible keys, N_k - N_q + i + 1 of them
    for causal query i (all N_k otherwise)."""
    v = randn((1, 1, Nk, d), seed)
    k = randn((1, 1, Nk, d), seed + 1)
    q = np.zeros((1, 1, Nq, d))
    for causal in (True, False):
        o, lse = orc.decode(q, k, v, 0.7, causal)
        for i in range(Nq):
            n = Nk - Nq + i + 1 if causal else Nk
            assert np.allclose(o[0, 0, i], v[0, 0, :n].mean(axis=0), rtol=0, atol=1e-14)
            assert abs(lse[0, 0, i] - math.log(n)) < 1e-14
    o1, l1 = orc.decode(randn((1, 1, 1, d), seed + 2), k, v, 0.7, True)
    o2, l2 = orc.decode(randn((1, 1, 1, d), seed + 2), k, v, 0.7, False)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)  # one query sees the whole cache


ALL_SMALL_PINS = [
    pin_uniform_v, pin_direct_lse, pin_causal_row0, pin_q_zero, pin_single_key, pin_two_keys,
    pin_invariants, pin_permutation,
    lambda orc: pin_finite_diff(orc, (1, 1, 6, 3), True),
    lambda orc: pin_finite_diff(orc, (1, 1, 5, 2), False),
    lambda orc: pin_torch(orc, *(randn((1, 2, 33, 8), 20 + t) for t in range(4)), 0.35, True),
    lambda orc: pin_torch(orc, *(randn((1, 2, 33, 8), 30 + t) for t in range(4)), 0.35, False),
    pin_gqa_torch, pin_gqa_shared_heads,
    pin_decode_torch, pin_decode_suffix, pin_decode_merge, pin_decode_q_zero,
]
