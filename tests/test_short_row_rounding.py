"""CPU model of the 16-bit kernels' rounding on short rows, against the oracle.

With one or two visible keys, dP_ij - D_i is as small as the rounding error
of a 16-bit O, so a D taken as rowsum(dO o O) from the stored O passes that
error to dS, dQ and dK at full size: bf16 at N = 2 misses the 2e-2 limit on
several percent of seeds.  The half-precision rounding behind it is the
error source the article "Revolutionizing Web-Based AI: How a Plain
JavaScript Prototype Paved the Way for High-Performance WebGPU Flash
Attention 2" names in "Numerical Stability and Loss Drift", and its "The
JavaScript-First Methodology" has gradients checked against a reference.
The dQ kernels therefore take D = sum_j P_ij dP_ij in fp32 from the
first 32-key block for every row whose visible keys all lie in it.

This model follows the kernels' arithmetic for N <= 32 (one key block, so
the forward's running max is the row max), in float64 except where the
kernels round to the element type:
  forward   P = exp(S - max) rounded before P V; O = (sum_j round(P_j) v_j) /
            sum_j P_j, rounded; LSE = max + ln sum_j P_j
  backward  P = exp(S - LSE); dP = dO V^T; D as above (or, for the check
            that the model sees the effect, rowsum(dO o round(O)));
            dS = P (dP - D) rounded before dQ = scale dS K and
            dK = scale dS^T Q; P rounded before dV = P^T dO; dQ, dK, dV
            rounded.
Inputs are exactly those of the GPU edge tests (``workloads.custom(1, 2, N,
d, dtype, causal, seed)``); many seeds are stacked along the batch axis so
one oracle call covers them.  The error measure and limits are those of the
GPU parity tests.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

TOL = {"bf16": 2e-2, "f16": 2.5e-3}
SEEDS = range(1000)


def _round(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(workloads.TORCH_DTYPES[dtype]).double().numpy()


def _model(q, k, v, dO, scale, causal, dtype, d_from_block):
    N = q.shape[2]
    assert N <= 32, "the model covers one key block"
    s = np.einsum("bhid,bhjd->bhij", q, k)
    if causal:
        s = np.where(np.triu(np.ones((N, N), bool), 1), -np.inf, s)
    smax = s.max(-1, keepdims=True)
    p = np.exp((s - smax) * scale)
    lsum = p.sum(-1, keepdims=True)
    o = _round(np.einsum("bhij,bhjd->bhid", _round(p, dtype), v) / lsum, dtype)
    lse = (smax * scale + np.log(lsum))[..., 0]
    P = np.exp(s * scale - lse[..., None])
    dP = np.einsum("bhid,bhjd->bhij", dO, v)
    D = (P * dP).sum(-1) if d_from_block else (dO * o).sum(-1)
    dS = _round(P * (dP - D[..., None]), dtype)
    dq = _round(scale * np.einsum("bhij,bhjd->bhid", dS, k), dtype)
    dk = _round(scale * np.einsum("bhij,bhid->bhjd", dS, q), dtype)
    dv = _round(np.einsum("bhij,bhid->bhjd", _round(P, dtype), dO), dtype)
    return o, lse, dq, dk, dv


def _per_seed_err(a, r):
    """max|a - r| / max|r| per leading index (|a - r| where r is all 0)."""
    ax = tuple(range(1, r.ndim))
    diff = np.abs(a - r).max(axis=ax)
    den = np.abs(r).max(axis=ax)
    return np.where(den > 0, diff / np.where(den > 0, den, 1.0), diff)


def _errors(N, d, dtype, causal, seeds, d_from_block):
    ins = [workloads.make_inputs(workloads.custom(1, 2, N, d, dtype, causal, s, name="edge")) for s in seeds]
    q, k, v, dO = (np.concatenate([x[i].double().numpy() for x in ins]) for i in range(4))
    scale = 1.0 / np.sqrt(d)
    refs = oracle.fwd(q, k, v, scale, causal) + oracle.bwd(q, k, v, dO, scale, causal)
    outs = _model(q, k, v, dO, scale, causal, dtype, d_from_block)
    # one sequence of 2 heads per seed: regroup the stacked batch per seed
    return np.stack([_per_seed_err(a, r) for a, r in zip(outs, refs)]).max(axis=0)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_block_d_keeps_every_seed_within_tolerance(d, causal, dtype):
    for N in (1, 2, 3, 5, 8):
        e = _errors(N, d, dtype, causal, SEEDS, d_from_block=True)
        worst = int(np.argmax(e))
        assert e[worst] <= TOL[dtype], "N=%d seed %d: %.3g above %g" % (N, worst, e[worst], TOL[dtype])


@pytest.mark.parametrize("dtype,d,seed", [("bf16", 64, 90), ("bf16", 128, 17), ("f16", 64, 7)])
def test_rowsum_of_rounded_o_fails_the_named_seeds(dtype, d, seed):
    """The model does see the effect: with D = rowsum(dO o round(O)) these
    causal N = 2 cases exceed the limit, and with D from the block they
    do not.  (They are also GPU edge cases.)"""
    old = _errors(2, d, dtype, True, [seed], d_from_block=False)[0]
    new = _errors(2, d, dtype, True, [seed], d_from_block=True)[0]
    assert old > TOL[dtype] and new <= TOL[dtype], (old, new)
