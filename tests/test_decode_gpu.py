"""GPU parity of decoding (N_q new queries against an N_k cache) against the
fp64 oracle's ``decode``.

Same error measure and limits as the forward and backward parity tests
(err = max|gpu - oracle| / max|oracle|, 2e-2 for bf16 inputs with fp32
accumulation); outputs are NaN-filled inside canary guard bands before the
call.  The cases cover the direct path (one chunk) and the split path (a
partial result per chunk and the merge kernel), ragged caches, more than 32
rows per key/value head, causal rows that see no key of a chunk, the
full-size decoding workload on sampled heads, and the other types and head
sizes, which run the generic forward kernel (float32 limit 1e-4).
"""
import pytest
import torch

import oracle
import tiled_attention_fwd_amd as fa
import workloads
from tests.test_parity_gpu import Guarded, log, rel_err

pytestmark = pytest.mark.gpu

# bf16 as stated for the method; fp16 derived from it (unit roundoff 2^-11
# against 2^-8: 2e-2 * 2^-3).
TOL = {"bf16": 2e-2, "f16": 2.5e-3, "f32": 1e-4}


def gpu_decode(q, k, v, causal, scale):
    B, H, Nq, d = q.shape
    o = Guarded(q.shape, q.dtype)
    lse = Guarded((B, H, Nq), torch.float32)
    fa.fa2_decode(q, k, v, o.t, lse.t, causal, scale)
    torch.cuda.synchronize()
    assert o.guards_intact(), "O: write outside the output tensor"
    assert lse.guards_intact(), "LSE: write outside the output tensor"
    return o.t, lse.t


def run_decode_case(w, heads=None, scale=None):
    """heads: (b, key/value head) pairs to compare (with their query heads);
    None compares everything.  scale: the factor on q . k (default: the
    workload's)."""
    scale = w.scale if scale is None else scale
    log("decode case: %s seed=%d scale=%g" % (w.describe(), w.seed, scale))
    q, k, v = workloads.make_decode_inputs(w, device="cuda")
    o, lse = gpu_decode(q, k, v, w.causal, scale)
    o, lse = o.float().cpu(), lse.cpu()
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    G = w.H // w.H_kv
    sel = [(slice(None), slice(None), slice(None))] if heads is None else \
        [(slice(b, b + 1), slice(h * G, (h + 1) * G), slice(h, h + 1)) for b, h in heads]
    eo = el = 0.0
    for bs, hs, ks in sel:
        o_r, lse_r = oracle.decode(qc[bs, hs], kc[bs, ks], vc[bs, ks], scale, w.causal)
        eo = max(eo, rel_err(o[bs, hs], o_r))
        el = max(el, rel_err(lse[bs, hs], lse_r))
    log("  errors: O=%.3g LSE=%.3g" % (eo, el))
    tol = TOL[w.dtype]
    assert eo <= tol and el <= tol, (w.describe(), eo, el)
    return o, lse


def dw(B, H, H_kv, Nq, Nk, causal, seed, dtype="bf16"):
    return workloads.DecodeWorkload("decode", B, H, H_kv, Nq, Nk, 128, dtype, causal, seed)


DECODE_CASES = [
    # split cache (8 chunks of 128 keys), ragged end, grouped heads
    (2, 8, 2, 1, 1000, False),
    (2, 8, 2, 4, 1000, True),
    # one chunk (direct output), ragged
    (1, 4, 4, 3, 70, True),
    (1, 2, 1, 1, 1, False),
    (1, 3, 1, 2, 33, True),
    # 100 rows (4 row blocks); rows i < 20 see no key of the last chunk
    (1, 1, 1, 100, 1040, True),
    # 64 rows per key/value head (groups of 8, 8 queries), split
    (3, 16, 2, 8, 2049, True),
    # N_q = N_k: the square causal pass
    (1, 8, 8, 16, 16, True),
    # many chunks (32 x 128 keys)
    (2, 6, 3, 5, 4096, False),
    # plain multi-head (one query head per cache head), split
    (4, 8, 8, 1, 3000, True),
]


@pytest.mark.parametrize("B,H,H_kv,Nq,Nk,causal", DECODE_CASES)
def test_decode_parity(B, H, H_kv, Nq, Nk, causal):
    seed = 4000 + 7 * B + 13 * H + H_kv + 31 * Nq + Nk + (1 if causal else 0)
    run_decode_case(dw(B, H, H_kv, Nq, Nk, causal, seed))


@pytest.mark.parametrize("B,H,H_kv,Nq,Nk,causal", [(2, 8, 2, 4, 1000, True), (1, 1, 1, 100, 1040, True),
                                                    (1, 3, 1, 2, 33, True), (2, 6, 3, 5, 4096, False)])
def test_decode_parity_f16(B, H, H_kv, Nq, Nk, causal):
    seed = 4200 + 7 * B + 13 * H + H_kv + 31 * Nq + Nk + (1 if causal else 0)
    run_decode_case(dw(B, H, H_kv, Nq, Nk, causal, seed, "f16"))


# The 16-bit types at d = 64 take the split-cache kernel on 128-byte rows;
# other types and head sizes the generic forward kernel with the cache as its
# keys (no split).
GENERIC_CASES = [
    (2, 4, 2, 1, 700, 64, "bf16", False),
    (1, 6, 3, 5, 300, 64, "f16", True),
    (2, 2, 1, 3, 129, 32, "f32", True),
    (1, 3, 3, 16, 16, 16, "f32", True),
    (1, 8, 2, 40, 1000, 128, "f32", False),
    (1, 2, 2, 200, 70, 64, "bf16", False),  # more queries than keys, no mask
    (4, 16, 2, 1, 9000, 64, "bf16", True),  # long cache: split into chunks
    (2, 16, 1, 3, 4133, 64, "f16", True),   # 48 rows per key/value head: two row blocks
]


@pytest.mark.parametrize("B,H,H_kv,Nq,Nk,d,dtype,causal", GENERIC_CASES)
def test_decode_parity_generic(B, H, H_kv, Nq, Nk, d, dtype, causal):
    seed = 4300 + 7 * B + 13 * H + H_kv + 31 * Nq + Nk + d + (1 if causal else 0)
    run_decode_case(workloads.DecodeWorkload("decode", B, H, H_kv, Nq, Nk, d, dtype, causal, seed))


# A negative factor on q . k: the split-cache kernel (d = 128 and 64) and the
# generic forward kernel decoding run it as |scale| * (-q) . k.
@pytest.mark.parametrize("B,H,H_kv,Nq,Nk,d,dtype,causal", [
    (2, 8, 2, 4, 1000, 128, "bf16", True),
    (1, 6, 3, 5, 300, 64, "f16", True),
    (2, 2, 1, 3, 129, 32, "f32", True),
])
def test_decode_negative_scale(B, H, H_kv, Nq, Nk, d, dtype, causal):
    seed = 4400 + 7 * B + 13 * H + H_kv + 31 * Nq + Nk + d
    run_decode_case(workloads.DecodeWorkload("decode", B, H, H_kv, Nq, Nk, d, dtype, causal, seed),
                    scale=-0.9 / d ** 0.5)


def test_decode_workload_sampled_heads():
    """The decoding workload at full size (16 sequences, 64 query heads over
    8 key/value heads, one query against a 16 K cache), as the benchmark
    runs it, on three key/value heads with their 8 query heads each."""
    run_decode_case(workloads.DECODE_WORKLOADS["decode_gqa_bf16"], heads=[(0, 0), (7, 3), (15, 7)])


def test_decode_square_matches_forward():
    """N_q = N_k causal decoding is the causal forward pass."""
    w = dw(1, 4, 4, 300, 300, True, 4101)
    q, k, v = workloads.make_decode_inputs(w, device="cuda")
    o, lse = gpu_decode(q, k, v, True, w.scale)
    of, lf = fa.forward(q, k, v, True, w.scale)
    torch.cuda.synchronize()
    assert rel_err(o.float().cpu(), of.float().cpu()) < TOL["bf16"]
    assert rel_err(lse.cpu(), lf.cpu()) < TOL["bf16"]


def test_decode_bitwise_repeatable():
    w = dw(2, 8, 2, 3, 3000, True, 4102)
    q, k, v = workloads.make_decode_inputs(w, device="cuda")
    a = fa.decode(q, k, v, True, w.scale)
    b = fa.decode(q, k, v, True, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_rejects_on_gpu():
    q = torch.zeros((1, 2, 4, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 2, 3, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.Fa2Error):  # causal with more queries than keys
        fa.decode(q, k, k, True)
    q48 = torch.zeros((1, 2, 1, 48), dtype=torch.float16, device="cuda")
    with pytest.raises(fa.Fa2Error):  # head size outside 16, 32, 64, 128
        fa.decode(q48, q48, q48, False)
