"""fa2_backward_noalloc (the backward with the library's static per-GPU
workspace) against fa2_backward_ex with a caller-allocated workspace.

Three calls in a row share the one static buffer, each on a smaller
problem than the one before (the first, fp32 with split walks, fills most
of the buffer with fp32 partial sums that later calls must not pick up).
The same kernels run either way, so the outputs must be the same bits; the
error against the oracle is checked too, to the parity tests' limits.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import tiled_attention_fwd_amd as fa
import workloads

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 2.5e-3}

CASES = [
    # fp32, long causal walks split over workgroups: fp32 partials in the buffer
    workloads.custom(1, 2, 2048, 64, "f32", True, 8301, name="noalloc"),
    # grouped-query d = 128 bf16 (split groups: fp32 partial dK, dV)
    workloads.custom(2, 8, 1000, 128, "bf16", True, 8302, name="noalloc", H_kv=2),
    # small ragged non-causal fp16
    workloads.custom(1, 4, 333, 64, "f16", False, 8303, name="noalloc", H_kv=2),
]


def _rel(a, r):
    a = np.asarray(a, dtype=np.float64)
    den = float(np.max(np.abs(r)))
    return float(np.max(np.abs(a - r))) / den if den > 0 else float(np.max(np.abs(a - r)))


def test_noalloc_matches_backward_ex_on_calls_in_a_row():
    sizes = [fa.fa2_backward_workspace_size_ex(w.B, w.H, w.kv_heads, w.N, w.d, w.torch_dtype) for w in CASES]
    assert sizes == sorted(sizes, reverse=True) and sizes[0] <= fa.NOALLOC_SCRATCH_BYTES
    for w, nbytes in zip(CASES, sizes):
        print("case: %s seed=%d workspace %d bytes" % (w.describe(), w.seed, nbytes), flush=True)
        sys.stdout.flush()
        q, k, v, dO = workloads.make_inputs(w, device="cuda")
        o, lse = fa.forward(q, k, v, w.causal, w.scale)
        ref = fa.backward(q, k, v, o, lse, dO, w.causal, w.scale)
        out = [torch.full_like(q, float("nan")), torch.full_like(k, float("nan")), torch.full_like(v, float("nan"))]
        torch.cuda.synchronize()
        fa.fa2_backward_noalloc(q, k, v, o, dO, lse, *out, w.causal, w.scale)
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), out, ref):
            assert torch.equal(a, b), "%s: fa2_backward_noalloc differs from fa2_backward_ex" % name
        refs = oracle.bwd(q.cpu(), k.cpu(), v.cpu(), dO.cpu(), w.scale, w.causal)
        errs = [_rel(a.float().cpu().numpy(), r) for a, r in zip(out, refs)]
        print("  errors dQ=%.3g dK=%.3g dV=%.3g" % tuple(errs), flush=True)
        assert max(errs) <= TOL[w.dtype]


def test_noalloc_rejects_a_problem_beyond_its_buffer():
    """Rejected by the size check before any HIP call: nothing is launched."""
    assert fa.fa2_backward_workspace_size_ex(64, 64, 64, 4096, 128, torch.bfloat16) > fa.NOALLOC_SCRATCH_BYTES
    t = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    st = fa.lib().fa2_backward_noalloc(*([t.data_ptr()] * 9), 64, 64, 64, 4096, 128, 0.125, 1, fa.FA2_BF16, None)
    assert st == fa.FA2_ERR_SCRATCH
