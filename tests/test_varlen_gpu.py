"""GPU parity of packed ragged batches (variable-length sequences, [H, T, d]
tensors with sequence offsets cu_seqlens) against the fp64 oracle.

Each sequence is compared with the oracle run on that sequence alone (a
[1, H, n, d] problem), with the same error measure and limits as the
fixed-length tests.  Outputs are NaN-filled inside canary guard bands, and
rows that belong to no sequence must come back untouched.  A batch of equal
lengths must give exactly the bits of the fixed-length calls.
"""

import pytest
import torch

import oracle
import tiled_attention_fwd_amd as fa
import workloads
from tests.test_parity_gpu import TOL, Guarded, log, rel_err

pytestmark = pytest.mark.gpu


def gpu_varlen(w, q, k, v, dO, cu, scale):
    H, T, d = q.shape
    o = Guarded(q.shape, q.dtype)
    lse = Guarded((H, T), torch.float32)
    fa.fa2_forward_varlen(q, k, v, o.t, lse.t, cu, w.max_seqlen, w.causal, scale)
    dq = Guarded(q.shape, q.dtype)
    dk, dv = Guarded(k.shape, q.dtype), Guarded(k.shape, q.dtype)
    fa.fa2_backward_varlen(q, k, v, o.t, dO, lse.t, dq.t, dk.t, dv.t, cu, w.max_seqlen, w.causal, scale)
    torch.cuda.synchronize()
    for g, name in ((o, "O"), (lse, "LSE"), (dq, "dQ"), (dk, "dK"), (dv, "dV")):
        assert g.guards_intact(), "%s: write outside the output tensor" % name
    return o.t, lse.t, dq.t, dk.t, dv.t


def run_varlen_case(w, seqs=None, scale=None):
    """seqs: indices of the sequences to compare (None: all); scale: the
    factor on q . k (default: the workload's)."""
    scale = w.scale if scale is None else scale
    log("varlen case: %s seed=%d lengths=%s scale=%g" % (w.describe(), w.seed, list(w.lengths), scale))
    q, k, v, dO, cu = workloads.make_varlen_inputs(w, device="cuda")
    outs = gpu_varlen(w, q, k, v, dO, cu, scale)
    o, lse, dq, dk, dv = (t.float().cpu() for t in outs)
    qc, kc, vc, gc = (t.cpu() for t in (q, k, v, dO))
    offs = w.cu_seqlens()
    errs = {n: 0.0 for n in ("O", "LSE", "dQ", "dK", "dV")}
    for b in (range(len(w.lengths)) if seqs is None else seqs):
        s, e = offs[b], offs[b + 1]
        if e == s:
            continue
        sl = lambda t: t[:, s:e].unsqueeze(0)  # noqa: E731  [1, heads, n, d]
        o_r, lse_r = oracle.fwd(sl(qc), sl(kc), sl(vc), scale, w.causal)
        dq_r, dk_r, dv_r = oracle.bwd(sl(qc), sl(kc), sl(vc), sl(gc), scale, w.causal)
        for name, a, r in (("O", sl(o), o_r), ("LSE", lse[:, s:e].unsqueeze(0), lse_r), ("dQ", sl(dq), dq_r),
                           ("dK", sl(dk), dk_r), ("dV", sl(dv), dv_r)):
            errs[name] = max(errs[name], rel_err(a, r))
    log("  errors: " + " ".join("%s=%.3g" % kv for kv in errs.items()))
    tol = TOL[w.dtype]
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, "%s exceeds tolerance %g: %r" % (w.describe(), tol, bad)
    # every row of every sequence was written (the outputs start as NaN),
    # in the sequences compared above and in the others
    for name, t in (("O", o), ("LSE", lse), ("dQ", dq), ("dK", dk), ("dV", dv)):
        assert torch.isfinite(t[:, offs[0]:offs[-1]]).all(), "%s: rows of a sequence were not written" % name
    # rows past the last sequence are no sequence's: still NaN
    tail = offs[-1]
    if tail < w.total:
        for name, t in (("O", o), ("LSE", lse), ("dQ", dq), ("dK", dk), ("dV", dv)):
            assert torch.isnan(t[:, tail:]).all(), "%s: rows outside every sequence were written" % name


def vw(lengths, H, H_kv, d, dtype, causal, seed, T=0, qk_mult=1.0):
    return workloads.VarlenWorkload("varlen", tuple(lengths), H, H_kv, d, dtype, causal, seed, qk_mult, T)


VARLEN_CASES = [
    # lengths around the 32/64/128 tile edges, an empty sequence, bf16 generic kernels
    ([1, 17, 128, 129, 300, 0, 64], 2, 2, 64, "bf16", True),
    ([1, 17, 128, 129, 300, 0, 64], 2, 2, 32, "f32", False),
    # d = 128 16-bit kernels with grouped heads (the dK/dV stage splits the group)
    ([1000, 33, 512], 4, 2, 128, "bf16", True),
    ([700, 1, 257], 4, 1, 128, "f16", False),
    ([5, 130, 0, 0, 999], 3, 3, 16, "f32", True),
    ([2049, 64, 640], 2, 2, 128, "bf16", False),
    # grouped heads in fp32 at d = 128 (generic kernels), and fp16 at d = 64
    ([300, 1, 129, 77], 4, 2, 128, "f32", True),
    ([513, 31], 6, 3, 64, "f16", True),
    # fp32 with a long sequence: the dK/dV and dQ walks split into pieces whose
    # partial sums are added over the packed rows only
    ([2000, 300, 0, 1100], 2, 2, 64, "f32", True),
    ([1700, 5, 900], 4, 2, 64, "f32", False),
]


@pytest.mark.parametrize("lengths,H,H_kv,d,dtype,causal", VARLEN_CASES)
def test_varlen_parity(lengths, H, H_kv, d, dtype, causal):
    seed = 5000 + sum(lengths) % 997 + 7 * H + H_kv + d + (1 if causal else 0)
    run_varlen_case(vw(lengths, H, H_kv, d, dtype, causal, seed))


@pytest.mark.parametrize("lengths,H,H_kv,d,dtype,causal", [
    ([300, 1, 129], 2, 2, 128, "bf16", True),
    ([513, 31], 6, 3, 64, "f16", True),
    ([700, 65], 2, 1, 64, "f32", False),
])
def test_varlen_negative_scale(lengths, H, H_kv, d, dtype, causal):
    """A negative factor on q . k through the packed entry points."""
    seed = 5300 + sum(lengths) % 997 + 7 * H + H_kv + d
    run_varlen_case(vw(lengths, H, H_kv, d, dtype, causal, seed), scale=-1.1 / d ** 0.5)


def test_varlen_rows_past_the_last_sequence_untouched():
    """T larger than the packed total: the last 123 rows of every head belong
    to no sequence and must not be written."""
    run_varlen_case(vw([100, 250, 31], 2, 2, 128, "bf16", True, 5101, T=381 + 123))


def test_varlen_split_group_rows_past_the_last_sequence_untouched():
    """The same with grouped heads at d = 128 in bf16, where the dK/dV stage
    splits each group and a second kernel sums the partials over all rows."""
    run_varlen_case(vw([300, 129], 8, 2, 128, "bf16", True, 5104, T=429 + 77))


def test_varlen_stress_rescaling():
    """Logits of about 64 nats (q, k x 8) over ragged lengths."""
    run_varlen_case(vw([1000, 77, 431], 4, 4, 64, "bf16", False, 5102, qk_mult=8.0))


def test_varlen_workload_all_sequences():
    """The packed benchmark workload (16 sequences of 512 .. 4096 tokens, 16
    heads, d = 128, causal bf16), as the benchmark runs it (its 256 sequence
    and head pairs take the head-grouped causal order), every sequence
    against the oracle."""
    w = workloads.VARLEN_WORKLOADS["varlen_causal_bf16"]
    run_varlen_case(w)


@pytest.mark.parametrize("dtype,d,H_kv", [("bf16", 128, 2), ("f32", 64, 4), ("f16", 128, 4)])
def test_varlen_equal_lengths_match_fixed_bitwise(dtype, d, H_kv):
    """Equal lengths packed as [H, B*N, d] run the same tiles as the fixed
    [B, H, N, d] call: every output must be the same bits."""
    B, H, N = 3, 4, 333
    w = workloads.custom(B, H, N, d, dtype, True, 5103, name="fixed", H_kv=H_kv)
    q, k, v, dO = workloads.make_inputs(w, device="cuda")
    o, lse = fa.forward(q, k, v, True, w.scale)
    dq, dk, dv = fa.backward(q, k, v, o, lse, dO, True, w.scale)
    pack = lambda t: t.permute(1, 0, 2, 3).reshape(t.shape[1], B * N, d).contiguous()  # noqa: E731
    unpack = lambda t: t.reshape(t.shape[0], B, N, d).permute(1, 0, 2, 3)  # noqa: E731
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device="cuda")
    qp, kp, vp, gp = pack(q), pack(k), pack(v), pack(dO)
    op = torch.empty_like(qp)
    lsep = torch.empty((H, B * N), dtype=torch.float32, device="cuda")
    fa.fa2_forward_varlen(qp, kp, vp, op, lsep, cu, N, True, w.scale)
    dqp, dkp, dvp = torch.empty_like(qp), torch.empty_like(kp), torch.empty_like(vp)
    fa.fa2_backward_varlen(qp, kp, vp, op, gp, lsep, dqp, dkp, dvp, cu, N, True, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(unpack(op), o)
    assert torch.equal(lsep.reshape(H, B, N).permute(1, 0, 2), lse)
    assert torch.equal(unpack(dqp), dq)
    assert torch.equal(unpack(dkp), dk)
    assert torch.equal(unpack(dvp), dv)


def test_varlen_rejects_on_gpu():
    q = torch.zeros((2, 10, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((2, 10), dtype=torch.float32, device="cuda")
    cu = torch.tensor([0, 4, 10], dtype=torch.int32, device="cuda")
    with pytest.raises(fa.Fa2Error):  # max_seqlen above T
        fa.fa2_forward_varlen(q, q, q, torch.empty_like(q), lse, cu, 11)
    with pytest.raises(ValueError):  # offsets must be int32
        fa.fa2_forward_varlen(q, q, q, torch.empty_like(q), lse, cu.long(), 6)
