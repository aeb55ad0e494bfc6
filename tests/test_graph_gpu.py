"""HIP graph capture of the forward and backward passes.

The library allocates nothing and records no memset, so a whole step
(forward, then the backward stages) can be captured into a HIP graph
(torch.cuda.CUDAGraph on ROCm) and replayed.  The graph is replayed several
times with unrelated eager work and synchronisations between the replays,
and every replay must give exactly the bits of the eager calls (the kernels
are deterministic).  Decoding is captured the same way.
"""
import pytest
import torch

import tiled_attention_fwd_amd as fa
import workloads
from tests.test_parity_gpu import log

pytestmark = pytest.mark.gpu


def _eager_noise(dev):
    # unrelated eager work on the same stream between replays
    x = torch.randn(1 << 16, device=dev)
    return float((x * x).sum().item())


def _capture(step):
    """Warm up on a side stream, then capture step() into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    return g


# Workload 3 (fp32) splits its dK/dV and dQ walks: the partial sums and
# their fixed-order reduction are captured too.
@pytest.mark.parametrize("wid", [3, 4, 5, 6])
def test_graph_replays_match_eager(wid):
    w = workloads.WORKLOADS[wid]
    if wid == 4:  # a smaller batch of the large shape keeps the test short
        w = workloads.custom(1, 4, 4096, 128, "bf16", True, 6001, name="graph")
    log("graph case: %s" % w.describe())
    dev = torch.device("cuda")
    q, k, v, dO = workloads.make_inputs(w, device=dev)
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(fa.fa2_backward_workspace_size_ex(B, H, k.shape[1], N, d, q.dtype), 16),
                     dtype=torch.uint8, device=dev)

    def step():
        fa.fa2_forward_ex(q, k, v, o, lse, w.causal, w.scale)
        fa.fa2_backward_ex(q, k, v, o, dO, lse, dq, dk, dv, w.causal, w.scale, ws)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, dq, dk, dv)]
    g = _capture(step)
    for r in range(4):
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        _eager_noise(dev)
        for name, t, e in zip(("O", "LSE", "dQ", "dK", "dV"), (o, lse, dq, dk, dv), ref):
            assert torch.equal(t, e), "replay %d: %s differs from the eager result" % (r, name)


def test_graph_decode_replays_match_eager():
    w = workloads.DecodeWorkload("graph_decode", 4, 16, 4, 2, 5000, 128, "bf16", True, 6002)
    log("graph case: %s" % w.describe())
    dev = torch.device("cuda")
    q, k, v = workloads.make_decode_inputs(w, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N_q), dtype=torch.float32, device=dev)
    ws = torch.empty(max(fa.fa2_decode_workspace_size(w.B, w.H, w.H_kv, w.N_q, w.N_k, w.d, q.dtype), 16),
                     dtype=torch.uint8, device=dev)

    def step():
        fa.fa2_decode(q, k, v, o, lse, w.causal, w.scale, ws)

    step()
    torch.cuda.synchronize()
    ref = (o.clone(), lse.clone())
    g = _capture(step)
    for r in range(4):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        _eager_noise(dev)
        assert torch.equal(o, ref[0]) and torch.equal(lse, ref[1]), "decode replay %d differs" % r
