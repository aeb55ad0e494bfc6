#!/usr/bin/env python3
"""FlashAttention-2 forward + backward throughput on one MI355X.

One step = the whole hot path over one batch of the large causal bf16
workload (B=4, H=16, N=4096, d=128): ``fa2_forward`` and then the two
backward stages (the dQ kernel, which also computes D; the dK/dV kernel),
i.e. exactly ``fa2_backward``, called stage by stage so that HIP events on
the launch stream can time each kernel.  The default 30 warmup steps let the
clocks settle; 100 timed steps take about 0.15 s.  Inputs are seeded synthetic tensors
already resident in HBM when the timed region starts.

Counted FLOP (causal halves it): forward 4*B*H*N^2*d/2, backward 2.5x that
(five products, the recomputation of S counted once), step 3.5x.

Prints ONE JSON line with the throughput, the roofline of the dominant
kernel (its counted FLOP per launch over its mean event-timed duration,
against the bf16 dense MFMA peak) and the oracle's CPU throughput on a
bounded sample of heads of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload 1..7]
    python bench.py --decode decode_gqa_bf16
    python bench.py --varlen varlen_causal_bf16

Workload 6 is the same shape with grouped-query attention (16 query heads
over 2 key/value heads) and workload 7 the same shape in fp16; their lines
are not the headline.  ``--decode`` times
decoding instead (one new query per sequence against a 16 K cache, 64 query
heads over 8 key/value heads): one step is one ``fa2_decode`` call (the
split-cache kernel and the merge kernel); it is bound by HBM, so its line
reports GB/s of algorithmic bytes (the cache read once, Q read, O and LSE
written) against the 8 TB/s HBM peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Public MI355X figures (dense, no sparsity), TFLOP/s.
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}
HBM_GBS = 8000.0
METRIC = "attention fwd+bwd TFLOP/s and % MFMA peak (bf16 B4 H16 N4096 d128 causal)"
CSRC = os.path.join(ROOT, "tiled_attention_fwd_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def counted_flop(w):
    fwd = 4.0 * w.B * w.H * w.N * w.N * w.d * (0.5 if w.causal else 1.0)
    return fwd, 2.5 * fwd, 3.5 * fwd


# Source files each kernel is compiled from (for tying stored counter
# readings to the kernel version they were taken on).
KERNEL_SOURCES = {
    "fwd_kernel": ["fa2_fwd.hip", "fa2_common.hpp", "fa2_launch.hpp", "fa2_swz.hpp"],
    "bwd_dkdv_kernel": ["fa2_bwd.hip", "fa2_common.hpp", "fa2_launch.hpp", "fa2_swz.hpp"],
    "bwd_dq_kernel": ["fa2_bwd.hip", "fa2_common.hpp", "fa2_launch.hpp", "fa2_swz.hpp"],
    "decode_kernel": ["fa2_decode.hip", "fa2_common.hpp", "fa2_launch.hpp", "fa2_swz.hpp"],
}


def stage_kernels(dtype: str, d: int) -> list:
    """Kernel names of the forward call and backward stages 1 and 2, in order:
    the dQ kernel computes D and LSE*log2(e) itself and runs as stage 1."""
    return ["fwd_kernel", "bwd_dq_kernel", "bwd_dkdv_kernel"]


def source_hash(kernel: str) -> str:
    """Hash of the HIP sources a kernel is built from."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is missing or was taken on other kernel sources."""
    path = os.path.join(PROFILES, "%s_%s_traffic.md" % (kernel, workload))
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_hash:\s*([0-9a-f]+)", text)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not b or m.group(1) != source_hash(kernel):
        return None
    return float(b.group(1))


def cpu_model() -> str:
    """The host CPU's model name (for the oracle's timing line)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, inputs, gpu_outs, budget_s: float):
    """Time the fp64 oracle (test infrastructure) on whole heads of the same
    workload until about ``budget_s`` seconds of work are done; also report
    the GPU's error on those heads.  With grouped-query attention the unit is
    a key/value head with its group of query heads (dK, dV are group sums)."""
    import numpy as np
    import oracle

    orc = oracle.default()
    q, k, v, dO = (t.cpu() for t in inputs)
    o, lse, dq, dk, dv = (t.float().cpu() for t in gpu_outs)
    G = w.H // w.kv_heads
    units = [(b, hk) for b in range(w.B) for hk in range(w.kv_heads)]
    done, t_total = 0, 0.0
    errs = {n: 0.0 for n in ("O", "LSE", "dQ", "dK", "dV")}

    def rel(a, r):
        a = np.asarray(a, dtype=np.float64)
        return float(np.max(np.abs(a - r)) / max(np.max(np.abs(r)), 1e-300))

    for b, hk in units:
        sq = (slice(b, b + 1), slice(hk * G, (hk + 1) * G))
        sk = (slice(b, b + 1), slice(hk, hk + 1))
        t0 = time.perf_counter()
        o_r, lse_r = orc.fwd(q[sq], k[sk], v[sk], w.scale, w.causal)
        dq_r, dk_r, dv_r = orc.bwd(q[sq], k[sk], v[sk], dO[sq], w.scale, w.causal)
        t_total += time.perf_counter() - t0
        done += 1
        for name, a, r in (("O", o[sq], o_r), ("LSE", lse[sq], lse_r), ("dQ", dq[sq], dq_r),
                           ("dK", dk[sk], dk_r), ("dV", dv[sk], dv_r)):
            errs[name] = max(errs[name], rel(a, r))
        if t_total >= budget_s:
            break
    step_flop_per_unit = counted_flop(w)[2] / (w.B * w.kv_heads)
    value = step_flop_per_unit * done / t_total / 1e12
    what = "heads" if G == 1 else "key/value heads (x%d query heads)" % G
    return {
        "value": value, "unit": "TFLOP/s", "cores": orc.max_threads(), "cpu_model": cpu_model(), "kind": "oracle",
        "sample": "%d of %d %s of %s, fp64 forward+backward, %.1f s" % (done, len(units), what, w.name, t_total),
    }, {"units_checked": done, "max_rel_err": errs}


def decode_bytes(w):
    """Algorithmic HBM bytes of one decoding pass: K and V read once, Q read,
    O and LSE written."""
    s = 2 if w.dtype == "bf16" else 4
    return 2 * w.B * w.H_kv * w.N_k * w.d * s + 2 * w.B * w.H * w.N_q * w.d * s + 4 * w.B * w.H * w.N_q


def decode_cpu_baseline(w, inputs, gpu_outs, budget_s: float):
    """The oracle's decode (test infrastructure) on whole key/value heads of
    the same workload, each with its group of query heads, until about
    ``budget_s`` seconds; GB/s of the same algorithmic bytes per unit."""
    import numpy as np
    import oracle

    orc = oracle.default()
    q, k, v = (t.cpu() for t in inputs)
    o, lse = (t.float().cpu() for t in gpu_outs)
    G = w.H // w.H_kv
    units = [(b, hk) for b in range(w.B) for hk in range(w.H_kv)]
    done, t_total, err = 0, 0.0, 0.0
    for b, hk in units:
        sq = (slice(b, b + 1), slice(hk * G, (hk + 1) * G))
        sk = (slice(b, b + 1), slice(hk, hk + 1))
        t0 = time.perf_counter()
        o_r, lse_r = orc.decode(q[sq], k[sk], v[sk], w.scale, w.causal)
        t_total += time.perf_counter() - t0
        done += 1
        for a, r in ((o[sq], o_r), (lse[sq], lse_r)):
            a = np.asarray(a, dtype=np.float64)
            err = max(err, float(np.max(np.abs(a - r)) / max(np.max(np.abs(r)), 1e-300)))
        if t_total >= budget_s:
            break
    per_unit = decode_bytes(w) / len(units)
    return {
        "value": per_unit * done / t_total / 1e9, "unit": "GB/s", "cores": orc.max_threads(),
        "cpu_model": cpu_model(), "kind": "oracle",
        "sample": "%d of %d key/value heads (x%d query heads) of %s, fp64 decode, %.1f s"
                  % (done, len(units), G, w.name, t_total),
    }, {"units_checked": done, "max_rel_err": err}


def bench_decode(args) -> int:
    import torch
    import tiled_attention_fwd_amd as fa
    import workloads

    w = workloads.DECODE_WORKLOADS[args.decode]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = workloads.make_decode_inputs(w, seed=args.seed, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N_q), dtype=torch.float32, device=dev)
    need = fa.fa2_decode_workspace_size(w.B, w.H, w.H_kv, w.N_q, w.N_k, w.d, q.dtype)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        fa.fa2_decode(q, k, v, o, lse, w.causal, w.scale, ws, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    # Per-call events in a second pass, outside the timed region.
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    ev[0].record(stream)
    for s in range(K):
        step()
        ev[s + 1].record(stream)
    torch.cuda.synchronize()
    launch_ms = statistics.fmean(ev[s].elapsed_time(ev[s + 1]) for s in range(K))
    nbytes = decode_bytes(w)
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (launch_ms * 1e-3) / 1e9
    result = {
        "metric": "attention decode GB/s of algorithmic HBM bytes (bf16 B16 H64/kv8 Nq1 Nk16384 d128)",
        "value": value, "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "H_kv": w.H_kv, "N_q": w.N_q, "N_k": w.N_k, "d": w.d,
                   "causal": w.causal, "seed": w.seed if args.seed is None else args.seed},
        # One fa2_decode call is the decode kernel plus the small merge kernel;
        # the events time both, so the kernel's own rate is a little higher.
        "roofline": {"bound": "hbm", "kernel": "decode_kernel", "achieved": achieved, "peak": HBM_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_GBS, "traffic": stored_traffic("decode_kernel", w.name),
                     "mean_launch_ms": launch_ms, "bytes_per_launch": nbytes},
    }
    detail = {"call_ms": launch_ms, "tflops": 4.0 * w.B * w.H * w.N_q * w.N_k * w.d / (launch_ms * 1e-3) / 1e12,
              "workspace_bytes": need}
    if args.cpu_budget > 0:
        cb, parity = decode_cpu_baseline(w, (q, k, v), (o, lse), args.cpu_budget)
        result["cpu_baseline"] = cb
        detail["parity_sampled_heads"] = parity
    else:
        result["cpu_baseline"] = None
    result["detail"] = detail
    print(json.dumps(result), flush=True)
    return 0


def bench_varlen(args) -> int:
    """One step of a packed ragged batch: fa2_forward_varlen and the two
    backward stages; counted FLOP summed over the sequences (4 H n^2 d per
    sequence forward, halved when causal; backward 2.5x, step 3.5x)."""
    import torch
    import tiled_attention_fwd_amd as fa
    import workloads

    w = workloads.VARLEN_WORKLOADS[args.varlen]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v, dO, cu = workloads.make_varlen_inputs(w, seed=args.seed, device=dev)
    H, T, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((H, T), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    B = len(w.lengths)
    ws = torch.empty(max(fa.fa2_backward_workspace_size_varlen(B, H, w.H_kv, T, w.max_seqlen, d, q.dtype), 16),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(evs=None):
        if evs:
            evs[0].record(stream)
        fa.fa2_forward_varlen(q, k, v, o, lse, cu, w.max_seqlen, w.causal, w.scale, stream)
        for s in (1, 2):
            if evs:
                evs[s].record(stream)
            fa.fa2_backward_varlen(q, k, v, o, dO, lse, dq, dk, dv, cu, w.max_seqlen, w.causal, w.scale, ws,
                                   stream, stage=s)
        if evs:
            evs[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / K
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    for s in range(K):
        step(events[s])
    torch.cuda.synchronize()
    names = stage_kernels(w.dtype, d)
    mean_ms = {n: statistics.fmean(events[s][i].elapsed_time(events[s][i + 1]) for s in range(K))
               for i, n in enumerate(names)}
    fwd_f = sum(4.0 * H * n * n * d * (0.5 if w.causal else 1.0) for n in w.lengths)
    step_f = 3.5 * fwd_f
    peak = PEAK_TFLOPS[w.dtype]
    value = step_f / (ms_per_step * 1e-3) / 1e12
    kflop = {"fwd_kernel": fwd_f, "bwd_dkdv_kernel": 0.8 * 2.5 * fwd_f, "bwd_dq_kernel": 0.2 * 2.5 * fwd_f}
    dom = max(kflop, key=lambda n: mean_ms[n])
    achieved = kflop[dom] / (mean_ms[dom] * 1e-3) / 1e12
    result = {
        "metric": "attention fwd+bwd TFLOP/s, packed ragged batch (bf16 16 seqs of 512-4096, H16 d128 causal)",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "lengths": list(w.lengths), "H": H, "H_kv": w.H_kv, "T": T, "d": d,
                   "causal": w.causal, "seed": w.seed if args.seed is None else args.seed},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": None, "mean_launch_ms": mean_ms[dom],
                     "flop_per_launch": kflop[dom]},
        "cpu_baseline": None,
        "detail": {"kernel_ms": mean_ms, "step_frac_peak": value / peak},
    }
    print(json.dumps(result), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", type=int, default=4)
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work (0: skip)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in a HIP graph (replays, no per-kernel events)")
    ap.add_argument("--decode", default=None, metavar="NAME",
                    help="time decoding on a named decoding workload instead (decode_gqa_bf16)")
    ap.add_argument("--varlen", default=None, metavar="NAME",
                    help="time a packed ragged batch instead (varlen_causal_bf16)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (3 times), to scale HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        return 2

    import torch
    import tiled_attention_fwd_amd as fa
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "repeats": 3}), flush=True)
        return 0
    if args.decode:
        return bench_decode(args)
    if args.varlen:
        return bench_varlen(args)
    w = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v, dO = workloads.make_inputs(w, seed=args.seed, device=dev)
    B, H, N, d = w.shape()
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(fa.fa2_backward_workspace_size_ex(B, H, k.shape[1], N, d, q.dtype), 16),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    # Grouped-query workloads go through the entry points with a key/value
    # head count; plain multi-head ones through the original calls.
    fwd_call = fa.fa2_forward_ex if w.kv_heads != H else fa.fa2_forward
    stage_call = fa.fa2_backward_stage_ex if w.kv_heads != H else fa.fa2_backward_stage

    def step(evs=None):
        if evs:
            evs[0].record(stream)
        fwd_call(q, k, v, o, lse, w.causal, w.scale, stream)
        for s in (1, 2):
            if evs:
                evs[s].record(stream)
            stage_call(s, q, k, v, o, dO, lse, dq, dk, dv, w.causal, w.scale, ws, stream)
        if evs:
            evs[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    # N = 1: there is no process group, so the barrier reduces to the sync.
    # The timed region is K plain steps; a second pass of K steps records
    # events around every kernel for the breakdown (an event record is a GPU
    # command of its own, so it stays out of the timed region).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    for s in range(K):
        step(events[s])
    torch.cuda.synchronize()

    names = stage_kernels(w.dtype, d)
    per = {n: [events[s][i].elapsed_time(events[s][i + 1]) for s in range(K)] for i, n in enumerate(names)}
    mean_ms = {n: statistics.fmean(x) for n, x in per.items()}
    fwd_f, bwd_f, step_f = counted_flop(w)
    bwd_ms = sum(mean_ms[n] for n in names[1:])
    peak = PEAK_TFLOPS[w.dtype]
    value = step_f / (ms_per_step * 1e-3) / 1e12

    # Counted FLOP per kernel: the backward's five products split as S, dP, dV,
    # dK (4/5, dK/dV kernel) and dQ (1/5, dQ kernel); the dQ kernel's
    # recomputation of S and dP is implementation work and is not counted.
    kflop = {"fwd_kernel": fwd_f, "bwd_dkdv_kernel": 0.8 * bwd_f, "bwd_dq_kernel": 0.2 * bwd_f}
    dom = max(kflop, key=lambda n: mean_ms[n])
    dom_flop = kflop[dom]
    achieved = dom_flop / (mean_ms[dom] * 1e-3) / 1e12
    traffic = stored_traffic(dom, w.name)
    roofline = {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": traffic,
                "mean_launch_ms": mean_ms[dom], "flop_per_launch": dom_flop}

    result = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "H_kv": w.kv_heads, "N": N, "d": d, "causal": w.causal,
                   "seed": w.seed if args.seed is None else args.seed},
        "roofline": roofline,
    }
    step_ms = sorted(events[s][0].elapsed_time(events[s][3]) for s in range(K))
    detail = {
        "step_events_median_ms": statistics.median(step_ms), "step_events_min_ms": step_ms[0],
        "fwd": {"ms": mean_ms["fwd_kernel"], "tflops": fwd_f / (mean_ms["fwd_kernel"] * 1e-3) / 1e12},
        "bwd": {"ms": bwd_ms, "tflops": bwd_f / (bwd_ms * 1e-3) / 1e12},
        "step_events_ms": mean_ms["fwd_kernel"] + bwd_ms,
        "kernel_ms": mean_ms,
        "peak_tflops": peak,
    }
    for kk in ("fwd", "bwd"):
        detail[kk]["frac_peak"] = detail[kk]["tflops"] / peak
    detail["step_frac_peak"] = value / peak
    detail["source_hash"] = {k: source_hash(k) for k in KERNEL_SOURCES}
    if args.graph:
        # The same step captured once in a HIP graph and replayed K times:
        # what the launch overhead costs the small workloads.
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fwd_call(q, k, v, o, lse, w.causal, w.scale)
            for st in (1, 2):
                stage_call(st, q, k, v, o, dO, lse, dq, dk, dv, w.causal, w.scale, ws)
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            graph.replay()
        torch.cuda.synchronize()
        g_ms = (time.perf_counter() - t0) * 1e3 / K
        detail["graph"] = {"ms_per_step": g_ms, "tflops": step_f / (g_ms * 1e-3) / 1e12}
    if args.cpu_budget > 0:
        cb, parity = cpu_baseline(w, (q, k, v, dO), (o, lse, dq, dk, dv), args.cpu_budget)
        result["cpu_baseline"] = cb
        detail["parity_sampled_heads"] = parity
    else:
        result["cpu_baseline"] = None
    result["detail"] = detail
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
