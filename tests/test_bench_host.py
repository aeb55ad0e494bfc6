"""Host-side logic of bench.py, checked without a GPU.

The FLOP convention (forward 4*B*H*N^2*d, halved when causal; backward 2.5x,
step 3.5x), the one-GPU guard, the kernels the stages enqueue, and the tie
between stored counter summaries and the kernel sources they were taken on.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


@pytest.mark.parametrize("wid,fwd,bwd,step", [
    (1, 2.62144e5, 6.5536e5, 9.17504e5),
    (2, 6.7108864e7, 1.6777216e8, 2.34881024e8),
    (3, 2.147483648e9, 5.36870912e9, 7.516192768e9),
    (4, 2.74877906944e11, 6.8719476736e11, 9.62072674304e11),
    (5, 4.9152e10, 1.2288e11, 1.72032e11),
])
def test_counted_flop_of_the_five_workloads(wid, fwd, bwd, step):
    f, b, s = bench.counted_flop(workloads.WORKLOADS[wid])
    assert (f, b, s) == pytest.approx((fwd, bwd, step), rel=1e-12)


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_stage_kernels():
    for dtype, d in (("bf16", 128), ("f16", 64), ("f32", 64), ("bf16", 32)):
        assert bench.stage_kernels(dtype, d) == ["fwd_kernel", "bwd_dq_kernel", "bwd_dkdv_kernel"]


def test_stored_traffic_is_tied_to_the_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    h = bench.source_hash("fwd_kernel")
    assert len(h) == 16 and h == bench.source_hash("fwd_kernel")
    path = tmp_path / "fwd_kernel_some_workload_traffic.md"
    path.write_text("hbm_bytes_per_launch: 1.25e+08\nsource_hash: %s\n" % h)
    assert bench.stored_traffic("fwd_kernel", "some_workload") == pytest.approx(1.25e8)
    path.write_text("hbm_bytes_per_launch: 1.25e+08\nsource_hash: %s\n" % ("0" * 16))
    assert bench.stored_traffic("fwd_kernel", "some_workload") is None  # taken on other sources
    assert bench.stored_traffic("fwd_kernel", "missing_workload") is None

