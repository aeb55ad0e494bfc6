"""The fp64 oracle against facts outside itself (CPU only).

Every pin lives in ``oracle_pins.py``; this file runs them on the shipped
oracle library, and runs the torch float64 library pin on the named
workloads (whole tensors for the three fp32 shapes, head slices of the two
bf16 shapes, whose full size would take minutes on the CPU).
"""
import json
import os

import numpy as np
import pytest

import oracle
import workloads
from tests import oracle_pins as pins

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=False)
    return oracle.default()


@pytest.mark.parametrize("i", range(len(pins.ALL_SMALL_PINS)))
def test_small_pins(orc, i):
    pins.ALL_SMALL_PINS[i](orc)


def test_finite_diff_config1_subset(orc):
    """256 seeded elements of each gradient at the tiny workload's shape."""
    w = workloads.WORKLOADS[1]
    pins.pin_finite_diff(orc, w.shape(), w.causal, seed=w.seed, sample=256)


@pytest.mark.parametrize("wid", [1, 2, 3])
def test_torch_pin_fp32_workloads(orc, wid):
    w = workloads.WORKLOADS[wid]
    q, k, v, dO = (t.double().numpy() for t in workloads.make_inputs(w))
    pins.pin_torch(orc, q, k, v, dO, w.scale, w.causal, tol=1e-10)


@pytest.mark.slow
@pytest.mark.parametrize("wid,heads", [(5, 2), (4, 1)])
def test_torch_pin_bf16_workload_heads(orc, wid, heads):
    w = workloads.WORKLOADS[wid]
    q, k, v, dO = (t[:1, :heads].double().numpy() for t in workloads.make_inputs(w))
    pins.pin_torch(orc, q, k, v, dO, w.scale, w.causal, tol=1e-10)


def test_ragged_stress_rescaling_is_exercised(orc):
    """The ragged workload's logits really are large (sigma near 64 nats), so
    the online softmax must rescale its running maximum: check on a head."""
    w = workloads.WORKLOADS[5]
    q, k, _, _ = (t[:1, :1].double().numpy() for t in workloads.make_inputs(w))
    S = w.scale * np.einsum("bhid,bhjd->bhij", q, k)
    assert 40.0 < float(S.std()) < 90.0


def test_article_figure_67mb_matches_mega_class_shape():
    fig = json.load(open(os.path.join(HERE, "golden", "article_figures.json")))
    mb = [f for f in fig["figures"] if f["name"].startswith("cached_matrix")][0]["value_mb"]
    w = workloads.WORKLOADS[3]
    nbytes = w.B * w.H * w.N * w.N * 4
    assert nbytes == 67_108_864
    assert round(nbytes / 1e6) == mb
