"""The composite call (medusa_step) against the five separate calls and the
oracle. The composite fuses the tree tokens into the head merge and the row
statistics, posterior and commit into one workgroup per sequence, with the
same arithmetic in the same order: every output must be bit-identical to the
separate calls'."""

import numpy as np
import pytest

from workloads import WORKLOADS, scaled

import parity
from gpu_helpers import require_gpu
from test_gpu_step import SMALL

pytestmark = pytest.mark.gpu

CASES = SMALL + [scaled(WORKLOADS["vicuna7b_exact"], d=256, H=2, V=1000, L=100,
                        L_range=(100, 100))]


@pytest.mark.parametrize("w", CASES, ids=lambda w: f"{w.name}-d{w.d}-V{w.V}-B{w.B}-{w.mode}")
def test_composite_matches_separate_calls(w):
    require_gpu()
    inp = parity.inputs_for(w)
    a = parity.gpu_step(w, inp, composite=False)
    b = parity.gpu_step(w, inp, composite=True)
    assert set(a) == set(b)
    for k in sorted(a):
        assert np.array_equal(a[k], b[k], equal_nan=True), k


def test_composite_full_size_7b():
    """The throughput configuration, through the composite call, against the
    oracle."""
    require_gpu()
    w = WORKLOADS["vicuna7b_typical"]
    inp = parity.inputs_for(w)
    o = parity.oracle_for(w)
    g = parity.gpu_step(w, inp, composite=True)
    report = {}
    parity.compare_step(w, inp, g, o, report)
    assert report.get("ambiguous", 0) <= 2, report
    parity.gpu_posterior_consistent(w, g, o["topo"])
