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


@pytest.mark.parametrize("w", CASES, ids=lambda w: f"{w.name}-d{w.d}-V{w.V}-B{w.B}-{w.mode}")
def test_composite_separate_prefix_lengths(w):
    """With kv_len_out_or_null set, kv_len is left unchanged, the advanced
    lengths land in the separate buffer, and every other output equals the
    in-place call's; a second step then runs over the same prefix and gives
    the same outputs again."""
    require_gpu()
    inp = parity.inputs_for(w)
    a = parity.gpu_step(w, inp, composite=True)
    b = parity.gpu_step(w, inp, composite=True, keep_kv_len=True)
    c = parity.gpu_step(w, inp, composite=True, keep_kv_len=True, repeat=2)
    assert np.array_equal(b.pop("kv_len_after"), np.asarray(inp["kv_len"]))
    assert np.array_equal(c.pop("kv_len_after"), np.asarray(inp["kv_len"]))
    assert set(a) == set(b) == set(c)
    for k in sorted(a):
        assert np.array_equal(a[k], b[k], equal_nan=True), k
        assert np.array_equal(a[k], c[k], equal_nan=True), k


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
