"""Run-to-run determinism: the same step, repeated ten times over the same
prefix (the advanced lengths written to a buffer of their own), must give
the same bits every time -- every output, both caches and the advanced
prefix lengths. Every reduction in the kernels has a fixed order, so nothing
may depend on which workgroup finishes first."""

import numpy as np
import pytest

from workloads import WORKLOADS, scaled

import parity
from gpu_helpers import require_gpu

pytestmark = pytest.mark.gpu

CASES = [
    WORKLOADS["vicuna7b_typical"],
    scaled(WORKLOADS["vicuna7b_batch8_ragged"], B=5, d=512, H=4, V=3001, L_range=(1, 900)),
    scaled(WORKLOADS["vicuna7b_exact"], B=3, d=256, H=2, V=1000, L=300, L_range=(300, 300)),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: f"{w.name}-B{w.B}-d{w.d}")
def test_step_repeats_bit_identical(w):
    require_gpu()
    import torch
    from medusa_tree_verification_forward_amd.step import VerifyStep, to_host
    inp = parity.inputs_for(w)
    st = VerifyStep(inp, H=w.H, Dh=w.Dh, s_max=w.s_max, mode=w.mode, tau=w.tau, eps=w.eps,
                    delta=w.delta, theta=w.rope_theta, want_logits=True)
    runs = []
    for _ in range(10):
        st.run_step(keep_kv_len=True)
        torch.cuda.synchronize()
        r = st.results()
        for k in ("k_cache", "v_cache", "kv_len"):
            r[k] = to_host(st.inp[k])
        r["kv_len_next"] = to_host(st.kv_len_next)
        runs.append(r)
    for i, r in enumerate(runs[1:], start=1):
        for k in runs[0]:
            assert np.array_equal(runs[0][k], r[k], equal_nan=True), (i, k)
