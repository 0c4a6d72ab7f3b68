"""The composite step recorded once in a HIP graph and replayed: every
replay, with eager steps and synchronisations in between, must reproduce
the eager step's outputs exactly (the prefix length is reset before each
step, so every step computes the same thing)."""

import numpy as np
import pytest

from workloads import WORKLOADS, scaled

import parity
from gpu_helpers import require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("w", [
    scaled(WORKLOADS["vicuna7b_typical"], d=512, H=4, V=3001, L=300, L_range=(300, 300)),
    scaled(WORKLOADS["vicuna7b_batch8_ragged"], B=3, d=256, H=2, V=2500, L_range=(1, 700)),
], ids=lambda w: f"{w.name}-{w.mode}")
def test_graph_replays_match_eager(w):
    require_gpu()
    import torch
    from medusa_tree_verification_forward_amd.step import VerifyStep, to_host
    inp = parity.inputs_for(w)
    st = VerifyStep(inp, H=w.H, Dh=w.Dh, s_max=w.s_max, mode=w.mode, tau=w.tau, eps=w.eps,
                    delta=w.delta, theta=w.rope_theta)

    def step():
        st.reset_kv_len()
        st.run_step()

    def snapshot():
        r = st.results()
        r["k_cache"] = to_host(st.inp["k_cache"])
        r["v_cache"] = to_host(st.inp["v_cache"])
        r["kv_len"] = to_host(st.inp["kv_len"])
        return r

    step()
    torch.cuda.synchronize()
    ref = snapshot()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for k in ref:
            assert np.array_equal(ref[k], got[k], equal_nan=True), (rep, k)
        step()               # eager work between replays
        torch.cuda.synchronize()
