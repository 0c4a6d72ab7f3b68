"""medusa_generate (the decoding loop with its state on the device) against
the oracle's loop on planted agreement: the committed tokens and accepted
depths of every step, and the final state, must be the oracle's; running the
loop in two calls (an odd first one, so the state is copied back once) must
give what one call gives."""

import numpy as np
import pytest

from oracle import generate as OG
from workloads import cartesian_ranks, planted_inputs

from gpu_helpers import require_gpu

pytestmark = pytest.mark.gpu

A = np.array([[0.70, 0.15, 0.05], [0.60, 0.15, 0.05], [0.50, 0.15, 0.05],
              [0.45, 0.10, 0.05], [0.40, 0.10, 0.05]])
SPEC = cartesian_ranks((3, 2, 2, 1, 1))
STEP = dict(H=4, Dh=128, s_max=3, tau=1.0, eps=0.09, delta=0.3, theta=10000.0)


def _inputs(n, B=1, seed=2024):
    inp = planted_inputs(A, SPEC, n_steps=n, B=B, seed=seed)
    return {k: v for k, v in inp.items() if k not in ("pi", "true_rank")}


def _step(inp, mode):
    from medusa_tree_verification_forward_amd.step import VerifyStep
    return VerifyStep(inp, mode=mode, want_logits=False, **STEP)


@pytest.mark.parametrize("mode,B", [("greedy", 1), ("typical", 1), ("greedy", 3)])
def test_generate_matches_oracle_loop(mode, B):
    require_gpu()
    import torch
    from medusa_tree_verification_forward_amd.step import to_host
    n = 12
    inp = _inputs(n, B=B)
    st = _step(inp, mode)
    toks, acc = st.generate(n)
    torch.cuda.synchronize()
    o = OG.generate(inp, n, mode=mode, bf16=True, **STEP)
    assert np.array_equal(to_host(acc), o["accept_len"])
    assert np.array_equal(to_host(toks), o["out_tokens"])
    assert np.array_equal(to_host(st.inp["root"]), o["root"])
    assert np.array_equal(to_host(st.inp["kv_len"]), o["kv_len"])
    assert np.max(np.abs(to_host(st.inp["h"]) - o["h"])) < 1e-3
    assert o["accept_len"].sum() > 0
    # committed cache rows (bf16): equal up to the rounding of rotated keys
    from workloads import bf16_bits_to_f32
    for name in ("k_cache", "v_cache"):
        g = bf16_bits_to_f32(to_host(st.inp[name]))
        r = bf16_bits_to_f32(o[name])
        for b in range(B):
            L = int(o["kv_len"][b])
            assert np.max(np.abs(g[b, :, :L] - r[b, :, :L])) < 2e-2, name


def test_generate_in_two_calls():
    require_gpu()
    import torch
    from medusa_tree_verification_forward_amd.step import to_host
    inp = _inputs(7)
    one = _step(inp, "greedy")
    t1, a1 = one.generate(7)
    two = _step(inp, "greedy")
    ta, aa = two.generate(3)
    tb, ab = two.generate(4)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(t1), np.concatenate([to_host(ta), to_host(tb)]))
    assert np.array_equal(to_host(a1), np.concatenate([to_host(aa), to_host(ab)]))
    for k in ("h", "root", "kv_len", "k_cache", "v_cache"):
        assert np.array_equal(to_host(one.inp[k]), to_host(two.inp[k])), k
