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


def _exact_loop_inputs(n, B, seed):
    inp = _inputs(n, B=B, seed=seed)
    rng = np.random.default_rng(seed + 1)
    T = SPEC.shape[0] + 1
    for name in ("u_draft", "u_accept", "u_resample"):
        inp[name + "_steps"] = rng.random((n, B, T), dtype=np.float32)
        inp[name] = inp[name + "_steps"][0].copy()
    return inp


U_NAMES = ("u_draft", "u_accept", "u_resample")


def test_generate_exact_mode_equals_single_steps():
    # Exact p/q rejection in the decoding loop, 6 steps on the 45-node tree
    # at B = 1 (a step's [B][T] uniform block is 46 floats, so the library's
    # per-step stride MEDUSA_ALIGN4(B*T) = 48 differs from B*T): the loop must
    # reproduce, bit for bit, the same steps issued one composite call at a
    # time with the state handed on by the caller.
    require_gpu()
    import torch
    from medusa_tree_verification_forward_amd.step import to_host, to_device
    n = 6
    for B in (1, 3):
        inp = _exact_loop_inputs(n, B, seed=77 + B)
        loop = _step(inp, "exact")
        toks, acc = loop.generate(n, uniforms={k: to_device(inp[k + "_steps"])
                                               for k in U_NAMES})
        one = _step(inp, "exact")
        s_toks, s_acc = [], []
        for i in range(n):
            for k in U_NAMES:
                one.inp[k].copy_(to_device(inp[k + "_steps"][i]))
            one.run_step()
            one.inp["h"].copy_(one.out["h_next"])
            one.inp["root"].copy_(one.out["next_root"])
            s_toks.append(one.out["out_tokens"].clone())
            s_acc.append(one.out["accept_len"].clone())
        torch.cuda.synchronize()
        assert np.array_equal(to_host(toks), np.stack([to_host(t) for t in s_toks])), B
        assert np.array_equal(to_host(acc), np.stack([to_host(a) for a in s_acc])), B
        for k in ("h", "root", "kv_len", "k_cache", "v_cache"):
            assert np.array_equal(to_host(loop.inp[k]), to_host(one.inp[k])), (B, k)
        assert to_host(acc).sum() > 0


def test_generate_exact_mode_matches_oracle_loop():
    # The same loop against the oracle's: every step of every sequence must
    # be the oracle loop's until the first step with a sampling decision
    # within float error of its flip point (a draft draw within float32
    # rounding of a CDF edge, an acceptance test within 1e-3 of log p/q, the
    # final draw within 1e-4 of an edge); later steps of that sequence
    # depend on it and are not compared.
    require_gpu()
    import torch
    from medusa_tree_verification_forward_amd.step import to_host, to_device
    n, B = 6, 3
    inp = _exact_loop_inputs(n, B, seed=77)
    st = _step(inp, "exact")
    toks, acc = st.generate(n, uniforms={k: to_device(inp[k + "_steps"]) for k in U_NAMES})
    torch.cuda.synchronize()
    o = OG.generate(inp, n, exact_margins=True, mode="exact", bf16=True, **STEP)
    gt, ga = to_host(toks), to_host(acc)
    near = ((o["draft_margin"] < 2e-6) | (o["accept_margin"] < 1e-3)
            | (o["draw_margin"] < 1e-4))
    compared = 0
    for b in range(B):
        for i in range(n):
            if near[i, b]:
                break
            assert ga[i, b] == o["accept_len"][i, b], (i, b)
            assert np.array_equal(gt[i, b], o["out_tokens"][i, b]), (i, b)
            compared += 1
    print("compared steps", compared, "of", n * B)
    assert compared >= n, (compared, o["draft_margin"], o["accept_margin"], o["draw_margin"])
    assert o["accept_len"].sum() > 0 and (o["accept_len"] == 0).any()


def test_generate_graph_replay():
    # The decoding loop (5 steps, so the final state copy runs too) recorded
    # in one HIP graph and replayed three times, the loop state restored by
    # eager copies between replays: every replay must equal the eager loop
    # bit for bit -- tokens, accepted depths, h, root, kv_len and both caches
    # -- and the oracle's loop.
    require_gpu()
    import torch
    from medusa_tree_verification_forward_amd.step import to_host
    n, B = 5, 3
    inp = _inputs(n, B=B, seed=99)
    st = _step(inp, "greedy")
    keys = ("h", "root", "kv_len", "k_cache", "v_cache")
    start = {k: st.inp[k].clone() for k in keys}

    def restore():
        for k in keys:
            st.inp[k].copy_(start[k])

    def snapshot(toks, acc):
        out = {"toks": to_host(toks), "acc": to_host(acc)}
        out.update({k: to_host(st.inp[k]) for k in keys})
        return out

    toks, acc = st.generate(n)
    torch.cuda.synchronize()
    ref = snapshot(toks, acc)
    o = OG.generate(inp, n, mode="greedy", bf16=True, **STEP)
    assert np.array_equal(ref["acc"], o["accept_len"])
    assert np.array_equal(ref["toks"], o["out_tokens"])
    assert o["accept_len"].sum() > 0

    restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gtoks, gacc = st.generate(n)
    for rep in range(3):
        restore()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot(gtoks, gacc)
        for k in ref:
            assert np.array_equal(ref[k], got[k]), (rep, k)
        # eager work between the replays
        restore()
        st.generate(1)
        torch.cuda.synchronize()
