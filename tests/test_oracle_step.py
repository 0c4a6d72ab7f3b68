"""Whole-step oracle invariants on the tiny fp32 workload (CPU only)."""

import numpy as np
import pytest

from oracle import posterior as OP
from oracle import step as OSTEP
from oracle import tree as OT
from oracle import verifier as OV
from workloads import WORKLOADS, make_inputs, scaled


def _run(w):
    inp = make_inputs(w)
    res = OSTEP.verify_step(inp, H=w.H, Dh=w.Dh, s_max=w.s_max, mode=w.mode, tau=w.tau,
                            eps=w.eps, delta=w.delta, theta=w.rope_theta,
                            bf16=(w.dtype == "bf16"))
    return inp, res


@pytest.mark.parametrize("mode", ["greedy", "typical", "exact"])
def test_tiny_step_invariants(mode):
    w = scaled(WORKLOADS["tiny_fp32"], mode=mode, tau=0.7 if mode == "typical" else 1.0)
    inp, res = _run(w)
    topo = res["topo"]
    assert topo.T == 15 and topo.P == 8
    b = 0
    a = int(res["accept_len"][b])
    assert 0 <= a <= w.K
    out = res["out_tokens"][b]
    assert out[0] == inp["root"][b]
    assert np.all(out[a + 1:] == -1) and np.all(out[:a + 1] >= 0)
    last = int(res["last_node"][b])
    assert topo.depth[last] == a
    assert list(out[:a + 1]) == list(res["tokens"][b][topo.path(last)])
    assert topo.retrieve[res["best_path"][b], a] == last
    L = int(inp["kv_len"][b])
    assert res["kv_len_next"][b] == L + a + 1
    assert np.array_equal(res["h_next"][b], res["y"][b][last])
    assert np.array_equal(res["positions"][b], L + topo.depth)
    if mode != "exact":
        assert res["next_root"][b] == res["argmax"][b][last]
        acc = res["acc"][b]
        ok, best = OP.longest_prefix_nodes(topo, acc)
        alen, pbest = OP.longest_prefix_paths(topo, acc)
        assert best == last and alen[pbest] == a
    else:
        # exact mode: drafted tokens are draws from the head distributions
        q = np.exp(res["head_logits"][b] - res["head_lse"][b][:, None])
        for n in range(1, topo.T):
            assert q[topo.depth[n] - 1, res["tokens"][b][n]] > 0


def test_tiny_lm_head_entropy_near_two_nats():
    # The tiny workload scales the LM head so its logits on h carry ~2 nats.
    w = WORKLOADS["tiny_fp32"]
    inp = make_inputs(w)
    logits = inp["h"][0].astype(np.float64) @ inp["W_lm"].astype(np.float64).T
    _, H, _ = OV.row_distribution(logits[None], 1.0)
    assert abs(H[0] - 2.0) < 0.01


def test_tiny_step_topk_feeds_tree():
    w = WORKLOADS["tiny_fp32"]
    inp, res = _run(w)
    topo = res["topo"]
    tok = OT.draft_tokens_topk(topo, int(inp["root"][0]), res["topk_ids"][0])
    assert np.array_equal(tok, res["tokens"][0])
