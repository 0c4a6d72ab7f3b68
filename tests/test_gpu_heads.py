"""GPU parity of medusa_heads_forward against the oracle's heads."""

import numpy as np
import pytest

from oracle import heads as OH
from oracle import numerics as ON
from workloads import WORKLOADS, cartesian_ranks, make_inputs, scaled

from gpu_helpers import assert_close, dev, host, poisoned, require_gpu, workspace

pytestmark = pytest.mark.gpu


def _run_heads(w, inp, with_logits=True, packed=False):
    import torch
    import medusa_tree_verification_forward_amd as M
    require_gpu()
    B, K, S = w.B, w.K, w.s_max
    N = cartesian_ranks(w.s).shape[0]
    shape = M.make_shape(w.B, w.d, w.V, w.K, w.H, w.Dh, 64, N, int(np.prod(w.s)), S, w.dtype)
    ws = workspace(M.workspace_bytes(shape))
    ids = poisoned((B, K, S), torch.int32)
    vals = poisoned((B, K, S), torch.float32)
    lse = poisoned((B, K), torch.float32)
    logits = poisoned((B, K, w.V), torch.float32) if with_logits else None
    z = poisoned((B, K, w.d), torch.float32)
    W1, W2 = dev(inp["W1"]), dev(inp["W2"])
    W1p = M.packed_heads_w1(shape, W1) if packed else None
    W2p = M.packed_heads_w2(shape, W2) if packed else None
    M.heads_forward(shape, dev(inp["h"]), W1, W2, ids, vals, ws,
                    head_lse=lse, head_logits=logits, z=z, W1_packed=W1p, W2_packed=W2p)
    torch.cuda.synchronize()
    out = dict(ids=host(ids), vals=host(vals), lse=host(lse), z=host(z))
    if with_logits:
        out["logits"] = host(logits)
    return out


def _check_topk_on_own_logits(g):
    # the fused top-s must equal a stable sort of the kernel's own logits
    B, K, S = g["ids"].shape
    for b in range(B):
        for k in range(K):
            row = g["logits"][b, k].astype(np.float64)
            ref = np.lexsort((np.arange(row.shape[0]), -row))[:S]
            assert list(g["ids"][b, k]) == list(ref), (b, k)
            assert np.array_equal(g["vals"][b, k], g["logits"][b, k][ref])


def _check_against_oracle(w, inp, g):
    z, logits = OH.heads_forward(inp["h"], inp["W1"], inp["W2"])
    ids, vals, lse = OH.heads_topk(logits, w.s_max)
    assert_close(g["z"], z, 1e-5, "z")
    assert_close(g["logits"], logits, 1e-5, "head logits")
    err = float(np.max(np.abs(g["logits"] - logits)))
    ambiguous = 0
    for b in range(w.B):
        for k in range(w.K):
            if OH.topk_margin(logits[b, k], w.s_max) < 4 * err:
                ambiguous += 1
                continue
            assert list(g["ids"][b, k]) == list(ids[b, k]), (b, k)
    assert ambiguous == 0 or ambiguous < w.B * w.K // 4
    assert np.allclose(g["lse"], lse, rtol=1e-5, atol=1e-5)
    return ambiguous


SMALL = [
    WORKLOADS["tiny_fp32"],
    # bf16, several row blocks with a ragged tail, 5 heads, d spanning many vectors
    scaled(WORKLOADS["vicuna7b_typical"], d=512, V=2999, H=4, Dh=128),
    # batch of 3 (ragged batch tile), fp32
    scaled(WORKLOADS["tiny_fp32"], B=3, V=777),
    # batches of 3 or more bf16 vectors (the batched MFMA passes): 8 at d=256,
    # 3 at d=512, 11 (passes of 8 and 3) at d=1024, 5 at d=320 (odd column
    # block count)
    scaled(WORKLOADS["vicuna7b_batch8_ragged"], d=256, V=1500, H=2, Dh=128),
    scaled(WORKLOADS["vicuna7b_batch8_ragged"], B=3, d=512, V=2999, H=4, Dh=128),
    scaled(WORKLOADS["vicuna7b_batch8_ragged"], B=11, d=1024, V=1000, H=8, Dh=128),
    scaled(WORKLOADS["vicuna7b_batch8_ragged"], B=5, d=320, V=777, H=5, Dh=64),
    # wide pools (s_max = 16)
    scaled(WORKLOADS["tiny_fp32"], s=(16, 2), K=2, V=4000),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: f"{w.name}-d{w.d}-V{w.V}-B{w.B}")
def test_heads_small_shapes(w):
    inp = make_inputs(w, only=("W1", "W2"))
    g = _run_heads(w, inp)
    _check_topk_on_own_logits(g)
    _check_against_oracle(w, inp, g)


BATCHED = [w for w in SMALL if w.dtype == "bf16" and w.B >= 3]


@pytest.mark.parametrize("w", BATCHED, ids=lambda w: f"{w.name}-d{w.d}-V{w.V}-B{w.B}")
def test_heads_packed_weights_equal_row_major(w):
    # The batched passes read W1 and W2 in packed tiles when given them: the
    # same fragments in the same order, so every output is bit-identical.
    inp = make_inputs(w, only=("W1", "W2"))
    g = _run_heads(w, inp)
    gp = _run_heads(w, inp, packed=True)
    for key in g:
        assert np.array_equal(g[key], gp[key]), key


def test_heads_bias_and_identity_init():
    # W1 = 0, b1 = 0, W2_k = W_lm: every head reproduces the LM head on h.
    import torch
    import medusa_tree_verification_forward_amd as M
    require_gpu()
    w = scaled(WORKLOADS["tiny_fp32"], V=1200)
    inp = make_inputs(w, only=("W_lm",))
    K, d = w.K, w.d
    W1 = np.zeros((K, d, d), dtype=np.float32)
    W2 = np.stack([inp["W_lm"]] * K)
    shape = M.make_shape(1, d, w.V, K, w.H, w.Dh, 64, 14, 8, w.s_max, "f32")
    ws = workspace(M.workspace_bytes(shape))
    ids = poisoned((1, K, w.s_max), torch.int32)
    vals = poisoned((1, K, w.s_max), torch.float32)
    z = poisoned((1, K, d), torch.float32)
    logits = poisoned((1, K, w.V), torch.float32)
    b1 = torch.zeros((K, d), dtype=torch.float32, device="cuda")
    M.heads_forward(shape, dev(inp["h"]), dev(W1), dev(W2), ids, vals, ws, b1=b1, z=z,
                    head_logits=logits)
    torch.cuda.synchronize()
    zh = host(z)
    lg = host(logits)
    for k in range(K):
        assert np.array_equal(zh[0, k], inp["h"][0])       # exact residual identity
        assert np.array_equal(lg[0, k], lg[0, 0])          # identical heads, identical logits
    ref = OH.lm_head(inp["W_lm"], inp["h"].astype(np.float64))
    assert_close(lg[0, 0], ref[0], 1e-5, "identity logits")


def test_heads_full_size_7b():
    # Full 7B shapes, the launch configuration the throughput run uses.
    w = WORKLOADS["vicuna7b_typical"]
    inp = make_inputs(w, only=("W1", "W2"))
    g = _run_heads(w, inp)
    _check_topk_on_own_logits(g)
    # oracle, head by head, in float64
    z = np.empty((1, w.K, w.d))
    for k in range(w.K):
        z[:, k] = OH.residual_block(inp["W1"][k], inp["h"].astype(np.float64))
    assert_close(g["z"], z, 1e-5, "z")
    rng = np.random.default_rng(0)
    for k in range(w.K):
        W2k = ON.widen(inp["W2"][k])
        logits = W2k @ z[0, k]
        assert_close(g["logits"][0, k], logits, 1e-5, f"head {k} logits")
        ids, vals = OH.top_s(logits, w.s_max)
        err = float(np.max(np.abs(g["logits"][0, k] - logits)))
        if OH.topk_margin(logits, w.s_max) >= 4 * err:
            assert list(g["ids"][0, k]) == list(ids)
        assert abs(g["lse"][0, k] - OH.log_sum_exp(logits)) < 1e-4
        # spot rows one by one
        rows = rng.integers(0, w.V, size=64)
        for r in rows:
            assert abs(g["logits"][0, k, r] - float(W2k[r] @ z[0, k])) < 1e-4


def test_heads_full_size_batch8():
    # Eight 7B-shaped sequences: the batched passes at the launch configuration
    # of the batch-8 workload; W1 in full, W2 on sampled rows of every head.
    w = WORKLOADS["vicuna7b_batch8_ragged"]
    inp = make_inputs(w, only=("W1", "W2"))
    g = _run_heads(w, inp)
    _check_topk_on_own_logits(g)
    # the packed-weight passes (as the step runs them) give the same bits
    gp = _run_heads(w, inp, packed=True)
    for key in g:
        assert np.array_equal(g[key], gp[key]), key
    z = np.empty((w.B, w.K, w.d))
    for k in range(w.K):
        z[:, k] = OH.residual_block(inp["W1"][k], inp["h"].astype(np.float64))
    assert_close(g["z"], z, 1e-5, "z")
    rng = np.random.default_rng(1)
    for k in range(w.K):
        rows = np.sort(rng.choice(w.V, size=256, replace=False))
        ref = ON.widen(inp["W2"][k][rows]) @ z[:, k].T          # [rows][B]
        assert_close(g["logits"][:, k, rows], ref.T, 1e-5, f"head {k} sampled logits")
        for b in range(w.B):
            assert abs(g["lse"][b, k] - OH.log_sum_exp(g["logits"][b, k].astype(np.float64))) < 1e-4
