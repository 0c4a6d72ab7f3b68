"""GPU parity of medusa_build_tree against the oracle's tree (bit-exact)."""

import numpy as np
import pytest

from oracle import tree as OT
from workloads import cartesian_ranks

from gpu_helpers import dev, host, poisoned, require_gpu

pytestmark = pytest.mark.gpu


def _random_spec(rng, K, smax, n_target):
    nodes = set()
    frontier = [()]
    while len(nodes) < n_target and frontier:
        t = frontier[int(rng.integers(len(frontier)))]
        if len(t) == K or all(t + (x,) in nodes for x in range(smax)):
            frontier.remove(t)
            continue
        c = t + (int(rng.integers(smax)),)
        if c not in nodes:
            nodes.add(c)
            frontier.append(c)
    rows = sorted(nodes, key=lambda t: (len(t), t))
    spec = np.full((len(rows), K), -1, dtype=np.int32)
    for i, t in enumerate(rows):
        spec[i, :len(t)] = t
    return spec


def _build(spec, K, S, B, V, root, topk_ids, kv_len):
    import torch
    import medusa_tree_verification_forward_amd as M
    require_gpu()
    N = spec.shape[0]
    T = N + 1
    topo = OT.topology(spec, K)
    shape = M.make_shape(B, 128, V, K, 1, 128, 8192, N, topo.P, S, "bf16")
    tok = poisoned((B, T), torch.int32)
    mask = poisoned((T, T), torch.uint8)
    pos = poisoned((B, T), torch.int32)
    ret = poisoned((topo.P, K + 1), torch.int32)
    par = poisoned((T,), torch.int32)
    dep = poisoned((T,), torch.int32)
    M.build_tree(shape, spec, dev(root), dev(kv_len), tok, mask, pos, ret, par, dep,
                 topk_ids=dev(topk_ids))
    torch.cuda.synchronize()
    return topo, dict(tok=host(tok), mask=host(mask), pos=host(pos), ret=host(ret),
                      par=host(par), dep=host(dep))


def _check(topo, g, root, topk_ids, kv_len):
    assert np.array_equal(g["mask"], topo.mask)
    assert np.array_equal(g["ret"], topo.retrieve)
    assert np.array_equal(g["par"], topo.parent)
    assert np.array_equal(g["dep"], topo.depth)
    for b in range(root.shape[0]):
        assert np.array_equal(g["tok"][b], OT.draft_tokens_topk(topo, int(root[b]), topk_ids[b]))
        assert np.array_equal(g["pos"][b], OT.position_ids(topo, int(kv_len[b])))


@pytest.mark.parametrize("s", [(2, 2, 2), (3, 2, 2, 1, 1), (4, 3, 2, 2, 1), (2,), (16, 14)])
def test_cartesian_trees(s):
    rng = np.random.default_rng(sum(s))
    K, S, B, V = len(s), max(s), 3, 32000
    spec = cartesian_ranks(s)
    root = rng.integers(0, V, size=B).astype(np.int32)
    topk = rng.integers(0, V, size=(B, K, S)).astype(np.int32)
    kv_len = rng.integers(0, 4096, size=B).astype(np.int32)
    topo, g = _build(spec, K, S, B, V, root, topk, kv_len)
    _check(topo, g, root, topk, kv_len)


def test_sparse_trees_mixed_depth_leaves():
    rng = np.random.default_rng(1)
    for trial in range(25):
        K = int(rng.integers(1, 9))
        S = int(rng.integers(1, 17))
        spec = _random_spec(rng, K, S, int(rng.integers(1, 120)))
        B, V = int(rng.integers(1, 5)), 1000
        root = rng.integers(0, V, size=B).astype(np.int32)
        topk = rng.integers(0, V, size=(B, K, S)).astype(np.int32)
        kv_len = rng.integers(0, 100, size=B).astype(np.int32)
        topo, g = _build(spec, K, S, B, V, root, topk, kv_len)
        _check(topo, g, root, topk, kv_len)


def test_root_only_tree():
    rng = np.random.default_rng(2)
    K, S, B, V = 3, 2, 2, 50
    spec = np.zeros((0, K), dtype=np.int32)
    root = np.array([7, 9], dtype=np.int32)
    topk = rng.integers(0, V, size=(B, K, S)).astype(np.int32)
    kv_len = np.array([5, 0], dtype=np.int32)
    topo, g = _build(spec, K, S, B, V, root, topk, kv_len)
    _check(topo, g, root, topk, kv_len)


@pytest.mark.parametrize("V", [32000, 32001, 70000])
def test_sampled_tree_tokens_follow_inverse_cdf(V):
    # Sampling mode: each node draws from its depth's head softmax by inverse
    # CDF with its own uniform. Fed the same fp32 logits, the oracle's float64
    # CDF can only disagree where u * total falls within rounding of a CDF
    # step; such draws are counted, everything else must match.
    import torch
    import medusa_tree_verification_forward_amd as M
    require_gpu()
    rng = np.random.default_rng(3)
    s = (3, 2, 2, 1, 1)
    K, S, B = 5, 3, 2
    spec = cartesian_ranks(s)
    topo = OT.topology(spec, K)
    T = topo.T
    logits = (rng.standard_normal((B, K, V)) * 2).astype(np.float32)
    lse = np.log(np.exp(logits.astype(np.float64)).sum(-1)).astype(np.float32)
    u = rng.random((B, T), dtype=np.float32)
    root = rng.integers(0, V, size=B).astype(np.int32)
    kv_len = np.array([10, 20], dtype=np.int32)
    shape = M.make_shape(B, 128, V, K, 1, 128, 8192, topo.T - 1, topo.P, S, "bf16")
    tok = poisoned((B, T), torch.int32)
    mask = poisoned((T, T), torch.uint8)
    pos = poisoned((B, T), torch.int32)
    ret = poisoned((topo.P, K + 1), torch.int32)
    par = poisoned((T,), torch.int32)
    dep = poisoned((T,), torch.int32)
    M.build_tree(shape, spec, dev(root), dev(kv_len), tok, mask, pos, ret, par, dep,
                 draft_mode=M.DRAFT_SAMPLE, head_logits=dev(logits), head_lse=dev(lse),
                 u_draft=dev(u))
    torch.cuda.synchronize()
    g = host(tok)
    mismatches = 0
    for b in range(B):
        ref = OT.draft_tokens_sampled(topo, int(root[b]), logits[b].astype(np.float64), u[b])
        for n in range(T):
            if g[b, n] != ref[n]:
                # allowed only at a CDF step within float32 rounding
                q = np.exp(logits[b, topo.depth[n] - 1].astype(np.float64))
                C = np.cumsum(q)
                t = u[b, n] * C[-1]
                near = np.min(np.abs(C - t)) / C[-1]
                assert near < 1e-5, (b, n, g[b, n], ref[n], near)
                mismatches += 1
    assert mismatches <= 2


@pytest.mark.gpu
def test_topology_outputs_optional():
    """Per-step calls pass NULL for the spec-only outputs: those buffers stay
    untouched and tokens / positions match a full call's."""
    import torch
    import medusa_tree_verification_forward_amd as M
    require_gpu()
    s = (3, 2, 2, 1, 1)
    rng = np.random.default_rng(7)
    K, S, B, V = len(s), max(s), 2, 32000
    spec = cartesian_ranks(s)
    root = rng.integers(0, V, size=B).astype(np.int32)
    topk = rng.integers(0, V, size=(B, K, S)).astype(np.int32)
    kv_len = rng.integers(0, 4096, size=B).astype(np.int32)
    topo, full = _build(spec, K, S, B, V, root, topk, kv_len)
    N = spec.shape[0]
    T = N + 1
    shape = M.make_shape(B, 128, V, K, 1, 128, 8192, N, topo.P, S, "bf16")
    tok = poisoned((B, T), torch.int32)
    pos = poisoned((B, T), torch.int32)
    mask = poisoned((T, T), torch.uint8)
    before = host(mask).copy()
    M.build_tree(shape, spec, dev(root), dev(kv_len), tok, None, pos, None, None, None,
                 topk_ids=dev(topk))
    torch.cuda.synchronize()
    assert np.array_equal(host(tok), full["tok"])
    assert np.array_equal(host(pos), full["pos"])
    assert np.array_equal(host(mask), before)
