"""GPU parity of medusa_tree_attention against the oracle's masked attention."""

import numpy as np
import pytest

from oracle import tree as OT
from oracle import verifier as OV
from oracle.numerics import widen
from workloads import cartesian_ranks, f32_to_bf16_bits

from gpu_helpers import assert_close, dev, host, poisoned, require_gpu, workspace

pytestmark = pytest.mark.gpu


def _case(rng, spec, K, B, H, Dh, Ls, Lmax, dtype):
    topo = OT.topology(spec, K)
    T = topo.T
    st = (lambda x: f32_to_bf16_bits(x.astype(np.float32))) if dtype == "bf16" else \
        (lambda x: x.astype(np.float32))
    q = st(rng.standard_normal((B, T, H, Dh)))
    kt = st(rng.standard_normal((B, T, H, Dh)))
    vt = st(rng.standard_normal((B, T, H, Dh)))
    kc = np.zeros((B, H, Lmax, Dh))
    vc = np.zeros((B, H, Lmax, Dh))
    for b in range(B):
        kc[b, :, :Ls[b]] = rng.standard_normal((H, Ls[b], Dh))
        vc[b, :, :Ls[b]] = rng.standard_normal((H, Ls[b], Dh))
    return topo, q, kt, vt, st(kc), st(vc)


def _run(topo, q, kt, vt, kc, vc, Ls, K, dtype, scale):
    import torch
    import medusa_tree_verification_forward_amd as M
    require_gpu()
    B, T, H, Dh = q.shape
    Lmax = kc.shape[2]
    shape = M.make_shape(B, H * Dh, 100, K, H, Dh, Lmax, T - 1, topo.P, 2, dtype)
    ws = workspace(M.workspace_bytes(shape))
    out = poisoned((B, T, H, Dh), torch.float32)
    M.tree_attention(shape, dev(q), dev(kt), dev(vt), dev(kc), dev(vc),
                     dev(np.array(Ls, dtype=np.int32)), dev(topo.mask), scale, out, ws)
    torch.cuda.synchronize()
    return host(out)


def _oracle(topo, q, kt, vt, kc, vc, Ls, scale):
    B = q.shape[0]
    return np.stack([OV.tree_attention(widen(q[b]), widen(kt[b]), widen(vt[b]), kc[b], vc[b],
                                       Ls[b], topo.mask, scale) for b in range(B)])


CASES = [
    # (tree s, B, H, Dh, prefix lengths, dtype)
    ((2, 2, 2), 1, 4, 64, [64], "f32"),
    ((3, 2, 2, 1, 1), 1, 4, 128, [2048], "bf16"),
    ((3, 2, 2, 1, 1), 3, 2, 128, [0, 1, 777], "bf16"),     # empty, single-row, ragged prefix
    ((4, 3, 2, 2, 1), 1, 2, 128, [4096], "bf16"),          # 137 rows: 9 query tiles
    ((4, 3, 2, 2, 1), 2, 3, 128, [3000, 40], "bf16"),      # 9 tiles, two ragged sequences
    ((2, 2), 2, 3, 64, [255, 257], "bf16"),               # Dh 64, around a chunk boundary
    ((16, 14), 1, 1, 128, [100], "bf16"),                  # 241 rows: 16 query tiles
    ((2, 2, 2), 2, 2, 128, [300, 5], "f32"),
    # B H = 256: one chunk per (b, h) in flight on a 256-CU device, so each
    # workgroup loops over its chunks with the next one prefetched
    ((3, 2), 4, 64, 64, [1000, 513, 256, 3], "bf16"),
    ((3, 2, 2), 2, 128, 128, [1100, 700], "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]}-B{c[1]}-H{c[2]}-Dh{c[3]}-{c[5]}")
def test_tree_attention(case):
    s, B, H, Dh, Ls, dtype = case
    rng = np.random.default_rng(sum(s) * 1000 + B * 100 + H * 10 + Dh + len(Ls))
    K = len(s)
    spec = cartesian_ranks(s)
    Lmax = max(Ls) + K + 1 + 64
    topo, q, kt, vt, kc, vc = _case(rng, spec, K, B, H, Dh, Ls, Lmax, dtype)
    scale = 1.0 / np.sqrt(Dh)
    g = _run(topo, q, kt, vt, kc, vc, Ls, K, dtype, scale)
    o = _oracle(topo, q, kt, vt, kc, vc, Ls, scale)
    tol = 2e-2 if dtype == "bf16" else 1e-5
    assert_close(g, o, tol, "attention")
    # elementwise: bf16 P rounding bounds the per-element error
    assert np.max(np.abs(g - o)) < (5e-2 if dtype == "bf16" else 1e-4)


# Several sequences whose prefix chunks outnumber the workgroups: balanced
# ranges over every (sequence, head)'s chunks, some ranges spanning several
# heads or sequences. (tree s, B, H, prefix lengths, Lmax)
BALANCED = [
    ((3, 2), 2, 128, [4000, 600], 4200),               # one query tile
    ((3, 2, 2, 1, 1), 8, 32, [2048, 512, 1700, 900, 64, 2000, 1, 1300], 2120),  # three tiles
    ((2, 2), 2, 128, [0, 100], 4200),                  # fewer chunks than workgroups, an empty prefix
    ((4, 3), 3, 96, [0, 2000, 257], 2100),             # two tiles, a sequence with no chunks first
    # the largest batch a call takes (64 sequences, one chunk count a lane),
    # lengths spread over [0, Lmax] with empty and full prefixes among them
    ((3, 2, 2, 1, 1), 64, 4, [(37 * i * i + 11 * i) % 2101 for i in range(63)] + [2100], 2100),
    # many short prefixes (one or two chunks a (sequence, head)) beside one
    # long one: narrow ranges, many of which end inside a (sequence, head)'s
    # start weight and leave its first chunk to the next range
    ((3, 2, 2, 1, 1), 16, 32, [(53 * i * i + 29 * i) % 300 + 1 for i in range(15)] + [1300], 1300),
]


@pytest.mark.parametrize("case", BALANCED, ids=lambda c: f"s{c[0]}-B{c[1]}-H{c[2]}-L{c[4]}")
def test_tree_attention_balanced(case):
    s, B, H, Ls, Lmax = case
    Dh = 128
    rng = np.random.default_rng(sum(s) * 1000 + B * 100 + H)
    K = len(s)
    topo, q, kt, vt, kc, vc = _case(rng, cartesian_ranks(s), K, B, H, Dh, Ls, Lmax, "bf16")
    scale = 1.0 / np.sqrt(Dh)
    g = _run(topo, q, kt, vt, kc, vc, Ls, K, "bf16", scale)
    o = _oracle(topo, q, kt, vt, kc, vc, Ls, scale)
    assert_close(g, o, 2e-2, "attention balanced")
    assert np.max(np.abs(g - o)) < 5e-2


def test_tree_attention_sparse_tree():
    rng = np.random.default_rng(11)
    spec = np.array([[0, -1, -1], [1, -1, -1], [2, -1, -1], [0, 0, -1], [0, 1, -1], [2, 0, -1],
                     [0, 0, 0], [0, 0, 1], [2, 0, 0]], dtype=np.int32)
    K, B, H, Dh, Ls = 3, 2, 2, 128, [33, 600]
    Lmax = 700
    topo, q, kt, vt, kc, vc = _case(rng, spec, K, B, H, Dh, Ls, Lmax, "bf16")
    g = _run(topo, q, kt, vt, kc, vc, Ls, K, "bf16", 0.1)
    o = _oracle(topo, q, kt, vt, kc, vc, Ls, 0.1)
    assert_close(g, o, 2e-2, "attention sparse")
