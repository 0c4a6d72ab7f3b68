"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test ties one oracle function to something other than itself: a value
the pages print (fixtures under tests/golden/), a closed form, a textbook or
library routine, an invariant, or brute force on tiny inputs.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import heads as OH
from oracle import numerics as ON
from oracle import posterior as OP
from oracle import sparse_tree as OS
from oracle import tree as OT
from oracle import verifier as OV
from workloads import cartesian_ranks, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- numerics

def test_round_bf16_matches_bit_rounding():
    # Independent implementation: integer rounding of the float32 bit pattern.
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    bits = f32_to_bf16_bits(x)
    ref = ON.widen(bits)
    assert np.array_equal(ON.round_bf16(x.astype(np.float64)), ref)


def test_round_bf16_ties_to_even():
    one = 1.0
    assert ON.round_bf16(np.array([one + 2.0 ** -8]))[0] == 1.0             # halfway, even below
    assert ON.round_bf16(np.array([one + 3 * 2.0 ** -8]))[0] == one + 2.0 ** -6  # halfway, even above
    assert ON.round_bf16(np.array([one + 2.0 ** -7]))[0] == one + 2.0 ** -7  # representable
    assert ON.round_bf16(np.array([0.0]))[0] == 0.0


def test_widen_bf16_exact():
    assert ON.widen(np.array([0x3F80], dtype=np.uint16))[0] == 1.0
    assert ON.widen(np.array([0xC000], dtype=np.uint16))[0] == -2.0
    assert ON.widen(np.array([0x3FC0], dtype=np.uint16))[0] == 1.5


# -------------------------------------------------------------------- heads

def test_silu_closed_forms():
    assert OH.silu(np.array([0.0]))[0] == 0.0
    assert math.isclose(OH.silu(np.array([1.0]))[0], 1.0 / (1.0 + math.exp(-1.0)), rel_tol=1e-15)
    x = np.linspace(-8, 8, 101)
    # x*sigmoid(x) - (-x)*sigmoid(-x) = x
    assert np.allclose(OH.silu(x) - OH.silu(-x), x, atol=1e-14)
    # x*sigmoid(x) = x * expit(x) (library sigmoid)
    assert np.allclose(OH.silu(x), x * scipy.special.expit(x), rtol=1e-14, atol=1e-300)
    assert OH.silu(np.array([50.0]))[0] == pytest.approx(50.0, rel=1e-15)


def test_heads_identity_at_init():
    # "Medusa 深读" §3.1: W1 = 0 and W2 = the LM head make every head repeat
    # the LM head exactly ("Medusa Part I", Part 3 initialisation).
    rng = np.random.default_rng(1)
    B, d, V, K = 2, 32, 40, 3
    h = rng.standard_normal((B, d))
    W_lm = rng.standard_normal((V, d)) / np.sqrt(d)
    W1 = np.zeros((K, d, d))
    W2 = np.stack([W_lm] * K)
    b1 = np.zeros((K, d))
    z, logits = OH.heads_forward(h, W1, W2, b1)
    for k in range(K):
        assert np.array_equal(z[:, k], h)
        assert np.array_equal(logits[:, k], OH.lm_head(W_lm, h))


def test_heads_single_entry_weights():
    # One nonzero W1 entry (k, i, j) = a: only z_i changes, by silu(a * h_j);
    # one nonzero W2 entry (v, i) = c: only logit v is nonzero, = c * z_i.
    # A transposed operand or dropped residual fails this.
    rng = np.random.default_rng(2)
    d, V, K = 8, 11, 2
    h = rng.standard_normal((1, d))
    W1 = np.zeros((K, d, d))
    W2 = np.zeros((K, V, d))
    a, c = 1.7, -0.6
    W1[1, 2, 5] = a
    W2[1, 7, 2] = c
    z, logits = OH.heads_forward(h, W1, W2)
    expect_z = h[0].copy()
    expect_z[2] = h[0, 2] + a * h[0, 5] / (1.0 + math.exp(-a * h[0, 5]))
    assert np.allclose(z[0, 1], expect_z, rtol=1e-15, atol=0)
    assert np.array_equal(z[0, 0], h[0])
    expect_l = np.zeros(V)
    expect_l[7] = c * expect_z[2]
    assert np.allclose(logits[0, 1], expect_l, rtol=1e-15, atol=0)
    assert np.array_equal(logits[0, 0], np.zeros(V))


def test_heads_bias_enters_inside_silu():
    d, V = 4, 3
    h = np.array([[0.5, -1.0, 2.0, 0.0]])
    W1 = np.zeros((1, d, d))
    b1 = np.array([[0.0, 0.0, 0.0, 1.25]])
    W2 = np.zeros((1, V, d))
    z, _ = OH.heads_forward(h, W1, W2, b1)
    assert z[0, 0, 3] == pytest.approx(1.25 / (1.0 + math.exp(-1.25)), rel=1e-15)


def test_top_s_brute_force_with_ties():
    rng = np.random.default_rng(3)
    for _ in range(200):
        V = int(rng.integers(3, 12))
        logits = rng.integers(-3, 3, size=V).astype(np.float64)   # many ties
        s = int(rng.integers(1, V))
        ids, vals = OH.top_s(logits, s)
        ref = sorted(range(V), key=lambda i: (-logits[i], i))[:s]
        assert list(ids) == ref
        assert np.array_equal(vals, logits[ref])


def test_log_sum_exp_library():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(1000) * 30
    assert OH.log_sum_exp(x) == pytest.approx(scipy.special.logsumexp(x), rel=1e-14)


# --------------------------------------------------------------------- tree

def test_node_count_printed_example():
    g = _golden("tree_count_example.json")
    s = g["s"]
    assert OT.node_count(s) == g["tree_nodes"]
    assert OT.path_count(s) == g["sequences"]
    assert OT.path_count(s) * len(s) == g["unshared_nodes"]
    topo = OT.topology(cartesian_ranks(s), len(s))
    assert topo.T == g["tree_nodes"] + 1
    assert topo.P == g["sequences"]


@pytest.mark.parametrize("s,N", [((2, 2, 2), 14), ((3, 2, 2, 1, 1), 45), ((4, 3, 2, 2, 1), 136)])
def test_node_count_workload_trees(s, N):
    assert OT.node_count(s) == N
    # brute force: distinct non-empty prefixes of all full rank paths
    prefixes = set()
    for full in itertools.product(*[range(x) for x in s]):
        for k in range(1, len(s) + 1):
            prefixes.add(full[:k])
    assert len(prefixes) == N
    topo = OT.topology(cartesian_ranks(s), len(s))
    assert topo.T == N + 1 and topo.P == OT.path_count(s)


def _random_spec(rng, K, smax, n_target):
    nodes = set()
    frontier = [()]
    while len(nodes) < n_target and frontier:
        t = frontier[int(rng.integers(len(frontier)))]
        if len(t) == K or all(t + (x,) in nodes for x in range(smax)):
            frontier.remove(t)
            continue
        r = int(rng.integers(smax))
        c = t + (r,)
        if c not in nodes:
            nodes.add(c)
            frontier.append(c)
    rows = sorted(nodes, key=lambda t: (len(t), t))
    spec = np.full((len(rows), K), -1, dtype=np.int32)
    for i, t in enumerate(rows):
        spec[i, :len(t)] = t
    return spec


def test_mask_is_prefix_relation():
    rng = np.random.default_rng(5)
    for trial in range(30):
        K = int(rng.integers(1, 6))
        spec = _random_spec(rng, K, 4, int(rng.integers(1, 40)))
        topo = OT.topology(spec, K)
        tuples = [()] + OT.spec_tuples(spec)
        for i, ti in enumerate(tuples):
            for j, tj in enumerate(tuples):
                want = len(tj) <= len(ti) and ti[:len(tj)] == tj
                assert topo.mask[i, j] == want
            assert topo.depth[i] == len(ti)


def test_retrieve_lists_leaf_paths():
    rng = np.random.default_rng(6)
    for trial in range(30):
        K = int(rng.integers(1, 6))
        spec = _random_spec(rng, K, 3, int(rng.integers(1, 30)))
        topo = OT.topology(spec, K)
        tuples = [()] + OT.spec_tuples(spec)
        leaves = [t for t in tuples[1:] if not any(u[:-1] == t for u in tuples[1:])]
        assert topo.P == len(leaves)
        assert [tuples[row[row >= 0][-1]] for row in topo.retrieve] == sorted(leaves)
        for row in topo.retrieve:
            nodes = [int(n) for n in row if n >= 0]
            assert nodes[0] == 0
            leaf = tuples[nodes[-1]]
            assert [tuples[n] for n in nodes] == [leaf[:k] for k in range(len(leaf) + 1)]
            assert all(n == -1 for n in row[len(nodes):])


def test_check_spec_rejects_bad_trees():
    assert OT.check_spec([(0,), (1,), (0, 0)]) is None
    assert OT.check_spec([(0,), (0, 0), (1,)]) == "not in canonical order"
    assert OT.check_spec([(0,), (1, 0)]) == "not prefix-closed"
    assert OT.check_spec([(0,), (0,)]) == "duplicate rank path"
    assert OT.check_spec([(0,), (0, 0)], K=1) == "rank path deeper than K"


def test_positions_shared_per_depth():
    topo = OT.topology(cartesian_ranks((3, 2, 2, 1, 1)), 5)
    pos = OT.position_ids(topo, 2048)
    for k in range(6):
        assert set(pos[topo.depth == k]) == {2048 + k}


def test_topk_tokens_follow_rank_paths():
    topo = OT.topology(cartesian_ranks((3, 2, 2)), 3)
    ids = np.array([[10, 11, 12], [20, 21, -5], [30, 31, -5]])
    tok = OT.draft_tokens_topk(topo, 7, ids)
    tuples = [()] + topo.tuples
    assert tok[0] == 7
    for n in range(1, topo.T):
        assert tok[n] == ids[len(tuples[n]) - 1, tuples[n][-1]]


def test_inverse_cdf_definition():
    w = np.array([0.0, 1.0, 0.0, 3.0, 0.0])
    # C = [0, 1, 1, 4, 4]; smallest x with C(x) > u * 4
    assert OT.inverse_cdf(w, 0.0) == 1
    assert OT.inverse_cdf(w, 0.2499) == 1
    assert OT.inverse_cdf(w, 0.25) == 3
    assert OT.inverse_cdf(w, 0.9999999) == 3
    # empirical law of the draw equals the normalised weights
    rng = np.random.default_rng(7)
    w = rng.random(6)
    u = rng.random(60000)
    draws = np.array([OT.inverse_cdf(w, x) for x in u])
    counts = np.bincount(draws, minlength=6)
    assert scipy.stats.chisquare(counts, w / w.sum() * counts.sum()).pvalue > 1e-4


# ---------------------------------------------------------------- verifier

def _tiny_layer(rng, d=32, H=2, Dh=16, V=50, L=7, Lmax=16, bf16=False):
    def st(x):
        return f32_to_bf16_bits(x.astype(np.float32)) if bf16 else x
    E = st(rng.standard_normal((V, d)))
    W_qkv = st(rng.standard_normal((3 * d, d)) / np.sqrt(d))
    W_o = st(rng.standard_normal((d, d)) / np.sqrt(d))
    W_lm = st(rng.standard_normal((V, d)) / np.sqrt(d))
    kc = np.zeros((H, Lmax, Dh))
    vc = np.zeros((H, Lmax, Dh))
    kc[:, :L] = rng.standard_normal((H, L, Dh))
    vc[:, :L] = rng.standard_normal((H, L, Dh))
    if bf16:
        kc, vc = st(kc), st(vc)
    return E, W_qkv, W_o, W_lm, kc, vc


@pytest.mark.parametrize("bf16", [False, True])
def test_tree_attention_equals_path_attention(bf16):
    # "Medusa 深读" §6.1 / "Medusa: Faster LLM text generation", Tree
    # attention: under the tree mask and shared depth positions, each node's
    # output is ordinary causal attention over prefix + its own path.
    rng = np.random.default_rng(8)
    H, Dh, L, theta = 2, 16, 7, 10000.0
    for trial in range(6):
        K = int(rng.integers(1, 5))
        spec = _random_spec(rng, K, 3, int(rng.integers(1, 20)))
        topo = OT.topology(spec, K)
        E, W_qkv, W_o, W_lm, kc, vc = _tiny_layer(rng, H=H, Dh=Dh, L=L, bf16=bf16)
        tok = rng.integers(0, 50, size=topo.T)
        pos = OT.position_ids(topo, L)
        out = OV.verifier_forward(E, W_qkv, W_o, W_lm, tok, pos, topo.mask, kc, vc, L, H, Dh,
                                  theta, bf16)
        for n in range(topo.T):
            path_tokens = tok[topo.path(n)]
            ref = OV.path_attention(path_tokens, E, W_qkv, kc, vc, L, H, Dh, theta,
                                    1.0 / np.sqrt(Dh), bf16)
            assert np.allclose(out["o"][n], ref, rtol=0, atol=1e-12)


def test_tree_attention_sibling_leak_is_caught():
    # A planted mistake (siblings visible) must break path equivalence.
    rng = np.random.default_rng(9)
    H, Dh, L, theta = 2, 16, 7, 10000.0
    topo = OT.topology(cartesian_ranks((2, 2)), 2)
    E, W_qkv, W_o, W_lm, kc, vc = _tiny_layer(rng, H=H, Dh=Dh, L=L)
    tok = rng.integers(0, 50, size=topo.T)
    pos = OT.position_ids(topo, L)
    leaky = np.tril(np.ones((topo.T, topo.T), dtype=np.uint8))
    out = OV.verifier_forward(E, W_qkv, W_o, W_lm, tok, pos, leaky, kc, vc, L, H, Dh, theta,
                              False)
    n = 2   # second depth-1 node: the leaky mask lets it see node 1
    ref = OV.path_attention(tok[topo.path(n)], E, W_qkv, kc, vc, L, H, Dh, theta,
                            1.0 / np.sqrt(Dh), False)
    assert not np.allclose(out["o"][n], ref, atol=1e-6)


def test_attention_uniform_when_query_zero():
    # q = 0 gives equal weights: the output is the plain mean of the visible
    # values (prefix rows plus masked tree rows).
    rng = np.random.default_rng(10)
    topo = OT.topology(cartesian_ranks((2, 2)), 2)
    T, H, Dh, L = topo.T, 2, 8, 5
    q = np.zeros((T, H, Dh))
    kt = rng.standard_normal((T, H, Dh))
    vt = rng.standard_normal((T, H, Dh))
    kc = rng.standard_normal((H, 9, Dh))
    vc = rng.standard_normal((H, 9, Dh))
    o = OV.tree_attention(q, kt, vt, kc, vc, L, topo.mask, 0.3)
    for i in range(T):
        for h in range(H):
            vis = np.concatenate([vc[h, :L], vt[np.nonzero(topo.mask[i])[0], h]])
            assert np.allclose(o[i, h], vis.mean(axis=0), atol=1e-14)


def test_rope_rotation_properties():
    rng = np.random.default_rng(11)
    H, Dh, theta = 3, 16, 10000.0
    x = rng.standard_normal((5, H, Dh))
    # position 0 is the identity; every (i, i+Dh/2) pair keeps its norm
    assert np.allclose(OV.rope(x, np.zeros(5), theta), x, atol=0)
    pos = rng.integers(0, 5000, size=5)
    r = OV.rope(x, pos, theta)
    half = Dh // 2
    assert np.allclose(r[..., :half] ** 2 + r[..., half:] ** 2,
                       x[..., :half] ** 2 + x[..., half:] ** 2, rtol=1e-12)
    # the dot product of rotated q, k depends only on the position difference
    q = rng.standard_normal((1, 1, Dh))
    k = rng.standard_normal((1, 1, Dh))
    a = np.sum(OV.rope(q, np.array([100]), theta) * OV.rope(k, np.array([37]), theta))
    b = np.sum(OV.rope(q, np.array([1063]), theta) * OV.rope(k, np.array([1000]), theta))
    assert a == pytest.approx(b, rel=1e-9)
    # pair 0 rotates by exactly `pos` radians (theta^0 = 1)
    e = np.zeros((1, 1, Dh))
    e[0, 0, 0] = 1.0
    r = OV.rope(e, np.array([2]), theta)
    assert r[0, 0, 0] == pytest.approx(math.cos(2.0), abs=1e-15)
    assert r[0, 0, half] == pytest.approx(math.sin(2.0), abs=1e-15)


def test_residual_and_lm_head_special_cases():
    rng = np.random.default_rng(12)
    H, Dh, L = 2, 16, 7
    d = H * Dh
    topo = OT.topology(cartesian_ranks((2,)), 1)
    E, W_qkv, W_o, W_lm, kc, vc = _tiny_layer(rng, d=d, H=H, Dh=Dh, L=L)
    tok = np.array([3, 4, 5])
    pos = OT.position_ids(topo, L)
    # W_o = 0: y is exactly the embedding row (residual path)
    out = OV.verifier_forward(E, W_qkv, np.zeros((d, d)), W_lm, tok, pos, topo.mask, kc, vc,
                              L, H, Dh, 10000.0, False)
    assert np.array_equal(out["y"], E[tok])
    assert np.allclose(out["logits"], E[tok] @ W_lm.T, rtol=1e-15)
    # W_o = identity: y = x + o
    out = OV.verifier_forward(E, W_qkv, np.eye(d), W_lm, tok, pos, topo.mask, kc, vc, L, H,
                              Dh, 10000.0, False)
    assert np.allclose(out["y"], E[tok] + out["o"].reshape(3, d), atol=1e-14)


def test_entropy_and_argmax_library():
    rng = np.random.default_rng(13)
    logits = rng.standard_normal((7, 300)) * 3
    for tau in (1.0, 0.7):
        p, H, am = OV.row_distribution(logits, tau)
        assert np.allclose(p, scipy.special.softmax(logits / tau, axis=-1), rtol=1e-13)
        assert np.allclose(H, scipy.stats.entropy(p, axis=-1), rtol=1e-12)
        assert np.array_equal(am, np.argmax(logits, axis=-1))
    p, H, am = OV.row_distribution(np.zeros((1, 4)), 1.0)
    assert H[0] == pytest.approx(math.log(4), rel=1e-15)
    tie = np.array([[1.0, 3.0, 3.0, 0.0]])
    assert OV.row_distribution(tie, 1.0)[2][0] == 1


# ---------------------------------------------------------------- posterior

def test_typical_closed_forms():
    # "Medusa 深读" §5: accept iff p > min(eps, delta * exp(-H)).
    eps, delta = 0.09, 0.3
    # uniform over 4: H = ln 4, threshold = min(0.09, 0.075) = 0.075 < 0.25
    p, H, _ = OV.row_distribution(np.zeros((1, 4)), 1.0)
    assert min(eps, delta * math.exp(-H[0])) == pytest.approx(0.075, rel=1e-14)
    assert all(OP.typical_accepts(p[0, x], H[0], eps, delta) for x in range(4))
    # one-hot: H = 0, threshold = min(0.09, 0.3) = 0.09; only the hot token passes
    p, H, _ = OV.row_distribution(np.array([[0.0, -np.inf, -np.inf, -np.inf]]), 1.0)
    assert H[0] == 0.0
    assert OP.typical_accepts(p[0, 0], H[0], eps, delta)
    assert not any(OP.typical_accepts(p[0, x], H[0], eps, delta) for x in (1, 2, 3))
    # strict inequality at the threshold
    assert not OP.typical_accepts(0.09, 0.0, eps, delta)
    assert OP.typical_accepts(np.nextafter(0.09, 1.0), 0.0, eps, delta)
    # high entropy lowers the bar: delta * exp(-H) below eps
    assert OP.typical_accepts(0.01, 5.0, eps, delta)       # thr = 0.3 e^-5 = 0.00202
    assert not OP.typical_accepts(0.002, 5.0, eps, delta)


def _planted_tree_case(rng, s, V=20, rho=0.6):
    K = len(s)
    topo = OT.topology(cartesian_ranks(s), K)
    tok = rng.integers(0, V, size=topo.T).astype(np.int32)
    argmax = rng.integers(0, V, size=topo.T).astype(np.int32)
    # plant agreement: with prob rho make some child of v carry argmax[v]
    for v in range(topo.T):
        kids = topo.children(v)
        if kids and rng.random() < rho:
            tok[kids[int(rng.integers(len(kids)))]] = argmax[v]
    return topo, tok, argmax


def test_greedy_equals_sequential_argmax_matching():
    # "Medusa Part I", Part 2: accept while the draft equals the target
    # argmax; the first mismatch ends the prefix. Brute force per path.
    rng = np.random.default_rng(14)
    for trial in range(300):
        s = tuple(int(x) for x in rng.integers(1, 4, size=int(rng.integers(1, 5))))
        topo, tok, am = _planted_tree_case(rng, s)
        acc = OP.accept_greedy(topo, tok, am)
        post = OP.posterior_deterministic(topo, tok, acc, am)
        best_len, best_tokens = -1, None
        for row in topo.retrieve:
            nodes = [int(n) for n in row if n >= 0]
            n_ok = 0
            for j in range(1, len(nodes)):
                if tok[nodes[j]] == am[nodes[j - 1]]:
                    n_ok += 1
                else:
                    break
            if n_ok > best_len:
                best_len, best_tokens = n_ok, [int(tok[n]) for n in nodes[:n_ok + 1]]
                best_next = int(am[nodes[n_ok]])
        assert post["accept_len"] == best_len
        assert list(post["out_tokens"][:best_len + 1]) == best_tokens
        assert all(t == -1 for t in post["out_tokens"][best_len + 1:])
        assert post["next_root"] == best_next
        assert post["out_tokens"][0] == tok[0]


def test_typical_low_temperature_is_greedy():
    rng = np.random.default_rng(15)
    for trial in range(40):
        topo = OT.topology(cartesian_ranks((3, 2, 2)), 3)
        V = 30
        logits = rng.standard_normal((topo.T, V))
        tok = rng.integers(0, V, size=topo.T).astype(np.int32)
        am = np.argmax(logits, axis=-1)
        for v in range(topo.T):
            kids = topo.children(v)
            if kids and rng.random() < 0.7:
                tok[kids[0]] = am[v]
        p, H, am2 = OV.row_distribution(logits, 1e-4)
        acc_t = OP.accept_typical(topo, tok, p, H, 0.09, 0.3)
        acc_g = OP.accept_greedy(topo, tok, am2)
        assert np.array_equal(acc_t, acc_g)


def test_longest_prefix_two_formulations_agree():
    rng = np.random.default_rng(16)
    for trial in range(600):
        K = int(rng.integers(1, 6))
        if trial % 2:
            s = tuple(int(x) for x in rng.integers(1, 4, size=K))
            spec = cartesian_ranks(s)
        else:   # sparse trees with leaves at several depths
            spec = _random_spec(rng, K, 3, int(rng.integers(1, 25)))
        topo = OT.topology(spec, K)
        acc = rng.random(topo.T) < rng.uniform(0.2, 0.95)
        acc[0] = True
        alen, pbest = OP.longest_prefix_paths(topo, acc)
        ok, nbest = OP.longest_prefix_nodes(topo, acc)
        assert alen[pbest] == topo.depth[nbest]
        assert topo.retrieve[pbest, alen[pbest]] == nbest
        assert OP.first_path_through(topo, nbest) == pbest


@pytest.mark.parametrize("mode", ["greedy", "typical", "exact"])
def test_first_token_always_committed(mode):
    # "Medusa 深读" §5 / "Medusa Part I", Part 2: each step commits at least
    # the root token, even when every draft is rejected.
    rng = np.random.default_rng(17)
    topo = OT.topology(cartesian_ranks((2, 2)), 2)
    V = 12
    tok = np.array([5] + [0] * (topo.T - 1), dtype=np.int32)
    logits = np.full((topo.T, V), -30.0)
    logits[:, 1] = 30.0            # target puts all mass on token 1; drafts carry 0
    p, H, am = OV.row_distribution(logits, 1.0)
    if mode == "greedy":
        post = OP.posterior_deterministic(topo, tok, OP.accept_greedy(topo, tok, am), am)
    elif mode == "typical":
        post = OP.posterior_deterministic(
            topo, tok, OP.accept_typical(topo, tok, p, H, 0.09, 0.3), am)
    else:
        q = np.zeros((2, V))
        q[:, 0] = 1.0
        post = OP.posterior_exact(topo, tok, p, q, rng.random(topo.T), rng.random(topo.T))
    assert post["accept_len"] == 0
    assert post["out_tokens"][0] == 5
    assert post["next_root"] == 1


def _exact_trial_setup(V=6):
    rng = np.random.default_rng(18)
    s = (2, 2)
    topo = OT.topology(cartesian_ranks(s), 2)
    # a Markov target: p(. | node) depends on the node's token (and depth)
    table = [scipy.special.softmax(rng.standard_normal((V, V)) * 1.2, axis=-1) for _ in range(3)]
    root_tok = 2
    q = np.stack([scipy.special.softmax(rng.standard_normal(V), axis=-1) for _ in range(2)])
    return topo, table, root_tok, q


def _exact_run(topo, table, root_tok, q, rng, trials):
    V = q.shape[1]
    pairs = np.zeros((V, V), dtype=np.int64)
    firsts = np.zeros(V, dtype=np.int64)
    lens = np.zeros(3, dtype=np.int64)
    hl = np.log(q)
    for _ in range(trials):
        u = rng.random((3, topo.T))
        tok = OT.draft_tokens_sampled(topo, root_tok, hl, u[0])
        p_rows = np.stack([table[topo.depth[n]][tok[n]] for n in range(topo.T)])
        post = OP.posterior_exact(topo, tok, p_rows, q, u[1], u[2])
        a = post["accept_len"]
        lens[a] += 1
        gen = [int(t) for t in post["out_tokens"][1:a + 1]] + [post["next_root"]]
        y1 = gen[0]
        if len(gen) >= 2:
            y2 = gen[1]
        else:   # continue autoregressively from the target itself
            y2 = int(rng.choice(V, p=table[1][y1]))
        firsts[y1] += 1
        pairs[y1, y2] += 1
    return firsts, pairs, lens


def test_exact_rule_preserves_target_distribution():
    # "Medusa 深读" §3.2 / "Medusa: Faster LLM text generation", Acceptance
    # rules: p/q acceptance with (p - q)+ resampling, drafts sampled from q,
    # reproduces the target's distribution.
    topo, table, root_tok, q = _exact_trial_setup()
    V = q.shape[1]
    rng = np.random.default_rng(19)
    n = 60000
    firsts, pairs, lens = _exact_run(topo, table, root_tok, q, rng, n)
    p1 = table[0][root_tok]
    assert scipy.stats.chisquare(firsts, p1 * n).pvalue > 1e-4
    joint = p1[:, None] * table[1]
    exp = joint.ravel() * n
    keep = exp > 5
    obs = pairs.ravel()[keep]
    assert scipy.stats.chisquare(obs, exp[keep] * obs.sum() / exp[keep].sum()).pvalue > 1e-4
    assert lens[1] + lens[2] > 0   # some drafts were accepted


def test_exact_rule_catches_missing_residual(monkeypatch):
    # Planted mistake: resampling from p instead of the residual biases the law.
    topo, table, root_tok, q = _exact_trial_setup()
    orig = OT.inverse_cdf

    def wrong_posterior(topo_, tok, p_rows, q_, ua, ur):
        v = 0
        while True:
            kids = topo_.children(v)
            if not kids:
                return OP._result(topo_, tok, v, orig(p_rows[v], float(ur[v])))
            qq = q_[topo_.depth[v]]
            taken = None
            for c in kids:
                x = int(tok[c])
                if float(ua[c]) * qq[x] < p_rows[v][x]:
                    taken = c
                    break
            if taken is None:
                return OP._result(topo_, tok, v, orig(p_rows[v], float(ur[v])))
            v = taken

    monkeypatch.setattr(OP, "posterior_exact", wrong_posterior)
    rng = np.random.default_rng(20)
    n = 30000
    firsts, _, _ = _exact_run(topo, table, root_tok, q, rng, n)
    p1 = table[0][root_tok]
    assert scipy.stats.chisquare(firsts, p1 * n).pvalue < 1e-6


def test_exact_special_cases():
    rng = np.random.default_rng(21)
    topo = OT.topology(cartesian_ranks((2, 2)), 2)
    V = 5
    qv = scipy.special.softmax(rng.standard_normal(V))
    q = np.stack([qv, qv])
    # q = p everywhere: every draft is accepted
    for _ in range(200):
        u = rng.random((3, topo.T))
        tok = OT.draft_tokens_sampled(topo, 0, np.log(q), u[0])
        post = OP.posterior_exact(topo, tok, np.stack([qv] * topo.T), q, u[1], u[2])
        assert post["accept_len"] == 2
    # disjoint supports: nothing is accepted and the output follows p
    q2 = np.zeros((2, V))
    q2[:, :2] = 0.5
    p = np.zeros(V)
    p[2:] = [0.2, 0.3, 0.5]
    counts = np.zeros(V)
    for _ in range(6000):
        u = rng.random((3, topo.T))
        tok = OT.draft_tokens_sampled(topo, 0, np.log(np.maximum(q2, 1e-300)), u[0])
        post = OP.posterior_exact(topo, tok, np.stack([p] * topo.T), q2, u[1], u[2])
        assert post["accept_len"] == 0
        counts[post["next_root"]] += 1
    assert counts[:2].sum() == 0
    assert scipy.stats.chisquare(counts[2:], p[2:] * 6000).pvalue > 1e-4


def test_commit_appends_path_rows():
    rng = np.random.default_rng(22)
    topo = OT.topology(cartesian_ranks((2, 2, 1)), 3)
    H, Dh, L, T = 2, 4, 6, topo.T
    kt = rng.standard_normal((T, H, Dh))
    vt = rng.standard_normal((T, H, Dh))
    y = rng.standard_normal((T, 8))
    kc = np.zeros((H, 12, Dh))
    vc = np.zeros((H, 12, Dh))
    last = topo.retrieve[1, 3]
    kc2, vc2, L2, hn = OP.commit(topo, last, kt, vt, y, kc, vc, L)
    path = topo.retrieve[1]
    assert L2 == L + 4
    for i, n in enumerate(path):
        assert np.array_equal(kc2[:, L + i], kt[n])
        assert np.array_equal(vc2[:, L + i], vt[n])
    assert np.all(kc2[:, :L] == 0) and np.all(kc2[:, L + 4:] == 0)
    assert np.array_equal(hn, y[last])


# --------------------------------------------------------------- sparse tree

def test_sparse_tree_worked_example():
    g = _golden("sparse_tree_worked_example.json")
    a = np.array(g["a"])
    picks = OS.greedy_tree(a, g["budget"])
    assert [tuple(r + 1 for r in t) for t in picks] == [tuple(t) for t in g["order"]]
    assert [OS.path_weight(a, t) for t in picks] == pytest.approx(g["weights"], rel=1e-12)
    assert OS.expected_cover(a, picks) == pytest.approx(g["expected_cover"], rel=1e-12)
    spec = OS.to_spec(picks, a.shape[0])
    assert OT.check_spec(OT.spec_tuples(spec), a.shape[0]) is None


def test_sparse_tree_cover_is_tail_sum():
    # E[L] = sum_k P(L >= k): simulate independent rank draws per head and
    # measure the depth the tree covers.
    rng = np.random.default_rng(23)
    a = np.array([[0.6, 0.25, 0.1], [0.5, 0.3, 0.1], [0.4, 0.3, 0.2]])
    picks = OS.greedy_tree(a, 7)
    tree = set(picks)
    n = 40000
    probs = np.concatenate([a, 1 - a.sum(axis=1, keepdims=True)], axis=1)
    depth_sum = 0
    for _ in range(n):
        ranks = [int(rng.choice(4, p=probs[k])) for k in range(3)]
        d = 0
        while d < 3 and tuple(ranks[:d + 1]) in tree:
            d += 1
        depth_sum += d
    assert depth_sum / n == pytest.approx(OS.expected_cover(a, picks), abs=0.02)


# ---------------------------------------------------------------- q/k/v block order

@pytest.mark.parametrize("blk", [0, 1, 2])
def test_qkv_single_entry_block_and_head(blk):
    # W_qkv rows are [q | k | v], each block d rows in head-major order
    # (row h*Dh + i is head h, lane i). A single nonzero weight in block blk
    # at (blk*d + h*Dh + i, j), fed the one-hot row e_j at position 0 (where
    # the rotation is the identity), must show up in that block's tensor at
    # [h, i] alone; the other two tensors stay zero.
    H, Dh = 3, 8
    d = H * Dh
    h_, i_, j_ = 2, 5, 7
    W = np.zeros((3 * d, d))
    W[blk * d + h_ * Dh + i_, j_] = 1.5
    x = np.zeros((1, d))
    x[0, j_] = 1.0
    q, k, v = OV.qkv_project(x, W, np.array([0]), H, Dh, 10000.0, bf16=False)
    outs = [q, k, v]
    for b, t in enumerate(outs):
        want = np.zeros((1, H, Dh))
        if b == blk:
            want[0, h_, i_] = 1.5
        assert np.array_equal(t, want), (blk, b)


@pytest.mark.parametrize("blk", [0, 1, 2])
def test_qkv_single_entry_rotation_stays_in_pair(blk):
    # At a nonzero position q and k rotate pairs (i, i + Dh/2) of one head and
    # v does not rotate: the single weight's output stays in its own head and
    # in lanes {i, partner} of its own block (v: lane i alone, unchanged),
    # and the pair's norm is kept.
    H, Dh = 2, 8
    d = H * Dh
    h_, i_, j_ = 1, 6, 3
    partner = i_ - Dh // 2
    W = np.zeros((3 * d, d))
    W[blk * d + h_ * Dh + i_, j_] = 2.0
    x = np.zeros((1, d))
    x[0, j_] = 1.0
    outs = OV.qkv_project(x, W, np.array([37]), H, Dh, 10000.0, bf16=False)
    for b, t in enumerate(outs):
        if b != blk:
            assert not np.any(t), (blk, b)
            continue
        nz = set(zip(*np.nonzero(t[0])))
        if blk == 2:
            assert nz == {(h_, i_)} and t[0, h_, i_] == 2.0
        else:
            assert nz <= {(h_, i_), (h_, partner)} and len(nz) == 2
            assert np.isclose(np.hypot(t[0, h_, i_], t[0, h_, partner]), 2.0, rtol=1e-14)


# ---------------------------------------------------------------- margin helpers

def test_topk_margin_closed_forms():
    row = np.array([5.0, 3.0, 3.5, 1.0, -2.0])
    # sorted 5, 3.5, 3, 1, -2: top-1 needs the gap 5-3.5, top-2 also 3.5-3
    assert OH.topk_margin(row, 1) == 1.5
    assert OH.topk_margin(row, 2) == 0.5
    assert OH.topk_margin(row, 3) == 0.5
    assert OH.topk_margin(np.array([2.0, 2.0, 1.0]), 1) == 0.0
    assert OH.topk_margin(np.array([4.0, 1.0, 0.0]), 2) == 1.0


def test_argmax_margin_closed_forms():
    assert OP.argmax_margin(np.array([1.0, 4.0, 2.0])) == 2.0
    assert OP.argmax_margin(np.array([3.0, -1.0, 3.0])) == 0.0
    assert OP.argmax_margin(np.array([-5.0, -2.5])) == 2.5


def test_decision_margins_closed_forms():
    topo = OT.topology(np.array([[0], [1]], dtype=np.int32), 1)
    logits = np.array([[1.0, 4.0, 2.0], [0, 0, 0], [0, 0, 0]])
    tokens = np.array([9, 0, 1])
    m = OP.decision_margins(topo, tokens, logits, 1.0, "greedy", 0.09, 0.3)
    assert m[0] == np.inf
    assert m[1] == 3.0          # token 0 (logit 1) against the best other, 4
    assert m[2] == 2.0          # token 1 (logit 4) against the best other, 2
    # typical, uniform p over 4 tokens: H = ln 4, threshold min(0.09, 0.3/4)
    p = np.full((3, 4), 0.25)
    Hh = np.full(3, np.log(4.0))
    m = OP.decision_margins(topo, tokens, np.zeros((3, 4)), 1.0, "typical", 0.09, 0.3, p, Hh)
    assert np.isclose(m[1], np.log(0.25 / 0.075), rtol=1e-14)
    assert np.isclose(m[2], np.log(0.25 / 0.075), rtol=1e-14)
    # a one-hot row: threshold min(eps, delta) = 0.09; the hot token's margin
    # is log(1/0.09)
    p1 = np.zeros((3, 4))
    p1[0, 1] = 1.0
    H1 = np.zeros(3)
    m = OP.decision_margins(topo, np.array([0, 1, 1]), np.zeros((3, 4)), 1.0, "typical",
                            0.09, 0.3, p1, H1)
    assert np.isclose(m[1], np.log(1 / 0.09), rtol=1e-14)


def test_inverse_cdf_margin_closed_forms():
    w = np.ones(4)                      # C = 1, 2, 3, 4 of 4
    assert OT.inverse_cdf(w, 0.3) == 1
    assert np.isclose(OT.inverse_cdf_margin(w, 0.3), 0.05, rtol=1e-12)
    assert np.isclose(OT.inverse_cdf_margin(w, 0.9), 0.1, rtol=1e-12)
    assert OT.inverse_cdf_margin(w, 0.0) == 0.0          # on the first edge
    w = np.array([0.0, 2.0, 0.0, 2.0])  # C = 0, 2, 2, 4: u = 0.5 sits on an edge
    assert OT.inverse_cdf(w, 0.5) == 3
    assert OT.inverse_cdf_margin(w, 0.5) == 0.0
    assert np.isclose(OT.inverse_cdf_margin(w, 0.625), 0.125, rtol=1e-12)
    # unnormalised weights: the margin is a fraction of the total
    assert np.isclose(OT.inverse_cdf_margin(10 * np.ones(4), 0.3), 0.05, rtol=1e-12)


def test_exact_posterior_margins_closed_form():
    # root -> one child (a leaf). p_root = (0.5, 0.5), q = (0.8, 0.2); the
    # child's token 0 with u = 0.5: u q = 0.4 < 0.5, accepted with log margin
    # log(0.5/0.4). The leaf's target (0.25, 0.75) is drawn with u = 0.1:
    # point 0.1 in token 0's step [0, 0.25), margin 0.1.
    topo = OT.topology(np.array([[0]], dtype=np.int32), 1)
    p_rows = np.array([[0.5, 0.5], [0.25, 0.75]])
    q = np.array([[0.8, 0.2]])
    r = OP.posterior_exact(topo, np.array([1, 0]), p_rows, q, np.array([0.0, 0.5]),
                           np.array([0.0, 0.1]), with_margins=True)
    assert r["accept_len"] == 1 and r["next_root"] == 0
    assert np.isclose(r["accept_margin"], np.log(0.5 / 0.4), rtol=1e-14)
    assert np.isclose(r["draw_margin"], 0.1, rtol=1e-12)
    # rejected (u = 0.7: 0.56 > 0.5): residual (0.5-0.8)+, (0.5-0.2)+ = (0, 0.3)
    # -> (0, 1); the draw with u = 0.2 takes token 1 at margin 0.2
    r = OP.posterior_exact(topo, np.array([1, 0]), p_rows, q, np.array([0.0, 0.7]),
                           np.array([0.2, 0.0]), with_margins=True)
    assert r["accept_len"] == 0 and r["next_root"] == 1
    assert np.isclose(r["accept_margin"], np.log(0.56 / 0.5), rtol=1e-14)
    assert np.isclose(r["draw_margin"], 0.2, rtol=1e-12)
    # margins do not change the decisions
    r0 = OP.posterior_exact(topo, np.array([1, 0]), p_rows, q, np.array([0.0, 0.7]),
                            np.array([0.2, 0.0]))
    assert all(np.array_equal(r0[k], r[k]) for k in r0)
