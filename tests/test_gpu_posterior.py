"""GPU parity of medusa_evaluate_posterior and medusa_commit.

Stage-isolated: the GPU kernel and the oracle rule see the same float32
inputs, so every decision must agree except those within float32 rounding of
the flip point. The exact rule is checked statistically on a 64-token
vocabulary slice, with drafting and acceptance on the GPU.
"""

import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import posterior as OP
from oracle import tree as OT
from workloads import cartesian_ranks

from gpu_helpers import dev, host, poisoned, require_gpu, workspace

pytestmark = pytest.mark.gpu


def _shape(M, B, K, T, P, V, s_max=4, d=128):
    return M.make_shape(B, d, V, K, 1, d, 4096, T - 1, P, s_max, "bf16")


def _outs(torch, B, K):
    i32 = torch.int32
    return dict(accept_len=poisoned((B,), i32), best_path=poisoned((B,), i32),
                last_node=poisoned((B,), i32), out_tokens=poisoned((B, K + 1), i32),
                next_root=poisoned((B,), i32))


def _post(M, shape, mode, tau, eps, delta, stats, argmax, child, tokens, topo, ws, o, **kw):
    M.evaluate_posterior(shape, mode, tau, eps, delta, dev(stats), dev(argmax), dev(child),
                         dev(tokens), dev(topo.parent), dev(topo.retrieve), o["accept_len"],
                         o["best_path"], o["last_node"], o["out_tokens"], o["next_root"], ws,
                         **kw)


@pytest.mark.parametrize("s", [(3, 2, 2, 1, 1), (4, 3, 2, 2, 1), (2, 2, 2), (16,)])
def test_greedy_planted(s):
    import torch
    import medusa_tree_verification_forward_amd as M
    require_gpu()
    rng = np.random.default_rng(len(s) * 7 + s[0])
    K = len(s)
    topo = OT.topology(cartesian_ranks(s), K)
    T, B, V = topo.T, 64, 50
    tokens = rng.integers(0, V, size=(B, T)).astype(np.int32)
    argmax = rng.integers(0, V, size=(B, T)).astype(np.int32)
    for b in range(B):     # plant agreement with a per-sequence rate, all depths reachable
        rho = rng.uniform(0, 1)
        for v in range(T):
            kids = topo.children(v)
            if kids and rng.random() < rho:
                tokens[b, kids[int(rng.integers(len(kids)))]] = argmax[b, v]
    shape = _shape(M, B, K, T, topo.P, V, s_max=max(s))
    ws = workspace(M.workspace_bytes(shape))
    o = _outs(torch, B, K)
    stats = np.zeros((B, T, 3), np.float32)
    child = np.zeros((B, T), np.float32)
    _post(M, shape, "greedy", 1.0, 0.09, 0.3, stats, argmax, child, tokens, topo, ws, o)
    torch.cuda.synchronize()
    g = {k: host(v) for k, v in o.items()}
    seen = set()
    for b in range(B):
        acc = OP.accept_greedy(topo, tokens[b], argmax[b])
        ref = OP.posterior_deterministic(topo, tokens[b], acc, argmax[b])
        for k in ("accept_len", "last_node", "best_path", "next_root"):
            assert g[k][b] == ref[k], (b, k)
        assert np.array_equal(g["out_tokens"][b], ref["out_tokens"])
        seen.add(int(ref["accept_len"]))
    assert len(seen) >= min(3, K + 1)


def _typical_inputs(rng, topo, B, V, tau, hot):
    logits = rng.standard_normal((B, topo.T, V)).astype(np.float32) * 2.0
    tokens = rng.integers(0, V, size=(B, topo.T)).astype(np.int32)
    for b in range(B):
        for v in range(topo.T):
            kids = topo.children(v)
            if kids and rng.random() < hot:
                tokens[b, kids[0]] = int(np.argmax(logits[b, v]))
    z = logits.astype(np.float64) / tau
    m = z.max(-1, keepdims=True)
    e = np.exp(z - m)
    stats = np.stack([logits.max(-1), e.sum(-1), (e * (z - m)).sum(-1)], -1).astype(np.float32)
    argmax = np.argmax(logits, -1).astype(np.int32)
    child = np.zeros((B, topo.T), np.float32)
    for b in range(B):
        for c in range(1, topo.T):
            child[b, c] = logits[b, topo.parent[c], tokens[b, c]]
    return logits, tokens, stats, argmax, child


@pytest.mark.parametrize("tau", [0.7, 1.0, 0.2])
def test_typical_same_float_inputs(tau):
    import torch
    import medusa_tree_verification_forward_amd as M
    require_gpu()
    rng = np.random.default_rng(int(tau * 100))
    s = (3, 2, 2, 1, 1)
    K = len(s)
    topo = OT.topology(cartesian_ranks(s), K)
    T, B, V = topo.T, 64, 40
    eps, delta = 0.09, 0.3
    logits, tokens, stats, argmax, child = _typical_inputs(rng, topo, B, V, tau, 0.5)
    shape = _shape(M, B, K, T, topo.P, V)
    ws = workspace(M.workspace_bytes(shape))
    o = _outs(torch, B, K)
    _post(M, shape, "typical", tau, eps, delta, stats, argmax, child, tokens, topo, ws, o)
    torch.cuda.synchronize()
    g = {k: host(v) for k, v in o.items()}
    checked = 0
    lens = set()
    for b in range(B):
        acc = np.zeros(T, bool)
        acc[0] = True
        near = False
        for c in range(1, T):
            m, S, W = stats[b, topo.parent[c]].astype(np.float64)
            logp = (float(child[b, c]) - m) / tau - np.log(S)
            H = np.log(S) - W / S
            q = logp - min(np.log(eps), np.log(delta) - H)
            near |= abs(q) < 1e-5
            acc[c] = q > 0
        if near:
            continue
        ref = OP.posterior_deterministic(topo, tokens[b], acc, argmax[b])
        for k in ("accept_len", "last_node", "best_path", "next_root"):
            assert g[k][b] == ref[k], (b, k)
        assert np.array_equal(g["out_tokens"][b], ref["out_tokens"])
        checked += 1
        lens.add(int(ref["accept_len"]))
    assert checked >= B - 2
    assert len(lens) >= 2


def test_typical_matches_oracle_distribution_rule():
    # The GPU's typical decision from row statistics equals the oracle's
    # decision from the full row distribution (the row statistics are exact
    # summaries of the same logits).
    import torch
    import medusa_tree_verification_forward_amd as M
    from oracle import verifier as OV
    require_gpu()
    rng = np.random.default_rng(5)
    s = (2, 2, 2)
    topo = OT.topology(cartesian_ranks(s), 3)
    T, B, V, tau = topo.T, 32, 500, 0.7
    logits, tokens, stats, argmax, child = _typical_inputs(rng, topo, B, V, tau, 0.6)
    shape = _shape(M, B, 3, T, topo.P, V)
    ws = workspace(M.workspace_bytes(shape))
    o = _outs(torch, B, 3)
    _post(M, shape, "typical", tau, 0.09, 0.3, stats, argmax, child, tokens, topo, ws, o)
    torch.cuda.synchronize()
    g = {k: host(v) for k, v in o.items()}
    for b in range(B):
        p, Hh, am = OV.row_distribution(logits[b].astype(np.float64), tau)
        acc = OP.accept_typical(topo, tokens[b], p, Hh, 0.09, 0.3)
        margins = [abs(np.log(p[topo.parent[c], tokens[b, c]])
                       - np.log(min(0.09, 0.3 * np.exp(-Hh[topo.parent[c]]))))
                   for c in range(1, T)]
        if min(margins) < 1e-4:
            continue
        ref = OP.posterior_deterministic(topo, tokens[b], acc, am)
        assert g["accept_len"][b] == ref["accept_len"]
        assert g["last_node"][b] == ref["last_node"]
        assert g["next_root"][b] == ref["next_root"]


def test_sparse_tree_posterior():
    import torch
    import medusa_tree_verification_forward_amd as M
    require_gpu()
    rng = np.random.default_rng(9)
    spec = np.array([[0, -1, -1], [1, -1, -1], [0, 0, -1], [0, 1, -1], [1, 0, -1], [0, 0, 0]],
                    dtype=np.int32)
    topo = OT.topology(spec, 3)
    T, B, V = topo.T, 64, 6
    tokens = rng.integers(0, V, size=(B, T)).astype(np.int32)
    argmax = rng.integers(0, V, size=(B, T)).astype(np.int32)
    shape = _shape(M, B, 3, T, topo.P, V, s_max=2)
    ws = workspace(M.workspace_bytes(shape))
    o = _outs(torch, B, 3)
    _post(M, shape, "greedy", 1.0, 0.09, 0.3, np.zeros((B, T, 3), np.float32), argmax,
          np.zeros((B, T), np.float32), tokens, topo, ws, o)
    torch.cuda.synchronize()
    g = {k: host(v) for k, v in o.items()}
    for b in range(B):
        acc = OP.accept_greedy(topo, tokens[b], argmax[b])
        ref = OP.posterior_deterministic(topo, tokens[b], acc, argmax[b])
        for k in ("accept_len", "last_node", "best_path", "next_root"):
            assert g[k][b] == ref[k], (b, k)


# ---------------------------------------------------------------- exact mode

def _exact_setup(V=64, K=5, seed=0):
    rng = np.random.default_rng(seed)
    s = (3, 2, 2, 1, 1)
    topo = OT.topology(cartesian_ranks(s), K)
    head_logits = rng.standard_normal((K, V)).astype(np.float32) * 1.5
    table = (rng.standard_normal((K + 1, V, V)) * 1.3).astype(np.float32)   # logits
    root_logits = rng.standard_normal(V).astype(np.float32) * 1.3
    return topo, head_logits, table, root_logits


def _exact_gpu_batches(topo, head_logits, table, root_logits, n_trials, seed):
    """Run n_trials exact-mode draft+accept trials on the GPU, 64 per call."""
    import torch
    import medusa_tree_verification_forward_amd as M
    K, V = head_logits.shape
    T, B = topo.T, 64
    rng = np.random.default_rng(seed)
    lse = scipy.special.logsumexp(head_logits.astype(np.float64), axis=-1).astype(np.float32)
    shape = M.make_shape(B, 128, V, K, 1, 128, 4096, T - 1, topo.P, 3, "bf16")
    ws = workspace(M.workspace_bytes(shape))
    hl = dev(np.ascontiguousarray(np.broadcast_to(head_logits, (B, K, V))))
    hlse = dev(np.ascontiguousarray(np.broadcast_to(lse, (B, K))))
    i32 = torch.int32
    tok = torch.zeros((B, T), dtype=i32, device="cuda")
    mask = torch.zeros((T, T), dtype=torch.uint8, device="cuda")
    pos = torch.zeros((B, T), dtype=i32, device="cuda")
    ret = torch.zeros((topo.P, K + 1), dtype=i32, device="cuda")
    par = torch.zeros((T,), dtype=i32, device="cuda")
    dep = torch.zeros((T,), dtype=i32, device="cuda")
    root = dev(np.zeros(B, np.int32))
    kv = dev(np.zeros(B, np.int32))
    o = _outs(torch, B, K)
    depth = topo.depth
    rows = []
    for it in range((n_trials + B - 1) // B):
        u = rng.random((3, B, T), dtype=np.float32)
        M.build_tree(shape, cartesian_ranks((3, 2, 2, 1, 1)), root, kv, tok, mask, pos, ret, par,
                     dep, draft_mode=M.DRAFT_SAMPLE, head_logits=hl, head_lse=hlse,
                     u_draft=dev(u[0]))
        t = host(tok)
        vl = np.empty((B, T, V), np.float32)
        vl[:, 0] = root_logits
        for n in range(1, T):
            vl[:, n] = table[depth[n], t[:, n]]
        M.evaluate_posterior(shape, "exact", 1.0, 0.0, 0.0, None, None, None, tok, par, ret,
                             o["accept_len"], o["best_path"], o["last_node"], o["out_tokens"],
                             o["next_root"], ws, verify_logits=dev(vl), head_logits=hl,
                             head_lse=hlse, u_accept=dev(u[1]), u_resample=dev(u[2]))
        torch.cuda.synchronize()
        rows.append((u, t, host(o["accept_len"]), host(o["out_tokens"]), host(o["next_root"])))
    return rows


def test_exact_rule_distribution_v64():
    require_gpu()
    topo, head_logits, table, root_logits = _exact_setup()
    K, V = head_logits.shape
    n = 100_000
    rows = _exact_gpu_batches(topo, head_logits, table, root_logits, n, seed=1)
    rng = np.random.default_rng(2)
    p_root = scipy.special.softmax(root_logits.astype(np.float64))
    p1 = scipy.special.softmax(table[1].astype(np.float64), axis=-1)   # p(. | depth-1 token)
    firsts = np.zeros(V)
    pairs = np.zeros((V, V))
    lens = np.zeros(K + 1)
    for u, t, alen, out, nxt in rows:
        for b in range(alen.shape[0]):
            a = int(alen[b])
            lens[a] += 1
            gen = [int(x) for x in out[b, 1:a + 1]] + [int(nxt[b])]
            y1 = gen[0]
            y2 = gen[1] if len(gen) > 1 else int(rng.choice(V, p=p1[y1]))
            firsts[y1] += 1
            pairs[y1, y2] += 1
    total = firsts.sum()
    assert scipy.stats.chisquare(firsts, p_root * total).pvalue > 1e-4
    joint = (p_root[:, None] * p1).ravel() * total
    keep = joint > 5
    obs = pairs.ravel()[keep]
    assert scipy.stats.chisquare(obs, joint[keep] * obs.sum() / joint[keep].sum()).pvalue > 1e-4
    assert lens[1:].sum() > 0.2 * total      # drafts do get accepted


def test_exact_rule_agrees_with_oracle_per_trial():
    # Same uniforms, same drafted tokens: the oracle's float64 rule and the
    # kernel's float32 rule may differ only where a uniform lands within
    # rounding of a decision boundary.
    require_gpu()
    topo, head_logits, table, root_logits = _exact_setup(seed=3)
    K, V = head_logits.shape
    rows = _exact_gpu_batches(topo, head_logits, table, root_logits, 2048, seed=4)
    q = scipy.special.softmax(head_logits.astype(np.float64), axis=-1)
    agree = total = 0
    for u, t, alen, out, nxt in rows:
        for b in range(alen.shape[0]):
            p_rows = np.empty((topo.T, V))
            p_rows[0] = scipy.special.softmax(root_logits.astype(np.float64))
            for n in range(1, topo.T):
                p_rows[n] = scipy.special.softmax(table[topo.depth[n], t[b, n]].astype(np.float64))
            ref = OP.posterior_exact(topo, t[b], p_rows, q, u[1, b], u[2, b])
            same = (ref["accept_len"] == alen[b] and ref["next_root"] == nxt[b]
                    and np.array_equal(ref["out_tokens"], out[b]))
            agree += same
            total += 1
    assert agree / total > 0.995, agree / total


def test_exact_rule_agrees_with_oracle_large_vocab():
    # V = 40000: the posterior past the vocabulary it holds in LDS (the
    # global-memory walk) and the sampler's 32-token CDF chunks. Verify rows
    # are the drafting head's logits plus noise, so children are accepted
    # and rejected (residual resampling) in a mix; per trial the kernel must
    # agree with the float64 rule except within rounding of a boundary.
    import torch
    import medusa_tree_verification_forward_amd as M
    require_gpu()
    K, V, B = 5, 40000, 16
    rng = np.random.default_rng(11)
    s = (3, 2, 2, 1, 1)
    spec = cartesian_ranks(s)
    topo = OT.topology(spec, K)
    T = topo.T
    head_logits = (rng.standard_normal((K, V)) * 1.5).astype(np.float32)
    lse = scipy.special.logsumexp(head_logits.astype(np.float64), axis=-1).astype(np.float32)
    q = scipy.special.softmax(head_logits.astype(np.float64), axis=-1)
    shape = M.make_shape(B, 128, V, K, 1, 128, 4096, T - 1, topo.P, 3, "bf16")
    ws = workspace(M.workspace_bytes(shape))
    hl = dev(np.ascontiguousarray(np.broadcast_to(head_logits, (B, K, V))))
    hlse = dev(np.ascontiguousarray(np.broadcast_to(lse, (B, K))))
    i32 = torch.int32
    tok = poisoned((B, T), i32)
    mask = poisoned((T, T), torch.uint8)
    pos = poisoned((B, T), i32)
    ret = poisoned((topo.P, K + 1), i32)
    par = poisoned((T,), i32)
    dep = poisoned((T,), i32)
    o = _outs(torch, B, K)
    agree = total = accepted = 0
    for it in range(4):
        u = rng.random((3, B, T), dtype=np.float32)
        M.build_tree(shape, spec, dev(np.zeros(B, np.int32)), dev(np.zeros(B, np.int32)), tok,
                     mask, pos, ret, par, dep, draft_mode=M.DRAFT_SAMPLE, head_logits=hl,
                     head_lse=hlse, u_draft=dev(u[0]))
        t = host(tok)
        # node n's verify row: the logits of the head that drafts its children
        vl = np.empty((B, T, V), np.float32)
        for n in range(T):
            k = min(topo.depth[n], K - 1)
            vl[:, n] = head_logits[k] + (rng.standard_normal((B, V)) * 0.6).astype(np.float32)
        M.evaluate_posterior(shape, "exact", 1.0, 0.0, 0.0, None, None, None, tok, par, ret,
                             o["accept_len"], o["best_path"], o["last_node"], o["out_tokens"],
                             o["next_root"], ws, verify_logits=dev(vl), head_logits=hl,
                             head_lse=hlse, u_accept=dev(u[1]), u_resample=dev(u[2]))
        torch.cuda.synchronize()
        alen, out, nxt = host(o["accept_len"]), host(o["out_tokens"]), host(o["next_root"])
        for b in range(B):
            # the drafted tokens themselves: an inverse-CDF draw per node
            ref_t = OT.draft_tokens_sampled(topo, 0, head_logits.astype(np.float64), u[0, b])
            assert np.mean(ref_t[1:] == t[b, 1:]) > 0.95
            p_rows = scipy.special.softmax(vl[b].astype(np.float64), axis=-1)
            ref = OP.posterior_exact(topo, t[b], p_rows, q, u[1, b], u[2, b])
            same = (ref["accept_len"] == alen[b] and ref["next_root"] == nxt[b]
                    and np.array_equal(ref["out_tokens"], out[b]))
            agree += same
            total += 1
            accepted += int(alen[b]) > 0
    assert total - agree <= 1, (agree, total)
    assert 0 < accepted < total          # both outcomes occur


def test_exact_lds_kernel_agrees_with_oracle_per_trial_v32000():
    # V = 32000, the 7B vocabulary: the posterior keeps the target in LDS and
    # reads its CDF in 16-token chunks. 1024 trials (64 sequences x 16
    # calls); drafting on the GPU, the oracle's rule on the GPU's drafted
    # tokens with the same float32 logits and uniforms. Verify rows are the
    # drafting head's logits plus noise drawn from a bank, so children are
    # accepted and rejected (residual resampling) in a mix. A trial may
    # disagree only where the oracle's walk lies within float32 rounding of
    # a flip point, and at most once.
    import torch
    import medusa_tree_verification_forward_amd as M
    require_gpu()
    K, V, B, calls = 5, 32000, 64, 16
    rng = np.random.default_rng(32000)
    spec = cartesian_ranks((3, 2, 2, 1, 1))
    topo = OT.topology(spec, K)
    T = topo.T
    head_logits = (rng.standard_normal((K, V)) * 1.5).astype(np.float32)
    lse = scipy.special.logsumexp(head_logits.astype(np.float64), axis=-1).astype(np.float32)
    q = scipy.special.softmax(head_logits.astype(np.float64), axis=-1)
    bank = (rng.standard_normal((64, V)) * 0.6).astype(np.float32)
    node_head = np.minimum(topo.depth, K - 1)
    shape = M.make_shape(B, 128, V, K, 1, 128, 4096, T - 1, topo.P, 3, "bf16")
    ws = workspace(M.workspace_bytes(shape))
    hl = dev(np.ascontiguousarray(np.broadcast_to(head_logits, (B, K, V))))
    hlse = dev(np.ascontiguousarray(np.broadcast_to(lse, (B, K))))
    i32 = torch.int32
    tok = poisoned((B, T), i32)
    mask = poisoned((T, T), torch.uint8)
    pos = poisoned((B, T), i32)
    ret = poisoned((topo.P, K + 1), i32)
    par = poisoned((T,), i32)
    dep = poisoned((T,), i32)
    o = _outs(torch, B, K)
    disagree, total, lens = [], 0, set()
    for it in range(calls):
        u = rng.random((3, B, T), dtype=np.float32)
        M.build_tree(shape, spec, dev(np.zeros(B, np.int32)), dev(np.zeros(B, np.int32)), tok,
                     mask, pos, ret, par, dep, draft_mode=M.DRAFT_SAMPLE, head_logits=hl,
                     head_lse=hlse, u_draft=dev(u[0]))
        t = host(tok)
        idx = rng.integers(0, bank.shape[0], size=(B, T))
        vl = head_logits[node_head][None, :, :] + bank[idx]
        M.evaluate_posterior(shape, "exact", 1.0, 0.0, 0.0, None, None, None, tok, par, ret,
                             o["accept_len"], o["best_path"], o["last_node"], o["out_tokens"],
                             o["next_root"], ws, verify_logits=dev(vl), head_logits=hl,
                             head_lse=hlse, u_accept=dev(u[1]), u_resample=dev(u[2]))
        torch.cuda.synchronize()
        g = {k: host(v) for k, v in o.items()}
        for b in range(B):
            ref_t = OT.draft_tokens_sampled(topo, 0, head_logits.astype(np.float64), u[0, b])
            dm = OT.draft_margins(topo, head_logits.astype(np.float64), u[0, b])
            bad = np.nonzero(ref_t[1:] != t[b, 1:])[0] + 1
            assert np.all(dm[bad] < 2e-6), (it, b, bad, dm[bad])
            p_rows = scipy.special.softmax(vl[b].astype(np.float64), axis=-1)
            ref = OP.posterior_exact(topo, t[b], p_rows, q, u[1, b], u[2, b], with_margins=True)
            total += 1
            lens.add(int(ref["accept_len"]))
            same = (all(g[k][b] == ref[k] for k in ("accept_len", "last_node", "best_path",
                                                     "next_root"))
                    and np.array_equal(ref["out_tokens"], g["out_tokens"][b]))
            if not same:
                disagree.append((it, b, ref["accept_margin"], ref["draw_margin"]))
    assert total == B * calls
    assert len(disagree) <= 1, disagree
    for _, _, am, dm in disagree:
        assert am < 1e-5 or dm < 2e-6, disagree
    assert len(lens) >= 3, lens          # accepted depths 0, 1, 2, ... all occur


def test_commit_capacity_guard():
    import torch
    import medusa_tree_verification_forward_amd as M
    require_gpu()
    topo = OT.topology(cartesian_ranks((2, 2)), 2)
    T, B, H, Dh, d, Lmax = topo.T, 2, 2, 64, 128, 16
    shape = M.make_shape(B, d, 100, 2, H, Dh, Lmax, T - 1, topo.P, 2, "bf16")
    rng = np.random.default_rng(0)
    kt = dev(rng.integers(0, 2**15, size=(B, T, H, Dh)).astype(np.uint16))
    vt = dev(rng.integers(0, 2**15, size=(B, T, H, Dh)).astype(np.uint16))
    y = dev(rng.standard_normal((B, T, d)).astype(np.float32))
    kc = dev(np.zeros((B, H, Lmax, Dh), np.uint16))
    vc = dev(np.zeros((B, H, Lmax, Dh), np.uint16))
    kv = dev(np.array([5, 14], np.int32))          # second sequence has no room for 3 rows
    last = dev(np.array([topo.retrieve[1, 2], topo.retrieve[2, 2]], np.int32))
    hn = poisoned((B, d), torch.float32)
    M.commit(shape, last, dev(topo.parent), kt, vt, y, kc, vc, kv, hn)
    torch.cuda.synchronize()
    kvh = host(kv)
    assert kvh[0] == 5 + 3 and kvh[1] == -1
    kch = host(kc)
    kth = host(kt)
    for i, n in enumerate(topo.path(int(topo.retrieve[1, 2]))):
        assert np.array_equal(kch[0, :, 5 + i], kth[0, n])
    assert np.all(kch[1] == 0)
    assert np.array_equal(host(hn)[0], host(y)[0, topo.retrieve[1, 2]])
