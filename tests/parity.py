"""Shared parity logic: cached workload inputs and oracle runs, the GPU step,
and the element-by-element comparison with the near-tie guard.

Near-tie guard: a discrete decision (top-s membership, argmax, acceptance)
whose oracle margin is smaller than 4x the measured difference between the
GPU's and the oracle's value of the quantity that decides it is reported as
tie-ambiguous instead of failing; every other decision must agree exactly.
"""

from __future__ import annotations

import numpy as np

from oracle import heads as OH
from oracle import posterior as OP
from oracle import step as OSTEP
from oracle import tree as OT
from oracle import verifier as OV
from oracle.numerics import widen
from workloads import make_inputs

from gpu_helpers import assert_close, normwise

_INPUTS = {}
_ORACLE = {}


def inputs_for(w):
    if w not in _INPUTS:
        _INPUTS.clear()
        _ORACLE.clear()
        _INPUTS[w] = make_inputs(w)
    return _INPUTS[w]


def oracle_for(w):
    if w not in _ORACLE:
        inp = inputs_for(w)
        _ORACLE[w] = OSTEP.verify_step(inp, H=w.H, Dh=w.Dh, s_max=w.s_max, mode=w.mode,
                                       tau=w.tau, eps=w.eps, delta=w.delta,
                                       theta=w.rope_theta, bf16=(w.dtype == "bf16"))
    return _ORACLE[w]


def gpu_step(w, inp, want_logits=True, composite=False, keep_kv_len=False, repeat=1):
    """One step on the GPU: the five calls, or the composite medusa_step.
    keep_kv_len (composite only): the advanced prefix lengths go to a buffer
    of their own and kv_len must come back unchanged (returned as
    "kv_len_after"); repeat: the step runs that many times in a row (each
    over the same prefix when keep_kv_len is set)."""
    import torch
    from medusa_tree_verification_forward_amd.step import VerifyStep, to_host
    st = VerifyStep(inp, H=w.H, Dh=w.Dh, s_max=w.s_max, mode=w.mode, tau=w.tau, eps=w.eps,
                    delta=w.delta, theta=w.rope_theta, want_logits=want_logits)
    for _ in range(repeat):
        if composite:
            st.run_step(keep_kv_len=keep_kv_len)
        else:
            st.run()
    torch.cuda.synchronize()
    res = st.results()
    res["k_cache_next"] = to_host(st.inp["k_cache"])
    res["v_cache_next"] = to_host(st.inp["v_cache"])
    if keep_kv_len:
        res["kv_len_next"] = to_host(st.kv_len_next)
        res["kv_len_after"] = to_host(st.inp["kv_len"])
    else:
        res["kv_len_next"] = to_host(st.inp["kv_len"])
    return res


def typical_quantity(logit_c, m, S, W, tau, eps, delta):
    """log p(x) - log threshold from row statistics (float64)."""
    logp = (logit_c - m) / tau - np.log(S)
    H = np.log(S) - W / S
    logthr = min(np.log(eps), np.log(delta) - H)
    return logp - logthr


# Float32 rounding of the kernels' own arithmetic: an inverse-CDF draw point
# may move by about this fraction of the total weight (a CDF of up to 32768
# weights summed in float32 in chunks), and a log ratio p/q by about this.
CDF_EDGE = 2e-6
LOG_EDGE = 1e-5


def exact_rule(topo, tokens, head_logits, verify_logits, tau, u_accept, u_resample):
    """The oracle's exact rule (float64) on given float head and verify
    logits, with its margins."""
    K = head_logits.shape[0]
    q = np.stack([OT.softmax(np.asarray(head_logits[k], dtype=np.float64)) for k in range(K)])
    p_rows = np.stack([OT.softmax(np.asarray(r, dtype=np.float64), tau) for r in verify_logits])
    return OP.posterior_exact(topo, tokens, p_rows, q, u_accept, u_resample, with_margins=True)


def near_flip(ref):
    """True when the walk is within float32 rounding of a flip point."""
    return ref["accept_margin"] < LOG_EDGE or ref["draw_margin"] < CDF_EDGE


_POST_KEYS = ("accept_len", "last_node", "best_path", "next_root", "out_tokens")


def _same_post(a, b):
    return all(np.array_equal(np.asarray(a[k]), np.asarray(b[k])) for k in _POST_KEYS)


def oracle_on_tokens(w, inp, tokens):
    """The oracle step re-run on the given tree tokens [B][T] (the GPU's own
    drafts), so that every later stage can be compared on the same tokens."""
    return OSTEP.verify_step(inp, H=w.H, Dh=w.Dh, s_max=w.s_max, mode=w.mode, tau=w.tau,
                             eps=w.eps, delta=w.delta, theta=w.rope_theta,
                             bf16=(w.dtype == "bf16"), tokens_override=tokens)


def compare_step(w, inp, g, o, report):
    """Compare a GPU step (g) with the oracle step (o); fill `report`.

    Every sequence's decisions are compared: where the GPU drafted other
    tokens than the oracle (a top-s near tie, or a sampled draw on a CDF
    edge, each checked to be one), the oracle is re-run on the GPU's tokens;
    an ambiguous child decision is replaced by the GPU's own decision for
    that child alone, and the longest prefix, the committed tokens and the
    commit are still compared exactly. Exact mode compares its decisions
    whenever the oracle's walk is farther from every flip point than the
    measured float difference allows (else the sequence is counted in
    report["exact_ambiguous"]). report["decisions_checked"] counts the
    sequences whose posterior outputs were compared."""
    topo = o["topo"]
    bf16 = w.dtype == "bf16"
    ftol = 2e-2
    report.setdefault("ambiguous", 0)
    report.setdefault("decisions_checked", 0)
    # ---- heads ----
    report["z"] = assert_close(g["z"], o["z"], 1e-5, "z")
    head_err = float(np.max(np.abs(g["head_logits"] - o["head_logits"])))
    report["head_logits"] = assert_close(g["head_logits"], o["head_logits"], 1e-5, "head logits")
    near_heads = set()
    for b in range(w.B):
        for k in range(w.K):
            if np.array_equal(g["topk_ids"][b, k], o["topk_ids"][b, k]):
                continue
            # only a near tie may reorder a pool
            assert OH.topk_margin(o["head_logits"][b, k], w.s_max) < 4 * head_err, (b, k)
            near_heads.add((b, k))
            report["ambiguous"] += 1
    assert np.allclose(g["head_lse"], o["head_lse"], rtol=1e-5, atol=1e-5)
    # ---- tree (bit-exact) ----
    assert np.array_equal(g["tree_mask"], topo.mask)
    assert np.array_equal(g["retrieve"], topo.retrieve)
    assert np.array_equal(g["parent"], topo.parent)
    assert np.array_equal(g["depth"], topo.depth)
    assert np.array_equal(g["position_ids"], o["positions"])
    diff = np.argwhere(g["tree_tokens"] != o["tokens"])
    for b, n in diff:
        if w.mode == "exact":
            # a sampled draft may differ only on a CDF step edge
            assert o["draft_margin"][b, n] < CDF_EDGE, (b, n, o["draft_margin"][b, n])
        else:
            assert (int(b), int(topo.depth[n]) - 1) in near_heads, (b, n)
    if w.mode == "exact":
        report["draft_agreement"] = float(np.mean(g["tree_tokens"] == o["tokens"]))
    if len(diff):
        report["oracle_rerun_on_gpu_tokens"] = int(len(diff))
        o_draft = o
        o = oracle_on_tokens(w, inp, g["tree_tokens"])
        if w.mode == "exact":
            o["draft_margin"] = o_draft["draft_margin"]
    assert np.array_equal(g["tree_tokens"], o["tokens"])
    # ---- verifier floats ----
    tol_kv = ftol if bf16 else 1e-4
    report["k_tree"] = assert_close(widen(g["k_tree"]), o["k"], tol_kv, "k_tree")
    report["v_tree"] = assert_close(widen(g["v_tree"]), o["v"], tol_kv, "v_tree")
    report["y"] = assert_close(g["y"], o["y"], tol_kv, "y")
    report["logits"] = assert_close(g["verify_logits"], o["logits"], tol_kv, "logits")
    gm = g["row_stats"][..., 0]
    assert_close(gm, o["row_max"], tol_kv, "row max")
    # row statistics against the oracle's own row distribution
    for b in range(w.B):
        z = o["logits"][b] / w.tau
        mm = z.max(-1, keepdims=True)
        e = np.exp(z - mm)
        S = e.sum(-1)
        Wsum = (e * (z - mm)).sum(-1)
        assert_close(g["row_stats"][b, :, 1], S, tol_kv, "S")
        assert_close(g["row_stats"][b, :, 2], Wsum, max(tol_kv, 2e-2), "W")
        # row statistics are consistent with the kernel's own logits
        gz = g["verify_logits"][b].astype(np.float64) / w.tau
        gmm = gz.max(-1, keepdims=True)
        ge = np.exp(gz - gmm)
        assert np.allclose(g["row_stats"][b, :, 1], ge.sum(-1), rtol=1e-4)
        assert np.array_equal(g["row_argmax"][b], np.argmax(g["verify_logits"][b], axis=-1))
        for c in range(1, topo.T):
            assert g["child_logit"][b, c] == g["verify_logits"][b, topo.parent[c],
                                                                 g["tree_tokens"][b, c]]
    # ---- decisions ----
    err_l = np.abs(g["verify_logits"].astype(np.float64) - o["logits"])
    report.setdefault("exact_ambiguous", 0)
    for b in range(w.B):
        tok = o["tokens"][b]
        if w.mode in ("greedy", "typical"):
            acc_ref = np.array(o["acc"][b], dtype=bool)
            for c in range(1, topo.T):
                v = topo.parent[c]
                x = int(tok[c])
                if w.mode == "greedy":
                    qo = o["logits"][b, v, x] - np.max(np.delete(o["logits"][b, v], x))
                    qg = (float(g["verify_logits"][b, v, x])
                          - float(np.max(np.delete(g["verify_logits"][b, v], x))))
                else:
                    ro = o["logits"][b, v]
                    zo = ro / w.tau
                    mo = zo.max()
                    eo = np.exp(zo - mo)
                    qo = typical_quantity(ro[x], ro.max(), eo.sum(), (eo * (zo - mo)).sum(),
                                          w.tau, w.eps, w.delta)
                    gs = g["row_stats"][b, v].astype(np.float64)
                    qg = typical_quantity(float(g["child_logit"][b, c]), gs[0], gs[1], gs[2],
                                          w.tau, w.eps, w.delta)
                assert (qo > 0) == bool(acc_ref[c]), "oracle decision bookkeeping"
                if abs(qo) < 4 * abs(qg - qo) + 1e-12:
                    # a near tie: this child takes the GPU's decision, the
                    # rest of the sequence is still compared
                    report["ambiguous"] += 1
                    acc_ref[c] = qg > 0
                    continue
                assert (qg > 0) == (qo > 0), (b, c, qo, qg)
            ref = OP.posterior_deterministic(topo, tok, acc_ref, o["argmax"][b])
            for k in ("accept_len", "last_node", "best_path"):
                assert g[k][b] == ref[k], (b, k, g[k][b], ref[k])
            assert np.array_equal(g["out_tokens"][b], ref["out_tokens"])
            last = int(ref["last_node"])
            if OP.argmax_margin(o["logits"][b, last]) < 4 * float(err_l[b, last].max()):
                report["ambiguous"] += 1
                assert g["next_root"][b] == g["row_argmax"][b, last]
            else:
                assert g["next_root"][b] == ref["next_root"]
            report["decisions_checked"] += 1
        else:
            # The oracle's rule on the oracle's floats (ref_o) and on the
            # kernel's own float logits (ref_g), same tokens and uniforms.
            # The kernel must give ref_g except within float32 rounding of a
            # flip of ref_g; where ref_o and ref_g agree that is ref_o, the
            # comparison with the oracle. Where they differ, the difference
            # between the two verifier evaluations is what flips the rule.
            ref_o = {k: o[k][b] for k in _POST_KEYS}
            ref_g = exact_rule(topo, tok, g["head_logits"][b], g["verify_logits"][b], w.tau,
                               inp["u_accept"][b], inp["u_resample"][b])
            gb = {k: g[k][b] for k in _POST_KEYS}
            if not _same_post(gb, ref_g):
                assert near_flip(ref_g), (b, gb, ref_g)
                report["exact_ambiguous"] += 1
            elif not _same_post(ref_o, ref_g):
                report["exact_ambiguous"] += 1
            else:
                report["decisions_checked"] += 1
        # commit: KV rows of the GPU's committed path, kv_len, h_next
        gl = int(g["last_node"][b])
        path = topo.path(gl)
        L0 = int(inp["kv_len"][b])
        assert g["kv_len_next"][b] == L0 + len(path)
        for i, n in enumerate(path):
            assert np.array_equal(g["k_cache_next"][b, :, L0 + i], g["k_tree"][b, n])
            assert np.array_equal(g["v_cache_next"][b, :, L0 + i], g["v_tree"][b, n])
        assert np.array_equal(g["k_cache_next"][b, :, :L0], inp["k_cache"][b, :, :L0])
        assert np.array_equal(g["h_next"][b], g["y"][b, gl])
        assert g["out_tokens"][b, 0] == inp["root"][b]
    report["accept_len"] = [int(x) for x in g["accept_len"]]
    return report


def gpu_posterior_consistent(w, g, topo, inp=None):
    """The GPU posterior equals the oracle's rule applied to the GPU's own
    float outputs (in exact mode with the same uniforms). A sequence with a
    decision within float32 rounding of its flip point is not compared;
    returns the number of sequences compared."""
    checked = 0
    for b in range(w.B):
        tok = g["tree_tokens"][b]
        if w.mode == "exact":
            post = exact_rule(topo, tok, g["head_logits"][b], g["verify_logits"][b], w.tau,
                              inp["u_accept"][b], inp["u_resample"][b])
            if near_flip(post):
                continue
        else:
            if w.mode == "greedy":
                acc = OP.accept_greedy(topo, tok, g["row_argmax"][b])
            else:
                acc = np.zeros(topo.T, dtype=bool)
                acc[0] = True
                near = False
                for c in range(1, topo.T):
                    gs = g["row_stats"][b, topo.parent[c]].astype(np.float64)
                    q = typical_quantity(float(g["child_logit"][b, c]), gs[0], gs[1], gs[2],
                                         w.tau, w.eps, w.delta)
                    near |= abs(q) < 1e-4
                    acc[c] = q > 0
                if near:
                    continue
            post = OP.posterior_deterministic(topo, tok, acc, g["row_argmax"][b])
        assert g["accept_len"][b] == post["accept_len"]
        assert g["last_node"][b] == post["last_node"]
        assert g["best_path"][b] == post["best_path"]
        assert np.array_equal(g["out_tokens"][b], post["out_tokens"])
        assert g["next_root"][b] == post["next_root"]
        checked += 1
    return checked
