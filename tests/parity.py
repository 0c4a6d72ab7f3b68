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


def compare_step(w, inp, g, o, report):
    """Compare a GPU step (g) with the oracle step (o); fill `report`."""
    topo = o["topo"]
    bf16 = w.dtype == "bf16"
    ftol = 2e-2
    report.setdefault("ambiguous", 0)
    # ---- heads ----
    report["z"] = assert_close(g["z"], o["z"], 1e-5, "z")
    head_err = float(np.max(np.abs(g["head_logits"] - o["head_logits"])))
    report["head_logits"] = assert_close(g["head_logits"], o["head_logits"], 1e-5, "head logits")
    topk_ok = True
    for b in range(w.B):
        for k in range(w.K):
            if OH.topk_margin(o["head_logits"][b, k], w.s_max) < 4 * head_err:
                report["ambiguous"] += 1
                topk_ok = topk_ok and np.array_equal(g["topk_ids"][b, k], o["topk_ids"][b, k])
                continue
            assert np.array_equal(g["topk_ids"][b, k], o["topk_ids"][b, k]), (b, k)
    assert np.allclose(g["head_lse"], o["head_lse"], rtol=1e-5, atol=1e-5)
    # ---- tree (bit-exact) ----
    assert np.array_equal(g["tree_mask"], topo.mask)
    assert np.array_equal(g["retrieve"], topo.retrieve)
    assert np.array_equal(g["parent"], topo.parent)
    assert np.array_equal(g["depth"], topo.depth)
    assert np.array_equal(g["position_ids"], o["positions"])
    if w.mode != "exact":
        if not topk_ok:
            report["skipped_downstream"] = "top-s near tie changed the tree tokens"
            return report
        assert np.array_equal(g["tree_tokens"], o["tokens"])
    else:
        agree = float(np.mean(g["tree_tokens"] == o["tokens"]))
        report["draft_agreement"] = agree
        if agree < 1.0:
            report["skipped_downstream"] = "sampled drafts differ at a CDF step"
            return report
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
    for b in range(w.B):
        ambiguous_here = False
        if w.mode in ("greedy", "typical"):
            for c in range(1, topo.T):
                v = topo.parent[c]
                tok = int(o["tokens"][b, c])
                if w.mode == "greedy":
                    qo = o["logits"][b, v, tok] - np.max(np.delete(o["logits"][b, v], tok))
                    qg = (float(g["verify_logits"][b, v, tok])
                          - float(np.max(np.delete(g["verify_logits"][b, v], tok))))
                else:
                    ro = o["logits"][b, v]
                    zo = ro / w.tau
                    mo = zo.max()
                    eo = np.exp(zo - mo)
                    qo = typical_quantity(ro[tok], ro.max(), eo.sum(), (eo * (zo - mo)).sum(),
                                          w.tau, w.eps, w.delta)
                    gs = g["row_stats"][b, v].astype(np.float64)
                    qg = typical_quantity(float(g["child_logit"][b, c]), gs[0], gs[1], gs[2],
                                          w.tau, w.eps, w.delta)
                if abs(qo) < 4 * abs(qg - qo) + 1e-12:
                    ambiguous_here = True
                    report["ambiguous"] += 1
                    continue
                assert (qo > 0) == bool(o["acc"][b][c]), "oracle decision bookkeeping"
                assert (qg > 0) == (qo > 0), (b, c, qo, qg)
            last = int(o["last_node"][b])
            if not ambiguous_here:
                am_margin = OP.argmax_margin(o["logits"][b, last])
                if am_margin < 4 * float(err_l[b, last].max()):
                    report["ambiguous"] += 1
                else:
                    assert g["next_root"][b] == o["next_root"][b]
        if ambiguous_here:
            continue
        if w.mode != "exact":
            assert g["accept_len"][b] == o["accept_len"][b]
            assert g["last_node"][b] == o["last_node"][b]
            assert g["best_path"][b] == o["best_path"][b]
            assert np.array_equal(g["out_tokens"][b], o["out_tokens"][b])
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


def gpu_posterior_consistent(w, g, topo):
    """The GPU posterior equals the oracle's rule applied to the GPU's own
    float outputs (decisions within float32 rounding of the flip point are
    skipped)."""
    for b in range(w.B):
        tok = g["tree_tokens"][b]
        if w.mode == "greedy":
            acc = OP.accept_greedy(topo, tok, g["row_argmax"][b])
        else:
            acc = np.zeros(topo.T, dtype=bool)
            acc[0] = True
            for c in range(1, topo.T):
                gs = g["row_stats"][b, topo.parent[c]].astype(np.float64)
                q = typical_quantity(float(g["child_logit"][b, c]), gs[0], gs[1], gs[2],
                                     w.tau, w.eps, w.delta)
                if abs(q) < 1e-4:
                    return False
                acc[c] = q > 0
        post = OP.posterior_deterministic(topo, tok, acc, g["row_argmax"][b])
        assert g["accept_len"][b] == post["accept_len"]
        assert g["last_node"][b] == post["last_node"]
        assert g["best_path"][b] == post["best_path"]
        assert np.array_equal(g["out_tokens"][b], post["out_tokens"])
        assert g["next_root"][b] == post["next_root"]
    return True
