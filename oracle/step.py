"""One whole verify step, composed from the oracle stages (test infrastructure only).

Order of the step ("Medusa Part I", introduction; "Medusa 深读", §3.1, §5,
§6.1): the heads read the shared hidden state, their top-s pools form the
candidate tree, the verifier scores the tree in one masked pass, the
posterior keeps the longest accepted prefix, and the accepted prefix becomes
the next context.
"""

from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from . import heads as H_
from . import posterior as P_
from . import tree as T_
from . import verifier as V_
from .numerics import widen


def verify_step(inp: Dict[str, np.ndarray], *, H: int, Dh: int, s_max: int, mode: str,
                tau: float, eps: float, delta: float, theta: float, bf16: bool,
                want_margins: bool = True,
                tokens_override: Optional[np.ndarray] = None) -> Dict:
    """Run one step for every sequence of a batch.

    ``inp`` holds h [B,d], W1, W2, E, W_qkv, W_o, W_lm, k_cache, v_cache
    [B,H,Lmax,Dh], kv_len [B], root [B], ranks [N,K] and (exact mode)
    u_draft, u_accept, u_resample [B,T]. Returns a dict of per-stage
    results, batched along the first axis. tokens_override [B,T], when
    given, replaces the drafted tree tokens (every later stage then runs on
    those tokens), so a run can be repeated on another drafter's tokens.
    """
    h = np.asarray(inp["h"], dtype=np.float64)
    B = h.shape[0]
    K = inp["W2"].shape[0]
    topo = T_.topology(inp["ranks"], K)
    T = topo.T
    z, hl = H_.heads_forward(h, inp["W1"], inp["W2"], inp.get("b1"))
    topk_ids, topk_vals, lse = H_.heads_topk(hl, s_max)

    res: Dict = dict(topo=topo, z=z, head_logits=hl, topk_ids=topk_ids,
                     topk_logits=topk_vals, head_lse=lse)
    keys = ["tokens", "positions", "q", "k", "v", "o", "y", "logits", "p_entropy",
            "argmax", "acc", "accept_len", "last_node", "best_path", "out_tokens",
            "next_root", "kv_len_next", "h_next", "k_cache_next", "v_cache_next",
            "row_max", "topk_margin", "decision_margin", "argmax_margin",
            "draft_margin", "accept_margin", "draw_margin"]
    per = {k_: [] for k_ in keys}
    for b in range(B):
        L = int(inp["kv_len"][b])
        if mode == "exact":
            tok = T_.draft_tokens_sampled(topo, int(inp["root"][b]), hl[b], inp["u_draft"][b])
        else:
            tok = T_.draft_tokens_topk(topo, int(inp["root"][b]), topk_ids[b])
        if tokens_override is not None:
            tok = np.asarray(tokens_override[b], dtype=np.int32).copy()
        pos = T_.position_ids(topo, L)
        vf = V_.verifier_forward(inp["E"], inp["W_qkv"], inp["W_o"], inp["W_lm"], tok, pos,
                                 topo.mask, inp["k_cache"][b], inp["v_cache"][b], L, H, Dh,
                                 theta, bf16)
        logits = vf["logits"]
        p, ent, am = V_.row_distribution(logits, tau)
        if mode == "greedy":
            acc = P_.accept_greedy(topo, tok, am)
            post = P_.posterior_deterministic(topo, tok, acc, am)
        elif mode == "typical":
            acc = P_.accept_typical(topo, tok, p, ent, eps, delta)
            post = P_.posterior_deterministic(topo, tok, acc, am)
        elif mode == "exact":
            qh = np.stack([T_.softmax(hl[b, k]) for k in range(K)])
            acc = np.zeros(T, dtype=bool)
            post = P_.posterior_exact(topo, tok, p, qh, inp["u_accept"][b],
                                      inp["u_resample"][b], with_margins=want_margins)
        else:
            raise ValueError(mode)
        kc, vc, Lnext, hnext = P_.commit(topo, post["last_node"], vf["k"], vf["v"], vf["y"],
                                         widen(inp["k_cache"][b]), widen(inp["v_cache"][b]), L)
        per["tokens"].append(tok)
        per["positions"].append(pos)
        for k_ in ("q", "k", "v", "o", "y", "logits"):
            per[k_].append(vf[k_])
        per["p_entropy"].append(ent)
        per["argmax"].append(am)
        per["acc"].append(acc)
        for k_ in ("accept_len", "last_node", "best_path", "out_tokens", "next_root"):
            per[k_].append(post[k_])
        per["kv_len_next"].append(Lnext)
        per["h_next"].append(hnext)
        per["k_cache_next"].append(kc)
        per["v_cache_next"].append(vc)
        per["row_max"].append(logits.max(axis=-1))
        if want_margins:
            per["topk_margin"].append([H_.topk_margin(hl[b, k], s_max) for k in range(K)])
            per["decision_margin"].append(
                P_.decision_margins(topo, tok, logits, tau, mode, eps, delta, p, ent))
            per["argmax_margin"].append(P_.argmax_margin(logits[post["last_node"]]))
            if mode == "exact":
                per["draft_margin"].append(T_.draft_margins(topo, hl[b], inp["u_draft"][b]))
                per["accept_margin"].append(post["accept_margin"])
                per["draw_margin"].append(post["draw_margin"])
    for k_, v_ in per.items():
        if v_:
            res[k_] = np.stack([np.asarray(x) for x in v_])
    return res
