"""Posterior evaluation, longest accepted prefix and commit (test infrastructure only).

Sources:

* Typical acceptance ("Medusa 深读", §5, acceptance equation): a candidate x
  is accepted iff p(x | context) > min(eps, delta * exp(-H(p(. | context)))),
  H(p) = -sum_x p(x) log p(x). The first token is the base LM head's greedy
  prediction and is accepted unconditionally, so every step makes progress;
  the longest fully accepted prefix is committed (same section).
* Greedy matching ("Medusa Part I", Part 2; "Medusa 深读", §5 rule table):
  starting at the first drafted position, accept while the draft equals the
  target's argmax; the first mismatch ends the prefix.
* Exact speculative sampling ("Medusa: Faster LLM text generation",
  Acceptance rules; "Medusa 深读", §3.2 and §5 rule table): accept with
  probability min(1, p/q); at the first rejection draw the replacement from
  the normalised positive residual max(0, p - q). Exact only if the drafts
  were sampled from q.

Readings:

* Typical: strict ">", natural log, p is the tempered verify distribution
  softmax(logits / tau) and H is taken of that same p. The condition is
  applied to each child c with the distribution of c's parent.
* Greedy: a child c is accepted iff its token equals the argmax (lowest id
  on ties) of its parent's logits; tau plays no part.
* Exact on a tree (the pages give only the chain rule): drafts are i.i.d.
  draws from q_depth; at an accepted node v with target p the children are
  tried in canonical order; child c is accepted iff u_acc[c] * q(x_c) <
  p(x_c); after each rejection p <- norm(max(0, p - q)) (kept as is if that
  residual is all zero). If no child is accepted, or v has no children, the
  next root is an inverse-CDF draw from the current p with u_res[v]. With
  one child per node this is the chain rule of the pages.
* An accepted node needs its parent accepted. The committed node is the
  deepest accepted node, the lowest canonical index among equals; the
  committed tokens are the root-to-node path. The best path is the first
  (canonical leaf order) path through that node.
* Next root (greedy, typical): the argmax of the committed node's logits (the
  base LM head's greedy prediction at the new last position).
"""

from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .tree import Topology, inverse_cdf, inverse_cdf_margin


def typical_accepts(p_tok: float, entropy: float, eps: float, delta: float) -> bool:
    """p(x) > min(eps, delta * exp(-H)), strict."""
    return bool(p_tok > min(eps, delta * np.exp(-entropy)))


def accept_greedy(topo: Topology, tokens: np.ndarray, argmax: np.ndarray) -> np.ndarray:
    acc = np.zeros(topo.T, dtype=bool)
    acc[0] = True
    for c in range(1, topo.T):
        acc[c] = int(tokens[c]) == int(argmax[topo.parent[c]])
    return acc


def accept_typical(topo: Topology, tokens: np.ndarray, p: np.ndarray, H: np.ndarray,
                   eps: float, delta: float) -> np.ndarray:
    acc = np.zeros(topo.T, dtype=bool)
    acc[0] = True
    for c in range(1, topo.T):
        v = topo.parent[c]
        acc[c] = typical_accepts(float(p[v, tokens[c]]), float(H[v]), eps, delta)
    return acc


def longest_prefix_paths(topo: Topology, acc: np.ndarray):
    """Per path: number of leading accepted nodes after the root.

    Returns (accept_len [P], best path = first path with the maximum)."""
    P = topo.P
    alen = np.zeros(P, dtype=np.int32)
    for p in range(P):
        n = 0
        for j in range(1, topo.K + 1):
            node = topo.retrieve[p, j]
            if node < 0 or not acc[node]:
                break
            n += 1
        alen[p] = n
    return alen, int(np.argmax(alen))


def longest_prefix_nodes(topo: Topology, acc: np.ndarray):
    """Per node: accepted = acc and parent accepted; the root always is.

    Returns (accepted [T], best node = lowest index among deepest accepted)."""
    ok = np.zeros(topo.T, dtype=bool)
    ok[0] = True
    for n in range(1, topo.T):          # parents precede children in canonical order
        ok[n] = bool(acc[n]) and ok[topo.parent[n]]
    dmax = int(topo.depth[ok].max())
    best = int(np.nonzero(ok & (topo.depth == dmax))[0][0])
    return ok, best


def first_path_through(topo: Topology, node: int) -> int:
    d = int(topo.depth[node])
    hits = np.nonzero(topo.retrieve[:, d] == node)[0]
    return int(hits[0])


def _result(topo: Topology, tokens: np.ndarray, best: int, next_root: int) -> Dict:
    path = topo.path(best)
    out = np.full(topo.K + 1, -1, dtype=np.int32)
    out[:len(path)] = tokens[path]
    return dict(accept_len=int(topo.depth[best]), last_node=int(best),
                best_path=first_path_through(topo, best), out_tokens=out,
                next_root=int(next_root))


def posterior_deterministic(topo: Topology, tokens: np.ndarray, acc: np.ndarray,
                            argmax: np.ndarray) -> Dict:
    """Greedy / typical: longest accepted prefix and the next root token."""
    _, best = longest_prefix_nodes(topo, acc)
    return _result(topo, tokens, best, int(argmax[best]))


def _log_gap(a: float, b: float) -> float:
    """|log a - log b| for the test a < b; inf when exactly one side is 0
    (the decision cannot flip), 0 when both are."""
    if a > 0 and b > 0:
        return float(abs(np.log(a) - np.log(b)))
    return 0.0 if a == b else float(np.inf)


def posterior_exact(topo: Topology, tokens: np.ndarray, p_rows: np.ndarray,
                    q_heads: np.ndarray, u_accept: np.ndarray,
                    u_resample: np.ndarray, with_margins: bool = False) -> Dict:
    """Recursive p/q rejection over the tree (reading above).

    p_rows [T, V]: target distribution at every node; q_heads [K, V]: the
    drafting distribution of each depth (head k drafts depth k+1, 0-based
    index k); u_accept, u_resample [T]. with_margins adds "accept_margin"
    (the smallest |log(u q(x)) - log p(x)| over the acceptance tests taken,
    inf if none) and "draw_margin" (``inverse_cdf_margin`` of the final
    draw): how far the walk's decisions are from flipping.
    """
    v = 0
    p = np.array(p_rows[0], dtype=np.float64)
    acc_margin = np.inf
    while True:
        kids = topo.children(v)
        if not kids:
            break
        q = q_heads[topo.depth[v]]
        taken = None
        for c in kids:
            x = int(tokens[c])
            uq = float(u_accept[c]) * q[x]
            acc_margin = min(acc_margin, _log_gap(uq, p[x]))
            if uq < p[x]:
                taken = c
                break
            r = np.maximum(p - q, 0.0)
            if r.sum() > 0:
                p = r / r.sum()
        if taken is None:
            break
        v = taken
        p = np.array(p_rows[v], dtype=np.float64)
    nxt = inverse_cdf(p, float(u_resample[v]))
    out = _result(topo, tokens, v, nxt)
    if with_margins:
        out["accept_margin"] = float(acc_margin)
        out["draw_margin"] = inverse_cdf_margin(p, float(u_resample[v]))
    return out


def commit(topo: Topology, last_node: int, k_tree: np.ndarray, v_tree: np.ndarray,
           y: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, L: int):
    """Append the committed path's K/V rows at prefix rows L.. and return
    (k_cache', v_cache', new length, h_next).

    k_tree, v_tree [T, H, Dh]; caches [H, Lmax, Dh] (one sequence, any dtype
    of values); y [T, d]. The next step's hidden state is y at the committed
    node (the accepted prefix becomes the next context, "Medusa: Faster LLM
    text generation", Introduction).
    """
    path = topo.path(last_node)
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    for i, n in enumerate(path):
        kc[:, L + i, :] = k_tree[n]
        vc[:, L + i, :] = v_tree[n]
    return kc, vc, L + len(path), np.array(y[last_node], dtype=np.float64)


def decision_margins(topo: Topology, tokens: np.ndarray, logits: np.ndarray,
                     tau: float, mode: str, eps: float, delta: float,
                     p: Optional[np.ndarray] = None, H: Optional[np.ndarray] = None):
    """Distance of every acceptance decision from its flip point.

    greedy: logit gap between the child's token and the best other token of
    the parent row; typical: |log p(x) - log threshold|. Returns [T] (root:
    inf). Used to tell true near-ties from disagreements.
    """
    logits = np.asarray(logits, dtype=np.float64)
    m = np.full(topo.T, np.inf)
    for c in range(1, topo.T):
        v = topo.parent[c]
        row = logits[v]
        x = int(tokens[c])
        if mode == "greedy":
            others = np.delete(row, x)
            m[c] = abs(row[x] - others.max())
        elif mode == "typical":
            thr = min(eps, delta * np.exp(-H[v]))
            m[c] = abs(np.log(p[v, x]) - np.log(thr))
    return m


def argmax_margin(row: np.ndarray) -> float:
    v = np.sort(np.asarray(row, dtype=np.float64))[::-1]
    return float(v[0] - v[1])
