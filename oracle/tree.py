"""Candidate tree (test infrastructure only).

Source: "Medusa 深读", §6.1 (tree construction and node-count equation) and
§6.2 (rank paths); "Medusa: Faster LLM text generation", Inference
("Proposals and a tree") and Tree attention.

* Head k keeps its top-s_k tokens; the candidate sequences are the
  Cartesian product of the pools, and a tree that stores shared prefixes once
  needs sum_k prod_{j<=k} s_j added nodes for prod_k s_k sequences (§6.1,
  node-count equation; its example with pools of 2 and 3 gives 8 nodes and 6
  sequences).
* A node is named by its rank path (i_1, ..., i_k): i_j is the rank of its
  depth-j token inside head j's pool (§6.2). Ranks here are 0-based
  (0 = best).
* The tree is verified in one pass with an attention mask under which each
  node sees the virtual root and its own ancestors, never a sibling branch,
  and every node at one depth shares one position index (§6.1, last
  paragraph).

Readings taken where the pages are silent:

* Canonical node order: the root is node 0; non-root nodes sorted by depth,
  then lexicographically by rank path. Siblings are therefore in head-rank
  order. Root-to-leaf paths are listed in lexicographic order of the leaf's
  rank path.
* The root is the base LM head's token and is a real row of the verify pass
  (so T = N + 1 rows); it sits at position L, a depth-k node at L + k, where
  L is the prefix length.
* A node sees itself (ordinary causal attention) besides its ancestors.
"""

from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np


def node_count(s: Sequence[int]) -> int:
    """Added (non-root) nodes of the Cartesian tree: sum_k prod_{j<=k} s_j."""
    total, prod = 0, 1
    for sk in s:
        prod *= int(sk)
        total += prod
    return total


def path_count(s: Sequence[int]) -> int:
    """Candidate sequences (root-to-leaf paths): prod_k s_k."""
    prod = 1
    for sk in s:
        prod *= int(sk)
    return prod


def spec_tuples(ranks: np.ndarray) -> List[Tuple[int, ...]]:
    """Rows of a [N][K] rank table (-1 padded) as rank-path tuples."""
    ranks = np.asarray(ranks)
    out = []
    for row in ranks:
        t = []
        for r in row:
            if r < 0:
                break
            t.append(int(r))
        out.append(tuple(t))
    return out


def canonical_key(t: Tuple[int, ...]):
    return (len(t), t)


def check_spec(tuples: List[Tuple[int, ...]], K: Optional[int] = None) -> Optional[str]:
    """Return None for a valid canonical spec, else a reason.

    Valid: non-empty tuples of non-negative ranks, no duplicates, depth at
    most K, every proper non-empty prefix present (prefix-closed), and listed
    in canonical order (depth, then lexicographic).
    """
    seen = set()
    for t in tuples:
        if len(t) == 0:
            return "empty rank path"
        if K is not None and len(t) > K:
            return "rank path deeper than K"
        if any(r < 0 for r in t):
            return "negative rank"
        if t in seen:
            return "duplicate rank path"
        seen.add(t)
    for t in tuples:
        if len(t) > 1 and t[:-1] not in seen:
            return "not prefix-closed"
    if list(tuples) != sorted(tuples, key=canonical_key):
        return "not in canonical order"
    return None


@dataclasses.dataclass
class Topology:
    tuples: List[Tuple[int, ...]]   # node n (>=1) has rank path tuples[n-1]; root is ()
    parent: np.ndarray              # [T] int32, parent[0] = -1
    depth: np.ndarray               # [T] int32
    last_rank: np.ndarray           # [T] int32, -1 for the root
    mask: np.ndarray                # [T, T] uint8, mask[i, j] = j is i or an ancestor of i
    retrieve: np.ndarray            # [P, K+1] int32, root-to-leaf node lists, -1 padded
    K: int

    @property
    def T(self) -> int:
        return self.parent.shape[0]

    @property
    def P(self) -> int:
        return self.retrieve.shape[0]

    def children(self, v: int) -> List[int]:
        """Children of node v in canonical (head-rank) order."""
        return [int(c) for c in np.nonzero(self.parent == v)[0]]

    def path(self, n: int) -> List[int]:
        """Node indices from the root to n inclusive."""
        out = [int(n)]
        while out[-1] != 0:
            out.append(int(self.parent[out[-1]]))
        return out[::-1]


def topology(ranks: np.ndarray, K: int) -> Topology:
    """Parent, depth, ancestor mask and root-to-leaf paths of a canonical spec."""
    tuples = spec_tuples(ranks)
    err = check_spec(tuples, K)
    if err is not None:
        raise ValueError(err)
    T = len(tuples) + 1
    index = {(): 0}
    for n, t in enumerate(tuples, start=1):
        index[t] = n
    parent = np.full(T, -1, dtype=np.int32)
    depth = np.zeros(T, dtype=np.int32)
    last_rank = np.full(T, -1, dtype=np.int32)
    for n, t in enumerate(tuples, start=1):
        parent[n] = index[t[:-1]]
        depth[n] = len(t)
        last_rank[n] = t[-1]
    topo = Topology(tuples, parent, depth, last_rank,
                    np.zeros((T, T), dtype=np.uint8),
                    np.zeros((0, K + 1), dtype=np.int32), K)
    for i in range(T):
        for j in topo.path(i):
            topo.mask[i, j] = 1
    has_child = np.zeros(T, dtype=bool)
    has_child[parent[1:]] = True
    # Paths are listed in lexicographic order of their leaf's rank path, so
    # that every path through a node precedes every path through a later
    # node of the same depth (this keeps "first longest path" and "first
    # deepest node" the same choice on trees with leaves at several depths).
    leaves = sorted((n for n in range(1, T) if not has_child[n]), key=lambda n: tuples[n - 1])
    if T == 1:
        leaves = [0]
    retrieve = np.full((len(leaves), K + 1), -1, dtype=np.int32)
    for p, leaf in enumerate(leaves):
        nodes = topo.path(leaf)
        retrieve[p, :len(nodes)] = nodes
    topo.retrieve = retrieve
    return topo


def position_ids(topo: Topology, L: int) -> np.ndarray:
    """Position of every node: the root at L, a depth-k node at L + k."""
    return (int(L) + topo.depth).astype(np.int32)


def draft_tokens_topk(topo: Topology, root: int, topk_ids: np.ndarray) -> np.ndarray:
    """Tokens of the top-s tree: node 0 carries the root token; a node of
    depth k and last rank r carries head k's rank-r token (topk_ids [K][s])."""
    tok = np.empty(topo.T, dtype=np.int32)
    tok[0] = root
    for n in range(1, topo.T):
        tok[n] = topk_ids[topo.depth[n] - 1, topo.last_rank[n]]
    return tok


def inverse_cdf(weights: np.ndarray, u: float) -> int:
    """Inverse-CDF draw from non-negative, not necessarily normalised weights.

    C is the inclusive prefix sum in ascending token id; the draw is the
    smallest x with C(x) > u * C(last). A draw that would land past every
    token with positive weight is clamped to the last such token.
    """
    w = np.asarray(weights, dtype=np.float64)
    C = np.cumsum(w)
    total = C[-1]
    x = int(np.searchsorted(C, u * total, side="right"))
    nz = np.nonzero(w > 0)[0]
    last = int(nz[-1]) if nz.size else w.shape[0] - 1
    return min(x, last)


def inverse_cdf_margin(weights: np.ndarray, u: float) -> float:
    """Distance of an inverse-CDF draw from its flip points.

    With C and the drawn token x as in ``inverse_cdf``, the draw point
    u * C(last) lies in x's step [C(x-1), C(x)); the margin is its distance
    to the nearer edge of that step as a fraction of C(last). A draw
    computed from weights (or a CDF) with relative errors below the margin
    picks the same token; a margin of 0 means the point sits on an edge.
    """
    w = np.asarray(weights, dtype=np.float64)
    C = np.cumsum(w)
    total = C[-1]
    if not total > 0:
        return 0.0
    x = inverse_cdf(w, u)
    point = u * total
    lo = C[x - 1] if x > 0 else 0.0
    return float(max(0.0, min(point - lo, C[x] - point)) / total)


def softmax(logits: np.ndarray, tau: float = 1.0) -> np.ndarray:
    z = np.asarray(logits, dtype=np.float64) / tau
    e = np.exp(z - z.max())
    return e / e.sum()


def draft_tokens_sampled(topo: Topology, root: int, head_logits: np.ndarray,
                         u_draft: np.ndarray) -> np.ndarray:
    """Tokens of a sampled tree (exact mode): every non-root node draws its
    token independently from its depth's head distribution q_k =
    softmax(head logits) with its own uniform u_draft[n]. The node's shape
    is the same as the top-s tree. Drafts must be sampled from a known q for
    p/q acceptance to be exact ("Medusa 深读", §3.2)."""
    q = [softmax(head_logits[k]) for k in range(head_logits.shape[0])]
    tok = np.empty(topo.T, dtype=np.int32)
    tok[0] = root
    for n in range(1, topo.T):
        tok[n] = inverse_cdf(q[topo.depth[n] - 1], float(u_draft[n]))
    return tok


def draft_margins(topo: Topology, head_logits: np.ndarray, u_draft: np.ndarray) -> np.ndarray:
    """inverse_cdf_margin of every node's draw in ``draft_tokens_sampled``
    ([T]; the root, which draws nothing, gets inf)."""
    q = [softmax(head_logits[k]) for k in range(head_logits.shape[0])]
    m = np.full(topo.T, np.inf)
    for n in range(1, topo.T):
        m[n] = inverse_cdf_margin(q[topo.depth[n] - 1], float(u_draft[n]))
    return m
