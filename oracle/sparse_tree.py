"""Calibrated sparse tree under a node budget (test infrastructure only).

Source: "Medusa 深读", §6.2. A calibration set gives, for each head k and
rank i, a_k^(i) = P(R_k = i), the probability that the true token sits at
rank i of head k. Under the cross-head independence approximation a rank path
(i_1, ..., i_k) has weight w = prod_j a_j^(i_j). The tree is grown greedily:
start with the depth-1 nodes on the frontier, and B times move the
frontier node of largest weight into the tree and put its children on the
frontier. By the tail-sum formula E[L] = sum_{k>=1} P(L >= k), the expected
depth covered by the tree is the sum of the path weights of its nodes, so
each greedy pick adds its own weight to that expectation.

Readings: ranks are 1-based in the page and 0-based here; equal weights are
broken by the lexicographically smaller rank path; the returned spec is
listed in canonical order (depth, then lexicographic) for the tree stages.
"""

from __future__ import annotations

from typing import List, Tuple

import numpy as np


def path_weight(a: np.ndarray, path: Tuple[int, ...]) -> float:
    """prod_j a[j, path[j]] (0-based ranks)."""
    w = 1.0
    for j, r in enumerate(path):
        w *= float(a[j, r])
    return w


def greedy_tree(a: np.ndarray, budget: int) -> List[Tuple[int, ...]]:
    """Rank paths in the order the greedy builder picks them.

    a [K, S]: a[k, i] = P(head k+1's true token has rank i) (0-based).
    """
    K, S = a.shape
    frontier = [(r,) for r in range(S)]
    picked: List[Tuple[int, ...]] = []
    while len(picked) < budget and frontier:
        best = min(frontier, key=lambda t: (-path_weight(a, t), t))
        frontier.remove(best)
        picked.append(best)
        if len(best) < K:
            frontier.extend(best + (r,) for r in range(S))
    return picked


def expected_cover(a: np.ndarray, paths: List[Tuple[int, ...]]) -> float:
    """E[L_cover] = sum of the path weights of the tree's nodes."""
    return float(sum(path_weight(a, t) for t in paths))


def to_spec(paths: List[Tuple[int, ...]], K: int) -> np.ndarray:
    """Canonical [N][K] rank table (-1 padded) of a prefix-closed path set."""
    rows = sorted(paths, key=lambda t: (len(t), t))
    out = np.full((len(rows), K), -1, dtype=np.int32)
    for i, t in enumerate(rows):
        out[i, :len(t)] = t
    return out
