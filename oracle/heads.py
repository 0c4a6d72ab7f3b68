"""Medusa heads (test infrastructure only).

Definition ("Medusa 深读", §3.1, head equation): head k maps the shared last
hidden state h_t to

    p_t^(k) = softmax( W2^(k) ( SiLU(W1^(k) h_t) + h_t ) )

with W1^(k) of shape d x d and W2^(k) of shape V x d (column-vector
convention). Head k (1-based) predicts the token k+1 positions past the
base model's next token, so head k supplies depth k of the candidate tree
(same section; the shift convention of "Medusa Part I", Part 5, agrees).
Every head reads the same h_t and owns separate weights ("Medusa Part I",
Part 3). The residual block there is ``h + silu(Linear(h))`` whose Linear
carries a bias initialised to zero; the bias is optional here and absent in
every workload.

SiLU(x) = x * sigmoid(x) (the activation ``F.silu`` of "Medusa Part I",
Part 3).
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from .numerics import widen


def silu(x: np.ndarray) -> np.ndarray:
    """x * sigmoid(x), evaluated as x / (1 + exp(-x))."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def lm_head(W: np.ndarray, y: np.ndarray) -> np.ndarray:
    """Logits of a vocab projection: W [V, d] applied to y [..., d]."""
    return np.asarray(y, dtype=np.float64) @ widen(W).T


def residual_block(W1k: np.ndarray, h: np.ndarray,
                   b1k: Optional[np.ndarray] = None) -> np.ndarray:
    """z = h + SiLU(W1 h (+ b1)) for h [B, d]; W1k [d, d] stored [out][in]."""
    h = np.asarray(h, dtype=np.float64)
    u = h @ widen(W1k).T
    if b1k is not None:
        u = u + widen(b1k)
    return h + silu(u)


def heads_forward(h: np.ndarray, W1: np.ndarray, W2: np.ndarray,
                  b1: Optional[np.ndarray] = None):
    """All K heads on h [B, d].

    Returns (z [B, K, d], logits [B, K, V]) in float64. Weights are widened
    one head at a time to bound memory.
    """
    h = np.asarray(h, dtype=np.float64)
    B, d = h.shape
    K, V = W2.shape[0], W2.shape[1]
    z = np.empty((B, K, d))
    logits = np.empty((B, K, V))
    for k in range(K):
        z[:, k, :] = residual_block(W1[k], h, None if b1 is None else b1[k])
        logits[:, k, :] = lm_head(W2[k], z[:, k, :])
    return z, logits


def top_s(logits: np.ndarray, s: int):
    """The s best tokens of one logit vector.

    Order: higher logit first; equal logits by lower token id. This is a
    stable sort on the key (-logit, id). Returns (ids [s] int64, values [s]).
    """
    logits = np.asarray(logits, dtype=np.float64)
    order = np.lexsort((np.arange(logits.shape[-1]), -logits))
    ids = order[:s]
    return ids, logits[ids]


def log_sum_exp(logits: np.ndarray) -> float:
    """log sum_v exp(logit_v), computed with the maximum factored out."""
    logits = np.asarray(logits, dtype=np.float64)
    m = logits.max()
    return float(m + np.log(np.exp(logits - m).sum()))


def heads_topk(logits: np.ndarray, s_max: int):
    """Top-s_max pools and log-sum-exp for every (sequence, head).

    logits [B, K, V] -> ids [B, K, s_max] int32, values [B, K, s_max],
    lse [B, K].
    """
    B, K, V = logits.shape
    ids = np.empty((B, K, s_max), dtype=np.int32)
    vals = np.empty((B, K, s_max))
    lse = np.empty((B, K))
    for b in range(B):
        for k in range(K):
            i, v = top_s(logits[b, k], s_max)
            ids[b, k] = i
            vals[b, k] = v
            lse[b, k] = log_sum_exp(logits[b, k])
    return ids, vals, lse


def topk_margin(logits: np.ndarray, s: int) -> float:
    """Smallest gap between consecutive logits among the s+1 best.

    The ordered top-s list is decided by these gaps (the set by the last one,
    the order inside it by the others), so this is the near-tie measure of
    the top-s decision.
    """
    v = np.sort(np.asarray(logits, dtype=np.float64))[::-1]
    n = min(s + 1, v.shape[0])
    if n < 2:
        return np.inf
    return float(np.min(v[:n - 1] - v[1:n]))
