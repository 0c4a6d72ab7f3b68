"""Synthetic one-layer verifier and tree attention (test infrastructure only).

What the pages fix: the target model scores the whole candidate tree in one
batched forward pass ("Medusa: Faster LLM text generation", Tree attention),
under a mask that lets a node see the prefix, the virtual root and its own
branch ancestors but no sibling branch, with one shared position index per
depth ("Medusa 深读", §6.1). Each root-to-leaf path is then causally the same
as an independent candidate sequence.

What the pages leave open, and the reading taken here: the target's
internals. The plainest single layer whose verify logits depend on the tree
tokens and positions is used:

    x  = E[token]                                  (embedding rows)
    q, k, v = RoPE(x Wq^T), RoPE(x Wk^T), x Wv^T   (per attention head)
    o  = tree-masked softmax(q k^T / sqrt(Dh)) v    over [prefix KV ; tree]
    y  = x + o Wo^T
    logits = y Wlm^T

RoPE uses base theta = 10000 and the rotate-half pairing (i, i + Dh/2), the
Llama-family convention (the pages' models are Vicuna / Llama). No
normalisation and no MLP. These internals are parity unpinned by the pages;
the path-equivalence invariant (``path_attention`` against
``tree_attention``) pins the mask and positions.

Rounding points (mirroring the bf16 storage of the HIP path): q, k, v are
rounded to bf16 after RoPE, o before the output projection and y before the
LM head. ``bf16=False`` turns every rounding point off (the fp32 workload).
"""

from __future__ import annotations

from typing import Dict, List

import numpy as np

from .numerics import round_bf16, widen


def _maybe_round(x: np.ndarray, bf16: bool) -> np.ndarray:
    return round_bf16(x) if bf16 else x


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate pairs (i, i + Dh/2) of x [n, H, Dh] by angle pos * theta^(-2i/Dh)."""
    x = np.asarray(x, dtype=np.float64)
    n, H, Dh = x.shape
    half = Dh // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / Dh)                       # [half]
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]  # [n, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def qkv_project(x: np.ndarray, W_qkv: np.ndarray, pos: np.ndarray, H: int, Dh: int,
                theta: float, bf16: bool):
    """q, k, v [n, H, Dh] for embedding rows x [n, d] at positions pos [n]."""
    d = H * Dh
    W = widen(W_qkv)
    qkv = np.asarray(x, dtype=np.float64) @ W.T
    n = qkv.shape[0]
    q = qkv[:, 0 * d:1 * d].reshape(n, H, Dh)
    k = qkv[:, 1 * d:2 * d].reshape(n, H, Dh)
    v = qkv[:, 2 * d:3 * d].reshape(n, H, Dh)
    q = _maybe_round(rope(q, pos, theta), bf16)
    k = _maybe_round(rope(k, pos, theta), bf16)
    v = _maybe_round(v, bf16)
    return q, k, v


def _softmax_attend(qi: np.ndarray, keys: np.ndarray, vals: np.ndarray, scale: float):
    """softmax(qi . keys^T * scale) @ vals for one query vector."""
    s = keys @ qi * scale
    s = s - s.max()
    p = np.exp(s)
    p /= p.sum()
    return p @ vals


def tree_attention(q, k_tree, v_tree, k_cache, v_cache, L: int, mask: np.ndarray,
                   scale: float) -> np.ndarray:
    """Masked attention of every tree node over [prefix ; tree].

    q, k_tree, v_tree [T, H, Dh]; k_cache, v_cache [H, >=L, Dh] (one
    sequence); node i attends to prefix rows 0..L-1 and to tree node j iff
    mask[i, j]. Returns o [T, H, Dh].
    """
    T, H, Dh = q.shape
    o = np.empty((T, H, Dh))
    kc = widen(k_cache)[:, :L, :]
    vc = widen(v_cache)[:, :L, :]
    for h in range(H):
        for i in range(T):
            sel = np.nonzero(mask[i])[0]
            keys = np.concatenate([kc[h], k_tree[sel, h, :]], axis=0)
            vals = np.concatenate([vc[h], v_tree[sel, h, :]], axis=0)
            o[i, h] = _softmax_attend(q[i, h], keys, vals, scale)
    return o


def path_attention(tokens_path: List[int], E, W_qkv, k_cache, v_cache, L: int,
                   H: int, Dh: int, theta: float, scale: float, bf16: bool) -> np.ndarray:
    """Ordinary causal attention of the last token of one candidate sequence.

    The candidate sequence is the prefix (given by its KV rows) followed by
    the tokens of one root-to-node path at positions L, L+1, ...; the layer
    runs as a plain causal transformer layer on it and the attention output
    of the last token is returned ([H, Dh]). This is the brute-force
    statement of what tree attention must reproduce for that node.
    """
    toks = np.asarray(tokens_path, dtype=np.int64)
    x = widen(E)[toks]
    pos = L + np.arange(len(toks))
    q, k, v = qkv_project(x, W_qkv, pos, H, Dh, theta, bf16)
    kc = widen(k_cache)[:, :L, :]
    vc = widen(v_cache)[:, :L, :]
    last = len(toks) - 1
    out = np.empty((H, Dh))
    for h in range(H):
        keys = np.concatenate([kc[h], k[:, h, :]], axis=0)
        vals = np.concatenate([vc[h], v[:, h, :]], axis=0)
        out[h] = _softmax_attend(q[last, h], keys, vals, scale)
    return out


def verifier_forward(E, W_qkv, W_o, W_lm, tokens, positions, mask, k_cache, v_cache,
                     L: int, H: int, Dh: int, theta: float, bf16: bool,
                     want_logits: bool = True) -> Dict[str, np.ndarray]:
    """One synthetic verifier layer over the T tree rows of one sequence.

    Returns q, k, v [T, H, Dh], o (attention output) [T, H, Dh],
    y [T, d] (pre-LM-head hidden state) and logits [T, V].
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    x = widen(E)[tokens]
    q, k, v = qkv_project(x, W_qkv, positions, H, Dh, theta, bf16)
    scale = 1.0 / np.sqrt(Dh)
    o = tree_attention(q, k, v, k_cache, v_cache, L, mask, scale)
    T = tokens.shape[0]
    o_in = _maybe_round(o.reshape(T, H * Dh), bf16)
    y = x + o_in @ widen(W_o).T
    out = dict(q=q, k=k, v=v, o=o, y=y)
    if want_logits:
        out["logits"] = _maybe_round(y, bf16) @ widen(W_lm).T
    return out


def row_distribution(logits: np.ndarray, tau: float):
    """Per-row tempered distribution p = softmax(logits / tau).

    Returns (p [T, V], entropy H [T] in nats, argmax [T]). The argmax takes
    the lowest token id among equal logits.
    """
    z = np.asarray(logits, dtype=np.float64) / tau
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    p = e / e.sum(axis=-1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        plogp = np.where(p > 0, p * np.log(p), 0.0)
    H = -plogp.sum(axis=-1)
    am = np.argmax(np.asarray(logits, dtype=np.float64), axis=-1).astype(np.int32)
    return p, H, am
