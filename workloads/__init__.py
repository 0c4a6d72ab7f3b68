"""Seeded synthetic workloads for one Medusa verify step.

This module only draws random tensors of the right shapes and distributions.
It holds none of the method's arithmetic: no heads, no tree, no attention, no
acceptance rule. Both the CPU oracle (``oracle/``) and the HIP path take their
inputs from here, so that the two sides see identical bytes.

The shapes follow the pages' workloads: batch 1, prefix KV up to 4096, five
Medusa heads, trees of a few dozen nodes, temperature 0.7 for typical
acceptance ("Medusa: Faster LLM text generation", Results; "Medusa 深读", §7.1
Table 1 and §7.2). The pages measure on MT-Bench with Vicuna weights and
trained heads; none of that exists here, so seeded Gaussian tensors of the same
shapes stand in for them.

Conventions
-----------
* bf16 tensors are numpy ``uint16`` arrays holding bf16 bit patterns
  (fp32 draws rounded to nearest-even). fp32 workloads keep ``float32``.
* Every tensor has its own generators: ``np.random.default_rng([seed, tid,
  sub, chunk])`` for each 2^20-element chunk of a Gaussian tensor (``sub``
  is the sequence index for the KV cache, else 0), ``default_rng([seed,
  tid])`` for the small integer and uniform draws; adding a tensor never
  shifts another one, and the values do not depend on the thread count.
* Weights are stored row-major ``[out][in]`` (``W1[k]`` is d x d, ``W2[k]``
  is V x d, ``W_qkv`` is 3d x d with the q, k, v blocks stacked, ``W_lm`` is
  V x d, the embedding ``E`` is V x d).
* The KV cache is ``[B][H][Lmax][Dh]``; rows at or past a sequence's prefix
  length are zero.
"""

from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional, Tuple

import numpy as np

# Tensor ids: one independent stream per tensor.
TID = dict(h=0, W1=1, b1=2, W2=3, E=4, W_qkv=5, W_o=6, W_lm=7, K=8, V=9,
           kv_len=10, root=11, u_draft=12, u_accept=13, u_resample=14)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape, tree, acceptance rule and value distributions of one workload."""

    name: str
    dtype: str                 # "f32" or "bf16": storage type of weights, E, KV
    B: int                     # sequences
    d: int                     # hidden width
    V: int                     # vocabulary
    K: int                     # Medusa heads = tree depth
    s: Tuple[int, ...]         # per-depth top-s of the Cartesian tree
    H: int                     # attention heads of the verifier layer
    Dh: int                    # head dimension
    L: Optional[int]           # prefix length (None: ragged, drawn per sequence)
    L_range: Tuple[int, int]   # inclusive range for ragged prefix lengths
    mode: str                  # "greedy", "typical" or "exact"
    tau: float                 # verifier temperature
    eps: float                 # typical acceptance hard threshold
    delta: float               # typical acceptance entropy factor
    w1_std: Optional[float]    # std of W1 entries (None: 1/sqrt(d))
    entropy_target: Optional[float]  # scale W_lm so LM logits on h have this entropy (nats)
    seed: int
    rope_theta: float = 10000.0

    @property
    def s_max(self) -> int:
        return max(self.s)


WORKLOADS: Dict[str, Workload] = {
    # Tiny fp32 case the oracle finishes in well under a second.
    "tiny_fp32": Workload(
        name="tiny_fp32", dtype="f32", B=1, d=256, V=1000, K=3, s=(2, 2, 2),
        H=4, Dh=64, L=64, L_range=(64, 64), mode="greedy", tau=1.0,
        eps=0.09, delta=0.3, w1_std=0.02, entropy_target=2.0, seed=1001),
    # Vicuna-7B-shaped step, typical acceptance: the throughput workload.
    "vicuna7b_typical": Workload(
        name="vicuna7b_typical", dtype="bf16", B=1, d=4096, V=32000, K=5,
        s=(3, 2, 2, 1, 1), H=32, Dh=128, L=2048, L_range=(2048, 2048),
        mode="typical", tau=0.7, eps=0.09, delta=0.3, w1_std=None,
        entropy_target=None, seed=1002),
    # Vicuna-13B-shaped step, wider 136-node tree, 4k prefix.
    "vicuna13b_typical": Workload(
        name="vicuna13b_typical", dtype="bf16", B=1, d=5120, V=32000, K=5,
        s=(4, 3, 2, 2, 1), H=40, Dh=128, L=4096, L_range=(4096, 4096),
        mode="typical", tau=0.7, eps=0.09, delta=0.3, w1_std=0.02,
        entropy_target=2.0, seed=1003),
    # Eight independent 7B-shaped sequences with ragged prefixes, greedy.
    "vicuna7b_batch8_ragged": Workload(
        name="vicuna7b_batch8_ragged", dtype="bf16", B=8, d=4096, V=32000, K=5,
        s=(3, 2, 2, 1, 1), H=32, Dh=128, L=None, L_range=(512, 4096),
        mode="greedy", tau=1.0, eps=0.09, delta=0.3, w1_std=None,
        entropy_target=None, seed=1004),
    # 7B shapes with exact p/q rejection sampling, 4k prefix.
    "vicuna7b_exact": Workload(
        name="vicuna7b_exact", dtype="bf16", B=1, d=4096, V=32000, K=5,
        s=(3, 2, 2, 1, 1), H=32, Dh=128, L=4096, L_range=(4096, 4096),
        mode="exact", tau=1.0, eps=0.09, delta=0.3, w1_std=None,
        entropy_target=None, seed=1005),
}


def scaled(w: Workload, **overrides) -> Workload:
    """A copy of ``w`` with some fields replaced (for small parity shapes)."""
    return dataclasses.replace(w, **overrides)


# --------------------------------------------------------------------------
# bf16 storage helpers (data preparation only)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); return uint16 bit patterns.

    Finite inputs only (the sum below cannot wrap for them)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    r = (b >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += b
    r >>= 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32)


def _rng(w: Workload, name: str) -> np.random.Generator:
    return np.random.default_rng([w.seed, TID[name]])


_CHUNK = 1 << 20   # elements per independent stream


def _normal(w: Workload, name: str, shape, std: float, store: str, sub: int = 0) -> np.ndarray:
    """N(0, std^2) draws for tensor `name`. The tensor is cut into fixed
    chunks of 2^20 elements; chunk c uses its own stream
    default_rng([seed, tensor id, sub, c]), so the values do not depend on
    how many threads produce them."""
    shape = tuple(int(x) for x in shape)
    total = int(np.prod(shape)) if shape else 1
    out = np.empty(total, dtype=np.uint16 if store == "bf16" else np.float32)
    nchunks = (total + _CHUNK - 1) // _CHUNK

    def work(c):
        lo, hi = c * _CHUNK, min(total, (c + 1) * _CHUNK)
        x = np.random.default_rng([w.seed, TID[name], sub, c]).standard_normal(
            hi - lo, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[lo:hi] = f32_to_bf16_bits(x) if store == "bf16" else x

    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
    else:
        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(work, range(nchunks)))
    return out.reshape(shape)


def _entropy_nats(logits: np.ndarray) -> float:
    # Plain entropy of a softmax, used only to size the LM-head scale of the
    # synthetic input (the input distribution, not a step of the method).
    z = logits - logits.max()
    e = np.exp(z)
    p = e / e.sum()
    nz = p > 0
    return float(-(p[nz] * np.log(p[nz])).sum())


def _lm_scale_for_entropy(W_lm_f32: np.ndarray, h: np.ndarray, target: float) -> float:
    """Bisect alpha so that softmax(alpha * W_lm h) has entropy ``target`` nats."""
    base = W_lm_f32.astype(np.float64) @ h.astype(np.float64)
    lo, hi = 1e-3, 1e3
    for _ in range(200):
        mid = np.sqrt(lo * hi)
        if _entropy_nats(mid * base) > target:
            lo = mid   # entropy too high: logits need more spread
        else:
            hi = mid
        if hi / lo < 1 + 1e-9:
            break
    return float(np.sqrt(lo * hi))


def cartesian_ranks(s) -> np.ndarray:
    """Rank tuples (0-based, -1 padded) of the Cartesian top-s tree, one row per
    non-root node, depth-major then lexicographic. This lists the tree the
    pages describe ("Medusa 深读", §6.1): every combination of per-head ranks,
    with shared prefixes stored once."""
    K = len(s)
    rows = []
    frontier = [()]
    for k in range(K):
        nxt = []
        for t in frontier:
            for r in range(s[k]):
                nxt.append(t + (r,))
        rows.extend(nxt)
        frontier = nxt
    out = np.full((len(rows), K), -1, dtype=np.int32)
    for i, t in enumerate(rows):
        out[i, :len(t)] = t
    return out


def lmax_for(w: Workload) -> int:
    """KV capacity: room for the longest prefix plus a full commit (K+1 rows),
    rounded up to a multiple of 64."""
    Lmax = w.L_range[1] + w.K + 1
    return (Lmax + 63) // 64 * 64


def make_inputs(w: Workload, with_weights: bool = True,
                only: Optional[Tuple[str, ...]] = None) -> Dict[str, np.ndarray]:
    """Draw every input of one verify step for workload ``w``.

    Returns a dict of numpy arrays (see the module docstring for layouts):
    h [B,d] f32; W1 [K,d,d]; W2 [K,V,d]; E [V,d]; W_qkv [3d,d]; W_o [d,d];
    W_lm [V,d]; k_cache, v_cache [B,H,Lmax,Dh]; kv_len [B] int32;
    root [B] int32; ranks [N,K] int32; u_draft, u_accept, u_resample [B,T] f32.
    ``only`` restricts the weight tensors drawn (names as in the dict); every
    tensor has its own stream, so a partial draw gives the same values.
    """

    def want(name):
        return with_weights and (only is None or name in only)

    store = w.dtype
    d, V, K, B, H, Dh = w.d, w.V, w.K, w.B, w.H, w.Dh
    ranks = cartesian_ranks(w.s)
    N = ranks.shape[0]
    T = N + 1
    Lmax = lmax_for(w)
    out: Dict[str, np.ndarray] = {"ranks": ranks}

    out["h"] = _rng(w, "h").standard_normal((B, d), dtype=np.float32)

    if w.L is not None:
        kv_len = np.full(B, w.L, dtype=np.int32)
    else:
        kv_len = _rng(w, "kv_len").integers(w.L_range[0], w.L_range[1],
                                            endpoint=True, size=B).astype(np.int32)
    out["kv_len"] = kv_len
    out["root"] = _rng(w, "root").integers(0, V, size=B).astype(np.int32)

    inv = 1.0 / np.sqrt(d)
    w1_std = w.w1_std if w.w1_std is not None else inv
    if want("W1"):
        out["W1"] = _normal(w, "W1", (K, d, d), w1_std, store)
    if want("W2"):
        out["W2"] = _normal(w, "W2", (K, V, d), inv, store)
    if want("E"):
        out["E"] = _normal(w, "E", (V, d), 1.0, store)
    if want("W_qkv"):
        out["W_qkv"] = _normal(w, "W_qkv", (3 * d, d), inv, store)
    if want("W_o"):
        out["W_o"] = _normal(w, "W_o", (d, d), inv, store)
    if want("W_lm"):
        if w.entropy_target is None:
            out["W_lm"] = _normal(w, "W_lm", (V, d), inv, store)
        else:
            raw = _normal(w, "W_lm", (V, d), inv, "f32")
            alpha = _lm_scale_for_entropy(raw, out["h"][0], w.entropy_target)
            raw *= np.float32(alpha)
            out["W_lm"] = f32_to_bf16_bits(raw) if store == "bf16" else raw
    for name in ("K", "V"):
        if want("k_cache" if name == "K" else "v_cache"):
            cache = np.zeros((B, H, Lmax, Dh),
                             dtype=np.uint16 if store == "bf16" else np.float32)
            for b in range(B):
                L = int(kv_len[b])
                if L > 0:
                    cache[b, :, :L, :] = _normal(w, name, (H, L, Dh), 1.0, store, sub=b)
            out["k_cache" if name == "K" else "v_cache"] = cache

    for name in ("u_draft", "u_accept", "u_resample"):
        out[name] = _rng(w, name).random((B, T), dtype=np.float32)
    return out


# --------------------------------------------------------------------------
# Planted agreement between the heads and the verifier (decoding loop)
# --------------------------------------------------------------------------

def planted_inputs(a: np.ndarray, ranks: np.ndarray, *, V: int = 512, H: int = 4,
                   Dh: int = 128, L: int = 64, n_steps: int = 32, B: int = 1,
                   seed: int = 2024) -> Dict[str, np.ndarray]:
    """Inputs under which the heads agree with the verifier at planted ranks.

    Random weights give the heads no agreement with the verifier, so the
    acceptance of a decoding loop says nothing. Here the "language" is a fixed
    permutation pi of a vocabulary of V tokens with one-hot embeddings
    (d = V): E[t] = e_t and W_lm[pi(t)] = 8 e_t, so the verifier's next token
    after t is pi(t) by a wide margin (the attention and output projection,
    random bf16 weights of magnitude ~1/sqrt(d) and ~1% of that, add little
    to the one-hot state); W1 = 0, so z_k = h. For each head k
    (1-based) and token t the true continuation pi^(k+1)(t) is placed at a
    rank drawn from the row a[k-1] (0-based ranks; beyond the head's pool
    with probability 1 - sum a[k-1]), decoys filling the other ranks, so the
    rank of the true token at depth k is distributed as a[k-1]. The state
    starts at h = e_t0, root = pi(t0). Returns the step inputs plus "pi" and
    "true_rank" [K][V] (the planted rank, S meaning beyond the pool).
    """
    a = np.asarray(a, dtype=np.float64)
    K, S = a.shape
    d = V
    rng = np.random.default_rng([seed, V, K, S])
    pi = rng.permutation(V).astype(np.int64)
    pipow = [np.arange(V)]
    for _ in range(K + 1):
        pipow.append(pi[pipow[-1]])
    out: Dict[str, np.ndarray] = {"ranks": np.ascontiguousarray(ranks, dtype=np.int32)}
    one, eight = 0x3F80, 0x4100                       # bf16 bit patterns of 1.0 and 8.0
    E = np.zeros((V, d), dtype=np.uint16)
    E[np.arange(V), np.arange(V)] = one
    W_lm = np.zeros((V, d), dtype=np.uint16)
    W_lm[pi, np.arange(V)] = eight
    W2 = np.zeros((K, V, d), dtype=np.uint16)
    true_rank = np.full((K, V), S, dtype=np.int32)
    p_ranks = np.concatenate([a, 1.0 - a.sum(axis=1, keepdims=True).clip(0, 1)], axis=1)
    p_ranks /= p_ranks.sum(axis=1, keepdims=True)
    level = f32_to_bf16_bits(8.0 * (1.0 - 0.0625 * np.arange(S + 2, dtype=np.float32)))
    ks, vs, ts, ls = [], [], [], []
    for k in range(K):
        for t in range(V):
            target = int(pipow[k + 2][t])
            r = int(rng.choice(S + 1, p=p_ranks[k]))
            true_rank[k, t] = r
            cand = rng.choice(V, size=S + 1, replace=False)
            slots = [int(x) for x in cand if x != target][:S]
            if r < S:
                slots[r] = target
            else:
                slots.append(target)          # just below the pool
            for i, v in enumerate(slots):
                ks.append(k)
                vs.append(v)
                ts.append(t)
                ls.append(level[i if i < S else S + 1])
    W2[np.array(ks), np.array(vs), np.array(ts)] = np.array(ls, dtype=np.uint16)
    def random_bf16(shape, exponent):
        # random sign and mantissa at a fixed binary exponent: |x| in [2^e, 2^(e+1))
        n = int(np.prod(shape))
        bits = np.frombuffer(rng.bytes(2 * n), dtype=np.uint16).reshape(shape)
        return (bits & np.uint16(0x807F)) | np.uint16((127 + exponent) << 7)
    e_qkv = int(np.floor(np.log2(1.0 / np.sqrt(d)))) - 1   # |w| ~ 1/sqrt(d)
    W_qkv = random_bf16((3 * d, d), e_qkv)
    W_o = random_bf16((d, d), e_qkv - 7)                   # ~1% of the residual
    Lmax = L + n_steps * (K + 1) + 8
    # the prefix rows are random; the rows the loop commits are written by it
    kc = np.zeros((B, H, Lmax, Dh), dtype=np.uint16)
    vc = np.zeros((B, H, Lmax, Dh), dtype=np.uint16)
    kc[:, :, :L] = f32_to_bf16_bits(rng.standard_normal((B, H, L, Dh), dtype=np.float32))
    vc[:, :, :L] = f32_to_bf16_bits(rng.standard_normal((B, H, L, Dh), dtype=np.float32))
    t0 = rng.integers(0, V, size=B)
    h = np.zeros((B, d), dtype=np.float32)
    h[np.arange(B), t0] = 1.0
    out.update(
        h=h, W1=np.zeros((K, d, d), dtype=np.uint16), W2=W2, E=E,
        W_qkv=W_qkv, W_o=W_o, W_lm=W_lm,
        k_cache=kc, v_cache=vc, kv_len=np.full(B, L, dtype=np.int32),
        root=pi[t0].astype(np.int32), pi=pi.astype(np.int32), true_rank=true_rank)
    return out
