"""Multi-step decoding, composed from the oracle step (test infrastructure only).

Source: "Medusa: Faster LLM text generation" (decoding with Medusa heads)
and "Medusa 深读" (the generate loop): every step drafts from the hidden
state of the last accepted token, verifies the tree in one pass, commits the
accepted prefix, and the base model's prediction at the last accepted node
becomes the next step's root. The state handed from step to step is (h,
root, kv_len, KV cache); h is kept in float32 and the cache in its storage
format, as the device keeps them.
"""

from __future__ import annotations

from typing import Dict

import numpy as np

from .step import verify_step


def _to_storage(x: np.ndarray, like: np.ndarray) -> np.ndarray:
    """Committed cache (float64, exactly representable in the storage type)
    back to the storage format: bf16 bit patterns (uint16) or float32."""
    if like.dtype == np.uint16:
        f = np.asarray(x, dtype=np.float32)
        if not np.array_equal(f.astype(np.float64), np.asarray(x, dtype=np.float64)):
            raise ValueError("cache value not representable in float32")
        bits = f.view(np.uint32)
        if np.any(bits & 0xFFFF):
            raise ValueError("cache value not representable in bf16")
        return (bits >> 16).astype(np.uint16)
    return np.asarray(x, dtype=np.float32)


def generate(inp: Dict[str, np.ndarray], n_steps: int, exact_margins: bool = False,
             **step_kw) -> Dict:
    """Run n_steps steps; returns out_tokens [n][B][K+1], accept_len [n][B]
    and the final state (h, root, kv_len, k_cache, v_cache). Exact mode takes
    per-step uniforms inp['u_*_steps'] [n][B][T]; with exact_margins it also
    returns, per step and sequence [n][B], the margins of the step's
    sampling decisions as the step oracle defines them: "draft_margin" (the
    smallest over the drafted nodes), "accept_margin" and "draw_margin"."""
    st = dict(inp)
    toks, acc = [], []
    margins = {"draft_margin": [], "accept_margin": [], "draw_margin": []}
    for i in range(n_steps):
        if "u_draft_steps" in inp:
            for name in ("u_draft", "u_accept", "u_resample"):
                st[name] = inp[name + "_steps"][i]
        r = verify_step(st, want_margins=exact_margins, **step_kw)
        toks.append(r["out_tokens"])
        acc.append(r["accept_len"])
        if exact_margins:
            margins["draft_margin"].append(r["draft_margin"].min(axis=1))
            margins["accept_margin"].append(r["accept_margin"])
            margins["draw_margin"].append(r["draw_margin"])
        st["h"] = np.asarray(r["h_next"], dtype=np.float32)
        st["root"] = np.asarray(r["next_root"], dtype=np.int32)
        st["kv_len"] = np.asarray(r["kv_len_next"], dtype=np.int32)
        st["k_cache"] = _to_storage(r["k_cache_next"], inp["k_cache"])
        st["v_cache"] = _to_storage(r["v_cache_next"], inp["v_cache"])
    K1 = inp["ranks"].shape[1] + 1
    B = np.asarray(inp["h"]).shape[0]
    out = dict(out_tokens=np.array(toks, dtype=np.int32).reshape(n_steps, B, K1),
                accept_len=np.array(acc, dtype=np.int32).reshape(n_steps, B),
                h=st["h"], root=st["root"], kv_len=st["kv_len"],
                k_cache=st["k_cache"], v_cache=st["v_cache"])
    if exact_margins:
        for k, v in margins.items():
            out[k] = np.array(v, dtype=np.float64).reshape(n_steps, B)
    return out
