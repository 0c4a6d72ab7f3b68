"""Device buffers and call sequence of one verify step (marshalling only).

``VerifyStep`` allocates, with PyTorch on the GPU, every buffer the five C
ABI calls of one step read or write, then issues them in order on one
stream: heads -> tree -> verify forward -> posterior -> commit. All
arithmetic happens in the HIP library.
"""

from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from . import _lib as L


def to_device(x: np.ndarray, device="cuda"):
    """numpy -> torch tensor on the GPU; uint16 arrays hold bf16 bit patterns."""
    import torch
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(x).to(device)


def to_host(t) -> np.ndarray:
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class VerifyStep:
    """One Medusa verify step on the GPU for fixed shapes.

    inputs: dict of numpy arrays as produced by the workload generator
    (h, W1, W2, E, W_qkv, W_o, W_lm, k_cache, v_cache, kv_len, root, ranks,
    u_draft, u_accept, u_resample).
    """

    def __init__(self, inputs: Dict[str, np.ndarray], *, H: int, Dh: int, s_max: int,
                 mode: str, tau: float, eps: float, delta: float, theta: float,
                 want_logits: bool = False):
        import torch
        self.torch = torch
        f32 = inputs["W2"].dtype == np.float32
        K, V, d = inputs["W2"].shape
        B = inputs["h"].shape[0]
        ranks = np.ascontiguousarray(inputs["ranks"], dtype=np.int32)
        N = ranks.shape[0]
        T = N + 1
        P = self._count_paths(ranks)
        Lmax = inputs["k_cache"].shape[2]
        self.shape = L.make_shape(B, d, V, K, H, Dh, Lmax, N, P, s_max, "f32" if f32 else "bf16")
        self.B, self.T, self.K, self.V, self.d, self.P = B, T, K, V, d, P
        self.mode, self.tau, self.eps, self.delta, self.theta = mode, tau, eps, delta, theta
        self.ranks = ranks
        dev = {k: to_device(v) for k, v in inputs.items()
               if k not in ("ranks",) and isinstance(v, np.ndarray)}
        self.inp = dev
        # the verify GEMMs read their weights in MFMA tile order, packed once here
        self.packed = {name: L.packed_copy(self.shape, kind, dev[name], rows)
                       for name, kind, rows in (("W_qkv", L.PACK_QKV, 3 * d),
                                                ("W_o", L.PACK_PLAIN, d),
                                                ("W_lm", L.PACK_PLAIN, V))}
        # batches of 3 or more bf16 sequences stream W2 as packed tiles
        # (a second copy of W2; the per-row passes of 1-2 sequences read W2)
        batched = B >= 3 and not f32
        self.w2_packed = L.packed_heads_w2(self.shape, dev["W2"]) if batched else None
        self.w1_packed = L.packed_heads_w1(self.shape, dev["W1"]) if batched else None
        self.kv_len0 = dev["kv_len"].clone()
        kv = np.asarray(inputs["kv_len"])
        self._uniform_kv = int(kv[0]) if np.all(kv == kv[0]) else None
        i32, f = torch.int32, torch.float32
        z = lambda shape, dt: torch.zeros(shape, dtype=dt, device="cuda")  # noqa: E731
        exact = mode == "exact"
        elem = torch.float32 if f32 else torch.bfloat16
        self.out = dict(
            topk_ids=z((B, K, s_max), i32), topk_logits=z((B, K, s_max), f),
            head_lse=z((B, K), f),
            head_logits=z((B, K, V), f) if (exact or want_logits) else None,
            z=z((B, K, d), f),
            tree_tokens=z((B, T), i32), tree_mask=z((T, T), torch.uint8),
            position_ids=z((B, T), i32), retrieve=z((P, K + 1), i32), parent=z((T,), i32),
            depth=z((T,), i32), k_tree=z((B, T, H, Dh), elem), v_tree=z((B, T, H, Dh), elem),
            y=z((B, T, d), f), row_stats=z((B, T, 3), f), row_argmax=z((B, T), i32),
            child_logit=z((B, T), f),
            verify_logits=z((B, T, V), f) if (exact or want_logits) else None,
            accept_len=z((B,), i32), best_path=z((B,), i32), last_node=z((B,), i32),
            out_tokens=z((B, K + 1), i32), next_root=z((B,), i32), h_next=z((B, d), f),
        )
        self.ws = torch.zeros(L.workspace_bytes(self.shape), dtype=torch.uint8, device="cuda")
        # the topology (mask, paths, parent, depth) depends only on the spec:
        # written once here, then every step writes tokens and positions only
        self.tree(topology=True)

    @staticmethod
    def _count_paths(ranks: np.ndarray) -> int:
        tuples = set()
        for row in ranks:
            t = tuple(int(r) for r in row if r >= 0)
            tuples.add(t)
        if not tuples:
            return 1
        parents = {t[:-1] for t in tuples}
        return sum(1 for t in tuples if t not in parents)

    # -- the five calls -------------------------------------------------------------
    def heads(self, stream=None):
        o, i = self.out, self.inp
        L.heads_forward(self.shape, i["h"], i["W1"], i["W2"], o["topk_ids"], o["topk_logits"],
                        self.ws, head_lse=o["head_lse"], head_logits=o["head_logits"], z=o["z"],
                        W1_packed=self.w1_packed, W2_packed=self.w2_packed, stream=stream)

    def tree(self, stream=None, topology: bool = False):
        o, i = self.out, self.inp
        sample = self.mode == "exact"
        topo = (lambda t: t) if topology else (lambda t: None)  # noqa: E731
        L.build_tree(self.shape, self.ranks, i["root"], i["kv_len"], o["tree_tokens"],
                     topo(o["tree_mask"]), o["position_ids"], topo(o["retrieve"]),
                     topo(o["parent"]), topo(o["depth"]),
                     draft_mode=L.DRAFT_SAMPLE if sample else L.DRAFT_TOPK,
                     topk_ids=o["topk_ids"], head_logits=o["head_logits"],
                     head_lse=o["head_lse"], u_draft=i.get("u_draft") if sample else None,
                     stream=stream)

    def verify(self, stream=None):
        o, i = self.out, self.inp
        w = self.packed
        L.verify_forward(self.shape, i["E"], w["W_qkv"], w["W_o"], w["W_lm"], self.theta,
                         o["tree_tokens"], o["position_ids"], o["tree_mask"], o["parent"],
                         i["k_cache"], i["v_cache"], i["kv_len"], self.tau, o["k_tree"],
                         o["v_tree"], o["y"], o["row_stats"], o["row_argmax"], o["child_logit"],
                         self.ws, verify_logits=o["verify_logits"], stream=stream)

    def posterior(self, stream=None):
        o, i = self.out, self.inp
        exact = self.mode == "exact"
        L.evaluate_posterior(self.shape, self.mode, self.tau, self.eps, self.delta,
                             o["row_stats"], o["row_argmax"], o["child_logit"],
                             o["tree_tokens"], o["parent"], o["retrieve"], o["accept_len"],
                             o["best_path"], o["last_node"], o["out_tokens"], o["next_root"],
                             self.ws, verify_logits=o["verify_logits"] if exact else None,
                             head_logits=o["head_logits"] if exact else None,
                             head_lse=o["head_lse"] if exact else None,
                             u_accept=i.get("u_accept") if exact else None,
                             u_resample=i.get("u_resample") if exact else None, stream=stream)

    def commit(self, stream=None):
        o, i = self.out, self.inp
        L.commit(self.shape, o["last_node"], o["parent"], o["k_tree"], o["v_tree"], o["y"],
                 i["k_cache"], i["v_cache"], i["kv_len"], o["h_next"], stream=stream)

    def reset_kv_len(self):
        """Restore the prefix lengths (one small fill kernel when they are all
        equal, else a device copy)."""
        if self._uniform_kv is not None:
            self.inp["kv_len"].fill_(self._uniform_kv)
        else:
            self.inp["kv_len"].copy_(self.kv_len0)

    def step_args(self, keep_kv_len: bool = False):
        """medusa_step arguments over this object's buffers (built once per
        variant). keep_kv_len: the commit writes the advanced prefix lengths
        to a buffer of their own (self.kv_len_next) and leaves kv_len as it
        is, so that the step can be repeated over the same prefix."""
        cached = getattr(self, "_args_keep" if keep_kv_len else "_args", None)
        if cached is not None:
            return cached
        o, i, w = self.out, self.inp, self.packed
        p = L._ptr
        exact = self.mode == "exact"
        self._ranks_host = np.ascontiguousarray(self.ranks, dtype=np.int32)
        a = L.StepArgs()
        a.h, a.W1, a.W2 = p(i["h"]), p(i["W1"]), p(i["W2"])
        a.W2_packed_or_null = p(self.w2_packed)
        a.W1_packed_or_null = p(self.w1_packed)
        a.b1_or_null = p(i.get("b1"))
        a.tree_ranks_host = self._ranks_host.ctypes.data if self._ranks_host.size else None
        a.draft_mode = L.DRAFT_SAMPLE if exact else L.DRAFT_TOPK
        a.root_tok = p(i["root"])
        a.u_draft_or_null = p(i.get("u_draft")) if exact else None
        a.tree_mask, a.parent, a.retrieve = p(o["tree_mask"]), p(o["parent"]), p(o["retrieve"])
        a.E, a.W_qkv, a.W_o, a.W_lm = p(i["E"]), p(w["W_qkv"]), p(w["W_o"]), p(w["W_lm"])
        a.rope_theta = self.theta
        a.k_cache, a.v_cache, a.kv_len = p(i["k_cache"]), p(i["v_cache"]), p(i["kv_len"])
        a.mode = L.MODES[self.mode]
        a.temperature, a.eps, a.delta = self.tau, self.eps, self.delta
        a.u_accept_or_null = p(i.get("u_accept")) if exact else None
        a.u_resample_or_null = p(i.get("u_resample")) if exact else None
        a.topk_ids, a.topk_logits = p(o["topk_ids"]), p(o["topk_logits"])
        a.head_lse_or_null, a.head_logits_or_null = p(o["head_lse"]), p(o["head_logits"])
        a.z_or_null = p(o["z"])
        a.tree_tokens, a.position_ids = p(o["tree_tokens"]), p(o["position_ids"])
        a.k_tree, a.v_tree, a.y = p(o["k_tree"]), p(o["v_tree"]), p(o["y"])
        a.row_stats, a.row_argmax = p(o["row_stats"]), p(o["row_argmax"])
        a.child_logit, a.verify_logits_or_null = p(o["child_logit"]), p(o["verify_logits"])
        a.accept_len, a.best_path, a.last_node = (p(o["accept_len"]), p(o["best_path"]),
                                                  p(o["last_node"]))
        a.out_tokens, a.next_root, a.h_next = (p(o["out_tokens"]), p(o["next_root"]),
                                               p(o["h_next"]))
        if keep_kv_len:
            import torch
            self.kv_len_next = torch.empty_like(i["kv_len"])
            a.kv_len_out_or_null = p(self.kv_len_next)
            self._args_keep = a
        else:
            self._args = a
        return a

    def run_step(self, stream=None, keep_kv_len: bool = False, w2_events=None):
        """The whole step as one composite call (medusa_step); see step_args
        for keep_kv_len. w2_events = (start, end): medusa_step_timed records
        them around the vocabulary-projection kernel."""
        if w2_events is None:
            # the call's marshalled arguments, built once per variant (the
            # stream is looked up each call: a graph capture changes it)
            key = "_call_keep" if keep_kv_len else "_call"
            call = getattr(self, key, None)
            if call is None:
                import ctypes
                call = (ctypes.byref(self.shape), ctypes.byref(self.step_args(keep_kv_len)),
                        self.ws.data_ptr(), self.ws.numel() * self.ws.element_size())
                setattr(self, key, call)
            L._check(L._lib.medusa_step(call[0], call[1], call[2], call[3], L._stream(stream)))
        else:
            L.step_timed(self.shape, self.step_args(keep_kv_len), self.ws, w2_events[0],
                         w2_events[1], stream=stream)

    def generate(self, n_steps: int, stream=None, uniforms=None):
        """medusa_generate: n_steps steps with the state kept on the device.
        Returns (out_tokens [n][B][K+1], accept_len [n][B]) device tensors;
        afterwards inp["h"], inp["root"], inp["kv_len"] and the caches hold the
        advanced state. Exact mode takes uniforms = {u_draft, u_accept,
        u_resample}, each a float32 [n][B][T] tensor on the device."""
        import torch
        a = L.StepArgs.from_buffer_copy(self.step_args(False))
        B, K, T = self.shape.B, self.shape.K, self.T
        if self.mode == "exact":
            if uniforms is None:
                raise ValueError("exact mode needs per-step uniforms")
            # the library reads step i's [B][T] block at element
            # i * MEDUSA_ALIGN4(B*T): copy into blocks of that stride (kept
            # alive on self until the next call)
            bt = (B * T + 3) & ~3
            self._u_blocks = {}
            for name in ("u_draft", "u_accept", "u_resample"):
                u = uniforms[name]
                if tuple(u.shape) != (n_steps, B, T):
                    raise ValueError(f"{name}: shape {tuple(u.shape)}, want {(n_steps, B, T)}")
                blk = torch.zeros((max(n_steps, 1), bt), dtype=torch.float32, device=u.device)
                blk[:n_steps, :B * T] = u.reshape(n_steps, B * T)
                self._u_blocks[name] = blk
            a.u_draft_or_null = L._ptr(self._u_blocks["u_draft"])
            a.u_accept_or_null = L._ptr(self._u_blocks["u_accept"])
            a.u_resample_or_null = L._ptr(self._u_blocks["u_resample"])
        ot, al = (B * (K + 1) + 3) & ~3, (B + 3) & ~3   # 16-byte aligned step blocks
        n = max(n_steps, 1)
        toks = torch.full((n, ot), -1, dtype=torch.int32, device="cuda")
        acc = torch.zeros((n, al), dtype=torch.int32, device="cuda")
        L.generate(self.shape, a, n_steps, toks, acc, self.ws, stream=stream)
        return (toks[:n_steps, :B * (K + 1)].reshape(n_steps, B, K + 1),
                acc[:n_steps, :B])

    def run(self, stream=None, commit: bool = True):
        """The whole step: heads, tree, verify forward, posterior, commit."""
        self.heads(stream)
        self.tree(stream)
        self.verify(stream)
        self.posterior(stream)
        if commit:
            self.commit(stream)

    def results(self) -> Dict[str, np.ndarray]:
        return {k: to_host(v) for k, v in self.out.items() if v is not None}
