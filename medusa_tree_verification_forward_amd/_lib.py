"""ctypes binding of ``libmedusa_mi355x.so`` (argument marshalling only).

Every function here converts its arguments (torch tensors on the GPU,
numpy arrays for host inputs) into the C ABI's plain pointers and sizes,
calls the library, and raises ``MedusaError`` on a nonzero return. No step
of the method runs in Python. The library must have been built (see
``build.py``); importing the package without it raises immediately.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmedusa_mi355x.so")

OK = 0
ERR_ARG = -1
ERR_UNSUPPORTED = -2
ERR_WORKSPACE = -3
ERR_CAPACITY = -4
ERR_HIP = -5

BF16 = 0
F32 = 1
GREEDY = 0
TYPICAL = 1
EXACT = 2
DRAFT_TOPK = 0
DRAFT_SAMPLE = 1
MODES = {"greedy": GREEDY, "typical": TYPICAL, "exact": EXACT}


class MedusaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"medusa error {code}: {msg}")
        self.code = code


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "d", "V", "K", "H", "Dh", "Lmax", "N", "P", "s_max", "dtype")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m medusa_tree_verification_forward_amd.build` "
        "or `__graft_entry__.build()`. There is no fallback path.")

_lib = ctypes.CDLL(LIB_PATH)


class StepArgs(ctypes.Structure):
    """Mirror of medusa_step_args (include/medusa.h), member for member."""
    _P, _I, _F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    _fields_ = [
        ("h", _P), ("W1", _P), ("b1_or_null", _P), ("W2", _P),
        ("tree_ranks_host", _P), ("draft_mode", _I), ("root_tok", _P), ("u_draft_or_null", _P),
        ("tree_mask", _P), ("parent", _P), ("retrieve", _P),
        ("E", _P), ("W_qkv", _P), ("W_o", _P), ("W_lm", _P), ("rope_theta", _F),
        ("k_cache", _P), ("v_cache", _P), ("kv_len", _P),
        ("mode", _I), ("temperature", _F), ("eps", _F), ("delta", _F),
        ("u_accept_or_null", _P), ("u_resample_or_null", _P),
        ("topk_ids", _P), ("topk_logits", _P), ("head_lse_or_null", _P),
        ("head_logits_or_null", _P), ("z_or_null", _P), ("tree_tokens", _P), ("position_ids", _P),
        ("k_tree", _P), ("v_tree", _P), ("y", _P), ("row_stats", _P), ("row_argmax", _P),
        ("child_logit", _P), ("verify_logits_or_null", _P), ("accept_len", _P),
        ("best_path", _P), ("last_node", _P), ("out_tokens", _P), ("next_root", _P),
        ("h_next", _P), ("kv_len_out_or_null", _P), ("W2_packed_or_null", _P),
        ("W1_packed_or_null", _P),
    ]

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t
_SP = ctypes.POINTER(Shape)

_SIGS = {
    "medusa_last_error": ([], ctypes.c_char_p),
    "medusa_version": ([], ctypes.c_char_p),
    "medusa_workspace_bytes": ([_SP], _SZ),
    "medusa_heads_forward": ([_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P],
                             _I),
    "medusa_build_tree": ([_SP, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P], _I),
    "medusa_tree_attention": ([_SP, _P, _P, _P, _P, _P, _P, _P, _F, _P, _P, _SZ, _P], _I),
    "medusa_packed_weight_bytes": ([_SP, _I], _SZ),
    "medusa_pack_weight": ([_SP, _I, _P, _I, _P, _P], _I),
    "medusa_verify_forward": ([_SP, _P, _P, _P, _P, _F, _P, _P, _P, _P, _P, _P, _P, _F,
                               _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], _I),
    "medusa_evaluate_posterior": ([_SP, _I, _F, _F, _F, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                   _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], _I),
    "medusa_commit": ([_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P], _I),
    "medusa_step": ([_SP, ctypes.POINTER(StepArgs), _P, _SZ, _P], _I),
    "medusa_step_timed": ([_SP, ctypes.POINTER(StepArgs), _P, _SZ, _P, _P, _P], _I),
    "medusa_step_static": ([_SP, ctypes.POINTER(StepArgs), _P], _I),
    "medusa_sparse_tree": ([_I, _I, _P, _I, _P, _P, _P, _P], _I),
    "medusa_generate": ([_SP, ctypes.POINTER(StepArgs), _I, _P, _P, _P, _SZ, _P], _I),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name, None)
    if _fn is not None:
        _fn.argtypes = _args
        _fn.restype = _res


def exported_symbols():
    """Names of the C ABI functions the loaded library exports."""
    return [n for n in _SIGS if getattr(_lib, n, None) is not None]


def last_error() -> str:
    return _lib.medusa_last_error().decode()


def version() -> str:
    return _lib.medusa_version().decode()


def _check(rc: int):
    if rc != OK:
        raise MedusaError(rc, last_error())


def _ptr(t) -> Optional[int]:
    """Device pointer of a torch tensor (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _current_stream() -> int:
    """torch's current stream on the current device (the capture stream while
    a graph is being recorded), without building a Stream object (~3 us a
    call)."""
    import torch
    C = torch._C
    if hasattr(C, "_cuda_getCurrentRawStream") and hasattr(C, "_cuda_getDevice"):
        return C._cuda_getCurrentRawStream(C._cuda_getDevice())
    return torch.cuda.current_stream().cuda_stream


def _stream(stream) -> Optional[int]:
    if stream is None:
        return _current_stream()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_shape(B, d, V, K, H, Dh, Lmax, N, P, s_max, dtype) -> Shape:
    return Shape(B, d, V, K, H, Dh, Lmax, N, P, s_max,
                 dtype if isinstance(dtype, int) else (F32 if dtype == "f32" else BF16))




def workspace_bytes(shape: Shape) -> int:
    n = _lib.medusa_workspace_bytes(ctypes.byref(shape))
    if n == 0:
        raise MedusaError(ERR_ARG, last_error())
    return int(n)


def heads_forward(shape, h, W1, W2, topk_ids, topk_logits, workspace, *, b1=None,
                  head_lse=None, head_logits=None, z=None, W1_packed=None, W2_packed=None,
                  stream=None):
    _check(_lib.medusa_heads_forward(
        ctypes.byref(shape), _ptr(h), _ptr(W1), _ptr(W1_packed), _ptr(b1), _ptr(W2),
        _ptr(W2_packed),
        _ptr(topk_ids),
        _ptr(topk_logits), _ptr(head_lse), _ptr(head_logits), _ptr(z), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def build_tree(shape, tree_ranks: np.ndarray, root_tok, kv_len, tree_tokens, tree_mask,
               position_ids, retrieve, parent, depth, *, draft_mode=DRAFT_TOPK, topk_ids=None,
               head_logits=None, head_lse=None, u_draft=None, stream=None):
    """tree_mask, retrieve, parent and depth may be None (not written)."""
    ranks = np.ascontiguousarray(tree_ranks, dtype=np.int32)
    rp = ranks.ctypes.data if ranks.size else None
    _check(_lib.medusa_build_tree(
        ctypes.byref(shape), rp, int(draft_mode), _ptr(root_tok), _ptr(topk_ids),
        _ptr(head_logits), _ptr(head_lse), _ptr(u_draft), _ptr(kv_len), _ptr(tree_tokens),
        _ptr(tree_mask), _ptr(position_ids), _ptr(retrieve), _ptr(parent), _ptr(depth),
        _stream(stream)))


def generate(shape, args: StepArgs, n_steps: int, out_tokens_steps, accept_len_steps, workspace,
             *, stream=None):
    """medusa_generate: n_steps composite steps with the state kept on the device."""
    _check(_lib.medusa_generate(ctypes.byref(shape), ctypes.byref(args), int(n_steps),
                                _ptr(out_tokens_steps), _ptr(accept_len_steps), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream)))


def sparse_tree(a, budget: int):
    """medusa_sparse_tree: (tree_ranks [N][K] int32 canonical, weights [N] float64,
    pick_order [N] int32) for the rank-probability table a [K][S]."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    if a.ndim != 2:
        raise ValueError("a must be [K][S]")
    K, S = a.shape
    cap = max(int(budget), 1)
    ranks = np.full((cap, max(K, 1)), -1, dtype=np.int32)
    weights = np.zeros(cap, dtype=np.float64)
    order = np.zeros(cap, dtype=np.int32)
    n = ctypes.c_int32(0)
    _check(_lib.medusa_sparse_tree(int(K), int(S), a.ctypes.data if a.size else None, int(budget),
                                   ranks.ctypes.data, weights.ctypes.data, order.ctypes.data,
                                   ctypes.addressof(n)))
    N = n.value
    return ranks[:N].copy(), weights[:N].copy(), order[:N].copy()


def tree_attention(shape, q, k_tree, v_tree, k_cache, v_cache, kv_len, tree_mask, scale, out,
                   workspace, *, stream=None):
    _check(_lib.medusa_tree_attention(
        ctypes.byref(shape), _ptr(q), _ptr(k_tree), _ptr(v_tree), _ptr(k_cache), _ptr(v_cache),
        _ptr(kv_len), _ptr(tree_mask), float(scale), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def packed_weight_bytes(shape: Shape, rows: int) -> int:
    n = _lib.medusa_packed_weight_bytes(ctypes.byref(shape), int(rows))
    if n == 0:
        raise MedusaError(ERR_ARG, last_error())
    return int(n)


PACK_PLAIN = 0
PACK_QKV = 1


def pack_weight(shape, kind, W, rows, W_packed, *, stream=None):
    """Pack a row-major [rows][d] weight into the verify GEMMs' tile order."""
    _check(_lib.medusa_pack_weight(ctypes.byref(shape), int(kind), _ptr(W), int(rows),
                                   _ptr(W_packed), _stream(stream)))


def packed_copy(shape, kind, W, rows, *, stream=None):
    """A new device buffer holding W packed (allocated with torch, same dtype)."""
    import torch
    n = packed_weight_bytes(shape, rows)
    out = torch.empty(n // W.element_size(), dtype=W.dtype, device=W.device)
    pack_weight(shape, kind, W, rows, out, stream=stream)
    return out


def packed_heads_w1(shape, W1, *, stream=None):
    """W1 [K][d][d] packed as one [K d][d] matrix (medusa_heads_forward's
    W1_packed_or_null)."""
    K, d = W1.shape[0], W1.shape[1]
    return packed_copy(shape, PACK_PLAIN, W1.reshape(K * d, d), K * d, stream=stream)


def packed_heads_w2(shape, W2, *, stream=None):
    """W2 [K][V][d] packed per head (medusa_heads_forward's W2_packed_or_null):
    each head's [V][d] block packed plain (rows = V), heads one after another."""
    import torch
    K, V = W2.shape[0], W2.shape[1]
    per = packed_weight_bytes(shape, V) // W2.element_size()
    out = torch.empty(K * per, dtype=W2.dtype, device=W2.device)
    for k in range(K):
        pack_weight(shape, PACK_PLAIN, W2[k], V, out[k * per:(k + 1) * per], stream=stream)
    return out


def verify_forward(shape, E, W_qkv, W_o, W_lm, rope_theta, tree_tokens, position_ids,
                   tree_mask, parent, k_cache, v_cache, kv_len, temperature, k_tree_out,
                   v_tree_out, y_out, row_stats, row_argmax, child_logit, workspace, *,
                   verify_logits=None, stream=None):
    _check(_lib.medusa_verify_forward(
        ctypes.byref(shape), _ptr(E), _ptr(W_qkv), _ptr(W_o), _ptr(W_lm), float(rope_theta),
        _ptr(tree_tokens), _ptr(position_ids), _ptr(tree_mask), _ptr(parent), _ptr(k_cache),
        _ptr(v_cache), _ptr(kv_len), float(temperature), _ptr(k_tree_out), _ptr(v_tree_out),
        _ptr(y_out), _ptr(row_stats), _ptr(row_argmax), _ptr(child_logit),
        _ptr(verify_logits), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def evaluate_posterior(shape, mode, temperature, eps, delta, row_stats, row_argmax,
                       child_logit, tree_tokens, parent, retrieve, accept_len, best_path,
                       last_node, out_tokens, next_root, workspace, *, verify_logits=None,
                       head_logits=None, head_lse=None, u_accept=None, u_resample=None,
                       stream=None):
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    _check(_lib.medusa_evaluate_posterior(
        ctypes.byref(shape), m, float(temperature), float(eps), float(delta), _ptr(row_stats),
        _ptr(row_argmax), _ptr(child_logit), _ptr(verify_logits), _ptr(tree_tokens),
        _ptr(parent), _ptr(retrieve), _ptr(head_logits), _ptr(head_lse), _ptr(u_accept),
        _ptr(u_resample), _ptr(accept_len), _ptr(best_path), _ptr(last_node),
        _ptr(out_tokens), _ptr(next_root), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def commit(shape, last_node, parent, k_tree, v_tree, y, k_cache, v_cache, kv_len, h_next, *,
           stream=None):
    _check(_lib.medusa_commit(
        ctypes.byref(shape), _ptr(last_node), _ptr(parent), _ptr(k_tree), _ptr(v_tree), _ptr(y),
        _ptr(k_cache), _ptr(v_cache), _ptr(kv_len), _ptr(h_next), _stream(stream)))


def step(shape, args: StepArgs, workspace, *, stream=None):
    """The composite step (medusa_step); `args` holds every pointer, and its
    tree_ranks_host member must point at host memory that outlives the call."""
    _check(_lib.medusa_step(ctypes.byref(shape), ctypes.byref(args), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(stream)))


def step_timed(shape, args: StepArgs, workspace, ev_w2_start, ev_w2_end, *, stream=None):
    """medusa_step_timed: the composite step, recording the two events
    (torch.cuda.Event, created by a first record, or raw handles) on the
    stream around the vocabulary-projection kernel."""
    def h(e):
        return e if isinstance(e, int) else e.cuda_event
    _check(_lib.medusa_step_timed(ctypes.byref(shape), ctypes.byref(args), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream),
                                  h(ev_w2_start), h(ev_w2_end)))


STATIC_WORKSPACE_BYTES = 64 << 20   # MEDUSA_STATIC_WORKSPACE_BYTES


def step_static(shape, args: StepArgs, *, stream=None):
    """medusa_step_static: the composite step on the library's own per-GPU
    workspace (no workspace argument, nothing allocated)."""
    _check(_lib.medusa_step_static(ctypes.byref(shape), ctypes.byref(args), _stream(stream)))
