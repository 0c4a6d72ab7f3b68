"""Host-side checks of the C ABI: the library loads, exports every function
include/medusa.h declares, and rejects bad arguments before touching the GPU
(no compute is launched here)."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    try:
        import medusa_tree_verification_forward_amd as M
    except ImportError as e:
        pytest.fail(f"library not built: {e}")
    return M


def _declared():
    src = open(os.path.join(ROOT, "include", "medusa.h")).read()
    return sorted(set(re.findall(r"\b(medusa_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    M = _lib()
    lib = ctypes.CDLL(M.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(_declared()) <= set(M.exported_symbols()) | {"medusa_last_error", "medusa_version"}


def _shape(M, **kw):
    base = dict(B=1, d=4096, V=32000, K=5, H=32, Dh=128, Lmax=2112, N=45, P=12, s_max=3,
                dtype="bf16")
    base.update(kw)
    return M.make_shape(**base)


def test_workspace_bytes_and_shape_validation():
    M = _lib()
    n = M.workspace_bytes(_shape(M))
    assert n > 0 and n % 256 == 0
    for bad, code in [(dict(Dh=100), M._lib.ERR_ARG), (dict(d=4000, H=40, Dh=100), M._lib.ERR_ARG),
                      (dict(K=9), M._lib.ERR_UNSUPPORTED), (dict(s_max=17), M._lib.ERR_UNSUPPORTED),
                      (dict(N=256, P=1), M._lib.ERR_UNSUPPORTED), (dict(B=0), M._lib.ERR_ARG),
                      (dict(dtype=7), M._lib.ERR_ARG), (dict(V=2), M._lib.ERR_ARG),
                      (dict(H=64, Dh=64, d=4096, Lmax=0), M._lib.ERR_ARG)]:
        with pytest.raises(M.MedusaError) as ei:
            M.workspace_bytes(_shape(M, **bad))
        assert ei.value.code in (M._lib.ERR_ARG, code), bad


class _FakePtr:
    """A non-null, aligned fake device pointer: validation must fail before
    any launch, so it is never dereferenced."""


FAKE = 1 << 20


def _call_tree(M, shape, ranks, **kw):
    args = dict(root_tok=FAKE, kv_len=FAKE, tree_tokens=FAKE, tree_mask=FAKE, position_ids=FAKE,
                retrieve=FAKE, parent=FAKE, depth=FAKE, topk_ids=FAKE)
    args.update(kw)
    lib = M._lib._lib
    return lib.medusa_build_tree(ctypes.byref(shape), ranks.ctypes.data if ranks.size else None,
                                 0, args["root_tok"], args["topk_ids"], None, None, None,
                                 args["kv_len"], args["tree_tokens"], args["tree_mask"],
                                 args["position_ids"], args["retrieve"], args["parent"],
                                 args["depth"], None)


@pytest.mark.parametrize("rows,why", [
    ([[0, -1], [0, 0], [1, -1]], "canonical"),      # depth-2 row before a depth-1 row
    ([[0, -1], [1, 0]], "prefix"),                  # (1,0) without (1,)
    ([[0, -1], [0, -1]], "canonical"),              # duplicate
    ([[0, -1], [3, -1]], "s_max"),                  # rank beyond the pool
    ([[-1, 0]], "padding"),                         # rank after padding
])
def test_tree_spec_rejected_on_host(rows, why):
    M = _lib()
    ranks = np.array(rows, dtype=np.int32)
    shape = _shape(M, K=2, N=len(rows), P=1, s_max=2)
    rc = _call_tree(M, shape, ranks)
    assert rc == M._lib.ERR_ARG
    assert M.last_error() != ""


def test_tree_path_count_must_match():
    M = _lib()
    from workloads import cartesian_ranks
    ranks = cartesian_ranks((2, 2))
    shape = _shape(M, K=2, N=6, P=3, s_max=2)
    assert _call_tree(M, shape, ranks) == M._lib.ERR_ARG
    assert "paths" in M.last_error()


def test_null_and_misaligned_pointers_rejected():
    M = _lib()
    from workloads import cartesian_ranks
    ranks = cartesian_ranks((2, 2))
    shape = _shape(M, K=2, N=6, P=4, s_max=2)
    assert _call_tree(M, shape, ranks, tree_tokens=None) == M._lib.ERR_ARG
    assert "tree_tokens" in M.last_error()
    assert _call_tree(M, shape, ranks, tree_mask=FAKE + 2) == M._lib.ERR_ARG
    assert "tree_mask" in M.last_error()
    assert _call_tree(M, shape, ranks, retrieve=FAKE + 4) == M._lib.ERR_ARG
    assert "aligned" in M.last_error()


def test_heads_workspace_too_small():
    M = _lib()
    shape = _shape(M)
    lib = M._lib._lib
    rc = lib.medusa_heads_forward(ctypes.byref(shape), FAKE, FAKE, None, None, FAKE, None, FAKE,
                                  FAKE, None, None, None, FAKE, 16, None)
    assert rc == M._lib.ERR_WORKSPACE


def test_step_args_layout_matches_header(tmp_path):
    """The binding's StepArgs mirrors medusa_step_args member for member."""
    import shutil
    import subprocess
    M = _lib()
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    names = [f for f, _ in M.StepArgs._fields_]
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "medusa.h"',
             "int main(void) {", '  printf("%zu\\n", sizeof(medusa_step_args));']
    lines += [f'  printf("%zu\\n", offsetof(medusa_step_args, {n}));' for n in names]
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(root, "include"), str(src), "-o", str(exe)],
                   check=True)
    out = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert out[0] == ctypes.sizeof(M.StepArgs)
    assert out[1:] == [getattr(M.StepArgs, n).offset for n in names]


def _step_args(M, ranks, exact=True):
    """medusa_step_args with every device pointer a fake aligned address."""
    a = M.StepArgs()
    for name, _ in M.StepArgs._fields_:
        if name not in ("draft_mode", "mode", "rope_theta", "temperature", "eps", "delta",
                        "tree_ranks_host", "b1_or_null", "kv_len_out_or_null"):
            setattr(a, name, FAKE)
    a.tree_ranks_host = ranks.ctypes.data
    a.draft_mode = M.DRAFT_SAMPLE if exact else M.DRAFT_TOPK
    a.mode = M.EXACT if exact else M.TYPICAL
    a.rope_theta, a.temperature, a.eps, a.delta = 10000.0, 1.0, 0.09, 0.3
    return a


def test_step_validates_every_part_before_launching():
    # A bad pointer of a late part (the verifier's embedding, the posterior's
    # uniforms) is reported as an argument error. On a machine without a GPU
    # a launch would fail with MEDUSA_ERR_HIP, so ERR_ARG shows that the
    # earlier parts (heads, tree) were not launched either.
    M = _lib()
    from workloads import cartesian_ranks
    ranks = cartesian_ranks((3, 2, 2, 1, 1))
    shape = _shape(M)
    nbytes = M.workspace_bytes(shape)
    lib = M._lib._lib
    for field, exact in (("E", False), ("W_lm", True), ("u_accept_or_null", True),
                         ("h_next", False), ("h_next", True)):
        a = _step_args(M, ranks, exact)
        setattr(a, field, None)
        rc = lib.medusa_step(ctypes.byref(shape), ctypes.byref(a), FAKE, nbytes, None)
        assert rc == M._lib.ERR_ARG, (field, rc, M.last_error())
        assert field.split("_or_null")[0] in M.last_error(), (field, M.last_error())


def test_generate_validates_every_step_before_launching():
    # Exact mode at B=1, T=46: a step's uniform block is 46 floats, not a
    # multiple of 4, so the library advances by MEDUSA_ALIGN4(B*T) = 48 per
    # step. A misaligned base pointer is rejected before anything launches,
    # and so is a null pointer that only a later stage reads.
    M = _lib()
    from workloads import cartesian_ranks
    ranks = cartesian_ranks((3, 2, 2, 1, 1))
    shape = _shape(M)
    nbytes = M.workspace_bytes(shape)
    lib = M._lib._lib
    for field, value in (("u_resample_or_null", FAKE + 4), ("u_draft_or_null", FAKE + 8),
                         ("y", None), ("k_tree", FAKE + 2)):
        a = _step_args(M, ranks, exact=True)
        setattr(a, field, value)
        rc = lib.medusa_generate(ctypes.byref(shape), ctypes.byref(a), 5, FAKE, FAKE, FAKE,
                                 nbytes, None)
        assert rc == M._lib.ERR_ARG, (field, rc, M.last_error())
        assert field.split("_or_null")[0] in M.last_error(), (field, M.last_error())
    # the per-step output blocks must be aligned too
    a = _step_args(M, ranks, exact=True)
    rc = lib.medusa_generate(ctypes.byref(shape), ctypes.byref(a), 5, FAKE + 4, FAKE, FAKE,
                             nbytes, None)
    assert rc == M._lib.ERR_ARG and "out_tokens_steps" in M.last_error()
    # the loop advances kv_len in place
    a = _step_args(M, ranks, exact=True)
    a.kv_len_out_or_null = FAKE
    rc = lib.medusa_generate(ctypes.byref(shape), ctypes.byref(a), 5, FAKE, FAKE, FAKE,
                             nbytes, None)
    assert rc == M._lib.ERR_ARG and "kv_len_out_or_null" in M.last_error()


def test_step_timed_needs_both_events():
    M = _lib()
    from workloads import cartesian_ranks
    ranks = cartesian_ranks((3, 2, 2, 1, 1))
    shape = _shape(M)
    a = _step_args(M, ranks, exact=False)
    lib = M._lib._lib
    rc = lib.medusa_step_timed(ctypes.byref(shape), ctypes.byref(a), FAKE,
                               M.workspace_bytes(shape), None, FAKE, None)
    assert rc == M._lib.ERR_ARG and "event" in M.last_error()


def test_step_static_rejects_shapes_beyond_its_workspace():
    # The 13B step (136-node tree, 4k prefix) needs more workspace than the
    # library's static array holds: refused before any device call.
    M = _lib()
    from workloads import cartesian_ranks
    ranks = cartesian_ranks((4, 3, 2, 2, 1))
    shape = _shape(M, d=5120, H=40, Lmax=4160, N=136, P=48, s_max=4)
    assert M.workspace_bytes(shape) > M.STATIC_WORKSPACE_BYTES
    a = _step_args(M, ranks, exact=False)
    rc = M._lib._lib.medusa_step_static(ctypes.byref(shape), ctypes.byref(a), None)
    assert rc == M._lib.ERR_WORKSPACE and "static workspace" in M.last_error()
