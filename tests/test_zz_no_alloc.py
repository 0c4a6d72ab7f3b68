"""medusa_step_static (the step on the library's own per-GPU workspace,
allocating nothing) against medusa_step with a caller workspace: three calls
in a row on one GPU -- the 7B step at full size, then a smaller bf16 step,
then the tiny fp32 step -- each bit-identical to the workspace call, so what
an earlier call left in the shared array changes nothing."""

import numpy as np
import pytest

from workloads import WORKLOADS, scaled

import parity
from gpu_helpers import require_gpu

pytestmark = pytest.mark.gpu


def _outputs(st):
    from medusa_tree_verification_forward_amd.step import to_host
    r = st.results()
    for k in ("k_cache", "v_cache", "kv_len"):
        r[k] = to_host(st.inp[k])
    r["kv_len_next"] = to_host(st.kv_len_next)
    return r


def test_static_workspace_step_equals_workspace_step():
    require_gpu()
    import torch
    import medusa_tree_verification_forward_amd as M
    from medusa_tree_verification_forward_amd.step import VerifyStep
    cases = [WORKLOADS["vicuna7b_typical"],
             scaled(WORKLOADS["vicuna7b_typical"], d=512, H=4, V=3001, L=300,
                    L_range=(300, 300)),
             WORKLOADS["tiny_fp32"]]
    sizes = []
    for w in cases:
        inp = parity.inputs_for(w)
        kw = dict(H=w.H, Dh=w.Dh, s_max=w.s_max, mode=w.mode, tau=w.tau, eps=w.eps,
                  delta=w.delta, theta=w.rope_theta)
        ref = VerifyStep(inp, **kw)
        ref.run_step(keep_kv_len=True)
        got = VerifyStep(inp, **kw)
        M.step_static(got.shape, got.step_args(keep_kv_len=True))
        torch.cuda.synchronize()
        a, b = _outputs(ref), _outputs(got)
        assert set(a) == set(b)
        for k in sorted(a):
            assert np.array_equal(a[k], b[k], equal_nan=True), (w.name, k)
        sizes.append(M.workspace_bytes(got.shape))
        del ref, got
        torch.cuda.empty_cache()
    assert sizes[0] > sizes[1] > sizes[2]
    assert sizes[0] <= M.STATIC_WORKSPACE_BYTES
