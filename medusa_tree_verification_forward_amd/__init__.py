"""MI355X-native Medusa verify step: Python binding of the gfx950 HIP library.

The library (``libmedusa_mi355x.so``, built from ``csrc/``) does all the
work; this package marshals arguments (``_lib``) and allocates the device
buffers of one step (``step``). Importing it without the built library raises.
"""

from ._lib import (  # noqa: F401
    BF16, DRAFT_SAMPLE, DRAFT_TOPK, EXACT, F32, GREEDY, LIB_PATH, MODES, PACK_PLAIN, PACK_QKV,
    STATIC_WORKSPACE_BYTES, TYPICAL, MedusaError,
    Shape, StepArgs, build_tree, commit, evaluate_posterior, exported_symbols, heads_forward, last_error,
    make_shape, pack_weight, packed_copy, packed_heads_w1, packed_heads_w2, packed_weight_bytes,
    step, step_static, step_timed, tree_attention, verify_forward, version, workspace_bytes)
