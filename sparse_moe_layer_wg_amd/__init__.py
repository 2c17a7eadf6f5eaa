"""MI355X (gfx950) GShard mixture-of-experts layer forward.

A thin ctypes binding over the C ABI in ``include/moe.h`` (``libmoe.so``):
argument marshalling only.  Every step of the layer runs in the library's
HIP kernels; PyTorch provides device memory and the stream.  Loading fails
loudly when ``libmoe.so`` has not been built: there is no fallback.
"""
from ._lib import (  # noqa: F401
    MOE_BF16,
    MOE_CFG_DROPLESS,
    MOE_CFG_REROUTE,
    MOE_F32,
    MOE_GATE_LOGITS_IN,
    MOE_NUM_BWD_EVENTS,
    MOE_NUM_STAGE_EVENTS,
    MOE_STATIC_SCRATCH_BYTES,
    MoeConfig,
    MoeError,
    backward_workspace_bytes,
    capacity,
    combine,
    config,
    dispatch,
    dispatch_rows,
    expert_ffn,
    gate,
    gate_noalloc,
    layer_backward,
    layer_forward,
    library,
    library_path,
    workspace_bytes,
)
