"""Decode-time quantized-expert MoE block for AMD Instinct MI355X (gfx950).

Python face of the C ABI in ``include/moe_decode.h``; the kernels are
hand-written HIP in ``csrc/``.  Importing the package does not load the
library; the first call does, and raises if it has not been built.
"""

from ._lib import (  # noqa: F401
    EXPORTS,
    MOE_ACT_GEGLU,
    MOE_ACT_SWIGLU,
    MOE_DOWN_COLS,
    MOE_DOWN_ROWS,
    MOE_DTYPE_BF16,
    MOE_DTYPE_F32,
    MOE_ERR_DEVICE,
    MOE_ERR_INVALID_ARG,
    MOE_ERR_UNSUPPORTED,
    MOE_ERR_WORKSPACE,
    MOE_OK,
    MOE_STATIC_SCRATCH_BYTES,
    DeviceLayer,
    LayerStruct,
    MoeError,
    Plan,
    PlanStruct,
    alloc_workspace,
    decode_layer,
    decode_layer_static,
    decode_step,
    expert_down_combine,
    expert_gate_up,
    route_gate_up,
    expert_plan,
    lib,
    library_path,
    route_plan,
    route_topk,
    router_logits,
    status_str,
    workspace_size,
)
