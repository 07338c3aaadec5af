"""Single-GPU Mixture-of-Experts layer for AMD Instinct MI355X (gfx950).

The layer (top-k routing, schedule, dispatch, expert-grouped SwiGLU FFN,
weighted combine, and the backward) runs in hand-written HIP kernels behind the
C ABI declared in ``include/moe.h``; this package is the thin Python binding.
"""
from .binding import (Config, MoEError, PREC_BF16, PREC_MXFP8, alloc_grads, alloc_saved,
                      alloc_schedule, alloc_weights_mx, alloc_workspace, device_supported, lib,
                      moe_backward, moe_check_device_error, moe_forward,
                      moe_quantize_weights_mxfp8, moe_schedule, ring_rows, status_string,
                      validate_config, workspace_size)

__all__ = ["Config", "MoEError", "PREC_BF16", "PREC_MXFP8", "alloc_grads", "alloc_saved",
           "alloc_schedule", "alloc_weights_mx", "alloc_workspace", "device_supported", "lib", "moe_backward",
           "moe_check_device_error", "moe_forward", "moe_quantize_weights_mxfp8", "moe_schedule", "ring_rows", "status_string",
           "validate_config", "workspace_size"]
