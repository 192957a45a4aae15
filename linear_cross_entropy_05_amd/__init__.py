"""MI355X (gfx950) fused linear + cross-entropy: HIP kernels behind a C ABI.

Public API (all GPU-only; the HIP library must be built):
    flce_fwd_bwd(X, W, targets, ignore_index=-100, chunk_tokens=0, token_scale=None) -> loss, dX, dW
    flce_forward(X, W, targets, ignore_index=-100) -> loss   (forward only)
    ce_fwd_bwd_inplace(logits, targets, ignore_index=-100) -> loss
    FusedLinearCrossEntropyLoss(ignore_index=-100, reduction="mean"|"none")(weight, input, target) -> loss
"""
from .binding import (  # noqa: F401
    FlceError,
    FusedLinearCrossEntropyLoss,
    KernelTimer,
    ce_fwd_bwd_inplace,
    ce_workspace_bytes,
    flce_chunk_tokens,
    flce_forward,
    flce_fwd_bwd,
    flce_fwd_workspace_bytes,
    flce_workspace_bytes,
    header_functions,
    load_library,
)
