"""MI355X (gfx950) fused linear + cross-entropy: HIP kernels behind a C ABI.

Public API (all GPU-only; the HIP library must be built):
    flce_fwd_bwd(X, W, targets, ignore_index=-100, chunk_tokens=0, token_scale=None) -> loss, dX, dW
    flce_forward(X, W, targets, ignore_index=-100) -> loss   (forward only)
    flce_orpo(X, W, targets, beta=0.1) -> loss, dX, dW                (fused-linear ORPO)
    ce_fwd_bwd_inplace(logits, targets, ignore_index=-100) -> loss
    ce_fwd_bwd_inplace_noalloc(logits, targets, ...) -> loss   (no allocation; static scratch)
    FusedLinearCrossEntropyLoss(ignore_index=-100, reduction="mean"|"none")(weight, input, target) -> loss
"""
from .binding import (  # noqa: F401
    FlceError,
    FusedLinearCrossEntropyLoss,
    FusedLinearORPOLoss,
    KernelTimer,
    ce_fwd_bwd_inplace,
    ce_fwd_bwd_inplace_noalloc,
    ce_noalloc_max_rows,
    ce_workspace_bytes,
    flce_chunk_tokens,
    flce_forward,
    flce_fwd_bwd,
    flce_fwd_workspace_bytes,
    flce_orpo,
    flce_orpo_workspace_bytes,
    flce_workspace_bytes,
    header_functions,
    load_library,
)
