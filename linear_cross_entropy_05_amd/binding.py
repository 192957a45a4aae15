"""Python binding of libflce (ctypes): argument marshalling only.

Every step of the loss runs in the HIP kernels behind ``include/flce.h``;
this module checks tensors, allocates outputs and the workspace through
PyTorch's caching allocator, and passes raw device pointers and the current
HIP stream.  There is no CPU or PyTorch fallback: if the library is missing
or the device is not a gfx950, the call raises.

The module form follows the low-level usage shown on "Liger-Kernel 項目詳細介紹"
(使用方法, item 3): ``loss_fn(weight, input, target)`` with the weight first,
then ``loss.backward()``.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libflce.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "flce.h")

FLCE_F32, FLCE_BF16 = 0, 1
STATUS = {
    0: "FLCE_OK",
    1: "FLCE_ERR_ARG",
    2: "FLCE_ERR_DTYPE",
    3: "FLCE_ERR_WORKSPACE",
    4: "FLCE_ERR_DEVICE",
    5: "FLCE_ERR_LAUNCH",
    6: "FLCE_ERR_TARGET",
    7: "FLCE_ERR_SHAPE",
    8: "FLCE_ERR_ALIGN",
    9: "FLCE_ERR_SCRATCH",
}
_DTYPES = {torch.float32: FLCE_F32, torch.bfloat16: FLCE_BF16}

_lib = None


class FlceError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = _lib.flce_status_str(status).decode() if _lib is not None else STATUS.get(status, "?")
        super().__init__(f"{what}: {STATUS.get(status, status)} ({msg})" if what else msg)


def _declare(lib):
    c = ctypes
    i64, vp, sz = c.c_int64, c.c_void_p, c.c_size_t
    lib.flce_chunk_tokens.argtypes = [i64, i64, i64, i64, c.c_int]
    lib.flce_chunk_tokens.restype = i64
    lib.flce_workspace_bytes.argtypes = [i64, i64, i64, i64, c.c_int]
    lib.flce_workspace_bytes.restype = sz
    lib.flce_fwd_bwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, c.c_int, vp, vp, vp, vp, vp, sz, vp, vp]
    lib.flce_fwd_bwd.restype = c.c_int
    lib.flce_fwd_workspace_bytes.argtypes = [i64, i64, i64, i64, c.c_int]
    lib.flce_fwd_workspace_bytes.restype = sz
    lib.flce_fwd.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, c.c_int, vp, vp, vp, sz, vp, vp]
    lib.flce_fwd.restype = c.c_int
    lib.flce_orpo_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, c.c_int]
    lib.flce_orpo_workspace_bytes.restype = sz
    lib.flce_orpo.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, c.c_float, i64, c.c_int, vp, vp, vp, vp, vp, sz,
                              vp, vp]
    lib.flce_orpo.restype = c.c_int
    lib.ce_workspace_bytes.argtypes = [i64, i64]
    lib.ce_workspace_bytes.restype = sz
    lib.ce_fwd_bwd_inplace.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, sz, vp, vp]
    lib.ce_fwd_bwd_inplace.restype = c.c_int
    lib.ce_noalloc_max_rows.argtypes = []
    lib.ce_noalloc_max_rows.restype = i64
    lib.ce_fwd_bwd_inplace_noalloc.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp]
    lib.ce_fwd_bwd_inplace_noalloc.restype = c.c_int
    lib.flce_status_str.argtypes = [c.c_int]
    lib.flce_status_str.restype = c.c_char_p
    lib.flce_device_supported.argtypes = [c.c_int]
    lib.flce_device_supported.restype = c.c_int
    lib.flce_profile_begin.argtypes = [c.c_int]
    lib.flce_profile_begin.restype = c.c_int
    lib.flce_profile_end.argtypes = [c.POINTER(c.c_double), c.POINTER(c.c_int64), c.c_int]
    lib.flce_profile_end.restype = c.c_int
    return lib


def load_library(path: str = LIB_PATH):
    """Load libflce.so (once).  torch is imported first so the library binds to
    the HIP runtime torch already loaded (same soname)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise ImportError(
                f"{path} is not built; run `python -m linear_cross_entropy_05_amd.build` (needs hipcc for gfx950)"
            )
        _lib = _declare(ctypes.CDLL(path))
    return _lib


def header_functions(header: str = HEADER) -> list[str]:
    """Names of the functions include/flce.h declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else ctypes.c_void_p(0)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_tensor(name, t, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")


def _same_device(dev, **tensors):
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev} (all operands on one device)")


def _check_out(name, t, shape, dtype, dev):
    """A caller-supplied output: the kernels write exactly `shape` elements of `dtype` there."""
    _check_tensor(name, t, dtype=dtype)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    _same_device(dev, **{name: t})


def _workspace(workspace, need: int, dev):
    """The caller's workspace (checked) or a new one of `need` bytes; returns (tensor, bytes)."""
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    else:
        _check_tensor("workspace", workspace)
        _same_device(dev, workspace=workspace)
    return workspace, workspace.numel() * workspace.element_size()


def flce_chunk_tokens(BT: int, H: int, V: int, chunk_tokens: int = 0, dtype=torch.bfloat16) -> int:
    return int(load_library().flce_chunk_tokens(BT, H, V, chunk_tokens, _DTYPES[dtype]))


def flce_workspace_bytes(BT: int, H: int, V: int, chunk_tokens: int = 0, dtype=torch.bfloat16) -> int:
    return int(load_library().flce_workspace_bytes(BT, H, V, chunk_tokens, _DTYPES[dtype]))


def ce_workspace_bytes(BT: int, V: int) -> int:
    return int(load_library().ce_workspace_bytes(BT, V))


def check_err_flag(err: torch.Tensor, what: str):
    v = int(err.item())
    if v != 0:
        raise FlceError(v, what)


def flce_fwd_bwd(X, W, targets, ignore_index: int = -100, chunk_tokens: int = 0, *, token_scale=None,
                 row_loss: bool = False, check: bool = True, out=None, workspace=None):
    """Fused linear + cross-entropy forward and backward.

    X [BT, H] and W [V, H] (fp32 or bf16, same dtype), targets [BT] int64.
    Returns (loss fp32 0-d, dX [BT, H] X.dtype, dW [V, H] fp32) and, with
    ``row_loss=True``, the per-token losses [BT] fp32.  ``token_scale``
    (fp32 [BT], optional) makes the gradients those of
    sum_i token_scale[i] * loss_i instead of the mean; the returned loss is
    the mean either way.  With ``check`` the call synchronises and raises if
    a target was out of range.  ``out`` may pass preallocated (loss, dX, dW,
    err) tensors and ``workspace`` a uint8 device tensor, to keep
    allocations out of timed loops.
    """
    lib = load_library()
    _check_tensor("X", X, ndim=2)
    _check_tensor("W", W, dtype=X.dtype, ndim=2)
    _check_tensor("targets", targets, dtype=torch.int64, ndim=1)
    if token_scale is not None:
        _check_tensor("token_scale", token_scale, dtype=torch.float32, ndim=1)
        if token_scale.shape[0] != X.shape[0]:
            raise ValueError("token_scale length must equal the number of tokens")
    if X.dtype not in _DTYPES:
        raise TypeError(f"dtype {X.dtype} not supported (float32, bfloat16)")
    BT, H = X.shape
    V = W.shape[0]
    if W.shape[1] != H or targets.shape[0] != BT:
        raise ValueError(f"shape mismatch X{tuple(X.shape)} W{tuple(W.shape)} targets{tuple(targets.shape)}")
    dev = X.device
    _same_device(dev, W=W, targets=targets, token_scale=token_scale)
    if out is None:
        loss = torch.empty((), dtype=torch.float32, device=dev)
        dX = torch.empty_like(X)
        dW = torch.empty((V, H), dtype=torch.float32, device=dev)
        err = torch.empty((1,), dtype=torch.int32, device=dev)
    else:
        loss, dX, dW, err = out
        _check_out("out loss", loss, (), torch.float32, dev)
        _check_out("out dX", dX, (BT, H), X.dtype, dev)
        _check_out("out dW", dW, (V, H), torch.float32, dev)
        _check_out("out err", err, (1,), torch.int32, dev)
    rl = torch.empty((BT,), dtype=torch.float32, device=dev) if row_loss else None
    need = lib.flce_workspace_bytes(BT, H, V, chunk_tokens, _DTYPES[X.dtype])
    workspace, ws_bytes = _workspace(workspace, need, dev)
    with torch.cuda.device(dev):
        st = lib.flce_fwd_bwd(
            _ptr(X), _ptr(W), _ptr(targets), _ptr(token_scale), BT, H, V, ignore_index, chunk_tokens,
            _DTYPES[X.dtype], _ptr(loss), _ptr(rl), _ptr(dX), _ptr(dW), _ptr(workspace), ws_bytes, _ptr(err),
            _stream(dev))
    if st != 0:
        raise FlceError(st, "flce_fwd_bwd")
    if check:
        check_err_flag(err, "flce_fwd_bwd")
    return (loss, dX, dW, rl) if row_loss else (loss, dX, dW)


def flce_fwd_workspace_bytes(BT: int, H: int, V: int, chunk_tokens: int = 0, dtype=torch.bfloat16) -> int:
    return int(load_library().flce_fwd_workspace_bytes(BT, H, V, chunk_tokens, _DTYPES[dtype]))


def flce_forward(X, W, targets, ignore_index: int = -100, chunk_tokens: int = 0, *, row_loss: bool = False,
                 check: bool = True, out=None, workspace=None):
    """Fused linear + cross-entropy, forward only: the loss (fp32 0-d) and,
    with ``row_loss=True``, the per-token losses, without gradients and
    without storing logits.  Arguments as for :func:`flce_fwd_bwd`; ``out``
    may pass preallocated (loss, err) tensors."""
    lib = load_library()
    _check_tensor("X", X, ndim=2)
    _check_tensor("W", W, dtype=X.dtype, ndim=2)
    _check_tensor("targets", targets, dtype=torch.int64, ndim=1)
    if X.dtype not in _DTYPES:
        raise TypeError(f"dtype {X.dtype} not supported (float32, bfloat16)")
    BT, H = X.shape
    V = W.shape[0]
    if W.shape[1] != H or targets.shape[0] != BT:
        raise ValueError(f"shape mismatch X{tuple(X.shape)} W{tuple(W.shape)} targets{tuple(targets.shape)}")
    dev = X.device
    _same_device(dev, W=W, targets=targets)
    if out is None:
        loss = torch.empty((), dtype=torch.float32, device=dev)
        err = torch.empty((1,), dtype=torch.int32, device=dev)
    else:
        loss, err = out
        _check_out("out loss", loss, (), torch.float32, dev)
        _check_out("out err", err, (1,), torch.int32, dev)
    rl = torch.empty((BT,), dtype=torch.float32, device=dev) if row_loss else None
    need = lib.flce_fwd_workspace_bytes(BT, H, V, chunk_tokens, _DTYPES[X.dtype])
    workspace, ws_bytes = _workspace(workspace, need, dev)
    with torch.cuda.device(dev):
        st = lib.flce_fwd(_ptr(X), _ptr(W), _ptr(targets), BT, H, V, ignore_index, chunk_tokens, _DTYPES[X.dtype],
                          _ptr(loss), _ptr(rl), _ptr(workspace), ws_bytes, _ptr(err), _stream(dev))
    if st != 0:
        raise FlceError(st, "flce_fwd")
    if check:
        check_err_flag(err, "flce_fwd")
    return (loss, rl) if row_loss else loss


def flce_orpo_workspace_bytes(n_seq: int, seq_len: int, H: int, V: int, chunk_tokens: int = 0,
                              dtype=torch.bfloat16) -> int:
    return int(load_library().flce_orpo_workspace_bytes(n_seq, seq_len, H, V, chunk_tokens, _DTYPES[dtype]))


def flce_orpo(X, W, targets, beta: float = 0.1, ignore_index: int = -100, chunk_tokens: int = 0, *,
              seq_logp: bool = False, check: bool = True):
    """Fused-linear ORPO loss: X [2B, T, H] (or [2B*T, H] with targets
    [2B, T]), chosen sequences first, W [V, H], targets [2B, T] int64.
    Returns (loss fp32 0-d, dX shaped like X, dW [V, H] fp32) and, with
    ``seq_logp=True``, the mean log-probability of each sequence [2B]."""
    lib = load_library()
    _check_tensor("W", W, ndim=2)
    _check_tensor("targets", targets, dtype=torch.int64, ndim=2)
    _check_tensor("X", X, dtype=W.dtype)
    if X.dtype not in _DTYPES:
        raise TypeError(f"dtype {X.dtype} not supported (float32, bfloat16)")
    n_seq, T = targets.shape
    V, H = W.shape
    if X.numel() != n_seq * T * H or X.shape[-1] != H:
        raise ValueError(f"X{tuple(X.shape)} does not match targets{tuple(targets.shape)} and H={H}")
    dev = X.device
    _same_device(dev, W=W, targets=targets)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    dX = torch.empty_like(X)
    dW = torch.empty((V, H), dtype=torch.float32, device=dev)
    err = torch.empty((1,), dtype=torch.int32, device=dev)
    sl = torch.empty((n_seq,), dtype=torch.float32, device=dev) if seq_logp else None
    ws = torch.empty((lib.flce_orpo_workspace_bytes(n_seq, T, H, V, chunk_tokens, _DTYPES[X.dtype]),),
                     dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        st = lib.flce_orpo(_ptr(X), _ptr(W), _ptr(targets), n_seq, T, H, V, ignore_index, float(beta), chunk_tokens,
                           _DTYPES[X.dtype], _ptr(loss), _ptr(sl), _ptr(dX), _ptr(dW), _ptr(ws), ws.numel(), _ptr(err),
                           _stream(dev))
    if st != 0:
        raise FlceError(st, "flce_orpo")
    if check:
        check_err_flag(err, "flce_orpo")
    return (loss, dX, dW, sl) if seq_logp else (loss, dX, dW)


def ce_fwd_bwd_inplace(logits, targets, ignore_index: int = -100, *, row_loss: bool = False, check: bool = True):
    """Cross-entropy on fp32 logits [BT, V]; overwrites logits with d loss / d logits.

    Returns the fp32 loss (0-d) and, with ``row_loss=True``, per-token losses."""
    lib = load_library()
    _check_tensor("logits", logits, dtype=torch.float32, ndim=2)
    _check_tensor("targets", targets, dtype=torch.int64, ndim=1)
    BT, V = logits.shape
    if targets.shape[0] != BT:
        raise ValueError("targets length must equal logits rows")
    dev = logits.device
    _same_device(dev, targets=targets)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    err = torch.empty((1,), dtype=torch.int32, device=dev)
    rl = torch.empty((BT,), dtype=torch.float32, device=dev) if row_loss else None
    ws = torch.empty((lib.ce_workspace_bytes(BT, V),), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        st = lib.ce_fwd_bwd_inplace(_ptr(logits), _ptr(targets), BT, V, ignore_index, _ptr(loss), _ptr(rl), _ptr(ws),
                                    ws.numel(), _ptr(err), _stream(dev))
    if st != 0:
        raise FlceError(st, "ce_fwd_bwd_inplace")
    if check:
        check_err_flag(err, "ce_fwd_bwd_inplace")
    return (loss, rl) if row_loss else loss


def ce_fwd_bwd_inplace_noalloc(logits, targets, ignore_index: int = -100, *, out=None, row_loss=None,
                               check: bool = True):
    """ce_fwd_bwd_inplace through the entry point that allocates nothing
    (its scratch is a static device array; at most ce_noalloc_max_rows()
    rows).  ``out`` may pass preallocated (loss fp32 0-d, err int32 [1])
    tensors and ``row_loss`` an fp32 [BT] tensor to fill; with both given,
    this wrapper allocates nothing either.  Calls that overlap on one GPU
    share its scratch and must be serialised.  Returns the loss tensor."""
    lib = load_library()
    _check_tensor("logits", logits, dtype=torch.float32, ndim=2)
    _check_tensor("targets", targets, dtype=torch.int64, ndim=1)
    BT, V = logits.shape
    if targets.shape[0] != BT:
        raise ValueError("targets length must equal logits rows")
    dev = logits.device
    _same_device(dev, targets=targets)
    if out is None:
        loss = torch.empty((), dtype=torch.float32, device=dev)
        err = torch.empty((1,), dtype=torch.int32, device=dev)
    else:
        loss, err = out
        _check_out("out loss", loss, (), torch.float32, dev)
        _check_out("out err", err, (1,), torch.int32, dev)
    if row_loss is not None:
        _check_out("row_loss", row_loss, (BT,), torch.float32, dev)
    with torch.cuda.device(dev):
        st = lib.ce_fwd_bwd_inplace_noalloc(_ptr(logits), _ptr(targets), BT, V, ignore_index, _ptr(loss),
                                            _ptr(row_loss), _ptr(err), _stream(dev))
    if st != 0:
        raise FlceError(st, "ce_fwd_bwd_inplace_noalloc")
    if check:
        check_err_flag(err, "ce_fwd_bwd_inplace_noalloc")
    return loss


def ce_noalloc_max_rows() -> int:
    return int(load_library().ce_noalloc_max_rows())


KERNEL_KINDS = ["count_valid", "logits", "lse", "grad_inplace", "dx_dw", "dx_reduce", "loss_final",
                "ce_rows", "fill_zero", "orpo_stats", "gather"]


class KernelTimer:
    """Per-kernel HIP-event timing of every library launch inside the block.

        with KernelTimer() as kt:
            ...calls...
        kt.ms["logits"], kt.launches["logits"]
    """

    def __init__(self, max_launches: int = 65536):
        self.max_launches = max_launches
        self.ms = {}
        self.launches = {}

    def __enter__(self):
        st = load_library().flce_profile_begin(self.max_launches)
        if st != 0:
            raise FlceError(st, "flce_profile_begin")
        return self

    def __exit__(self, *exc):
        n = len(KERNEL_KINDS)
        ms = (ctypes.c_double * n)()
        cnt = (ctypes.c_int64 * n)()
        st = load_library().flce_profile_end(ms, cnt, n)
        self.ms = {k: ms[i] for i, k in enumerate(KERNEL_KINDS)}
        self.launches = {k: cnt[i] for i, k in enumerate(KERNEL_KINDS)}
        if st != 0 and exc[0] is None:
            raise FlceError(st, "flce_profile_end")
        return False


class _FLCEFunction(torch.autograd.Function):
    """Mean reduction.  Forward computes the loss and both gradients at once
    (one pass over the chunks); backward hands them on, scaled by the
    upstream gradient unless that is exactly 1."""

    @staticmethod
    def forward(ctx, weight, inp, target, ignore_index, chunk_tokens):
        loss, dX, dW = flce_fwd_bwd(inp.contiguous(), weight.contiguous(), target.contiguous(), ignore_index,
                                    chunk_tokens)
        ctx.save_for_backward(dX, dW)
        ctx.weight_dtype = weight.dtype
        return loss

    @staticmethod
    def backward(ctx, grad):
        dX, dW = ctx.saved_tensors
        if bool(torch.equal(grad, torch.ones_like(grad))):
            gx = dX if ctx.needs_input_grad[1] else None
            gw = dW.to(ctx.weight_dtype) if ctx.needs_input_grad[0] else None
            return gw, gx, None, None, None
        g = grad.to(torch.float32)
        gx = (dX.float() * g).to(dX.dtype) if ctx.needs_input_grad[1] else None
        gw = (dW * g).to(ctx.weight_dtype) if ctx.needs_input_grad[0] else None
        return gw, gx, None, None, None


class _FLCETokenFunction(torch.autograd.Function):
    """No reduction: forward returns the per-token losses (forward-only path,
    no logits kept); backward runs the fused pass with the upstream per-token
    gradients as the token scales."""

    @staticmethod
    def forward(ctx, weight, inp, target, ignore_index, chunk_tokens):
        weight, inp, target = weight.contiguous(), inp.contiguous(), target.contiguous()
        _, rl = flce_forward(inp, weight, target, ignore_index, chunk_tokens, row_loss=True)
        ctx.save_for_backward(weight, inp, target)
        ctx.ignore_index, ctx.chunk_tokens = ignore_index, chunk_tokens
        return rl

    @staticmethod
    def backward(ctx, grad_rows):
        weight, inp, target = ctx.saved_tensors
        scale = grad_rows.to(torch.float32).contiguous()
        _, dX, dW = flce_fwd_bwd(inp, weight, target, ctx.ignore_index, ctx.chunk_tokens, token_scale=scale)
        gx = dX if ctx.needs_input_grad[1] else None
        gw = dW.to(weight.dtype) if ctx.needs_input_grad[0] else None
        return gw, gx, None, None, None


class _ORPOFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, weight, x, target, beta, ignore_index, chunk_tokens):
        loss, dX, dW = flce_orpo(x.contiguous(), weight.contiguous(), target.contiguous(), beta, ignore_index,
                                 chunk_tokens)
        ctx.save_for_backward(dX, dW)
        ctx.weight_dtype = weight.dtype
        return loss

    @staticmethod
    def backward(ctx, grad):
        dX, dW = ctx.saved_tensors
        if bool(torch.equal(grad, torch.ones_like(grad))):
            gx = dX if ctx.needs_input_grad[1] else None
            gw = dW.to(ctx.weight_dtype) if ctx.needs_input_grad[0] else None
        else:
            g = grad.to(torch.float32)
            gx = (dX.float() * g).to(dX.dtype) if ctx.needs_input_grad[1] else None
            gw = (dW * g).to(ctx.weight_dtype) if ctx.needs_input_grad[0] else None
        return gw, gx, None, None, None, None


class FusedLinearORPOLoss(torch.nn.Module):
    """``loss = FusedLinearORPOLoss()(lm_head.weight, x, target)`` (the call
    shape of "Liger-Kernel 項目詳細介紹", 使用方法 item 4): x [2B, T, H] hidden
    states with the B chosen responses first, target [2B, T]; odds-ratio
    preference loss with weight ``beta`` plus the chosen-token cross-entropy."""

    def __init__(self, ignore_index: int = -100, beta: float = 0.1, chunk_tokens: int = 0):
        super().__init__()
        self.ignore_index = ignore_index
        self.beta = beta
        self.chunk_tokens = chunk_tokens

    def forward(self, weight, x, target):
        return _ORPOFunction.apply(weight, x, target, self.beta, self.ignore_index, self.chunk_tokens)


class FusedLinearCrossEntropyLoss(torch.nn.Module):
    """``loss = FusedLinearCrossEntropyLoss()(weight, input, target)``:
    cross-entropy of ``input @ weight.T`` over targets != ignore_index, as
    the mean (``reduction="mean"``) or per token (``reduction="none"``, 0 on
    ignored tokens)."""

    def __init__(self, ignore_index: int = -100, chunk_tokens: int = 0, reduction: str = "mean"):
        super().__init__()
        if reduction not in ("mean", "none"):
            raise ValueError(f"reduction must be 'mean' or 'none', got {reduction!r}")
        self.ignore_index = ignore_index
        self.chunk_tokens = chunk_tokens
        self.reduction = reduction

    def forward(self, weight, inp, target):
        grad = torch.is_grad_enabled() and (weight.requires_grad or inp.requires_grad)
        if self.reduction == "none":
            if grad:
                return _FLCETokenFunction.apply(weight, inp, target, self.ignore_index, self.chunk_tokens)
            return flce_forward(inp.contiguous(), weight.contiguous(), target.contiguous(), self.ignore_index,
                                self.chunk_tokens, row_loss=True)[1]
        if grad:
            return _FLCEFunction.apply(weight, inp, target, self.ignore_index, self.chunk_tokens)
        # no gradient wanted: the forward-only path (no logits chunk, a third of the work)
        return flce_forward(inp.contiguous(), weight.contiguous(), target.contiguous(), self.ignore_index,
                            self.chunk_tokens)
