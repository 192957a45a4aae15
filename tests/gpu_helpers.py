"""Shared helpers for the GPU parity tests (HIP path vs the float64 oracle)."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import synth_inputs as si

# Tolerances: fp32 inputs -> 1e-5 relative loss error and 1e-5 max-abs
# gradient error over the reference's max-abs; bf16 inputs with fp32
# accumulation -> 2e-3 and 2e-2.
TOL = {"fp32": (1e-5, 1e-5), "bf16": (2e-3, 2e-2)}


def ensure_built():
    from linear_cross_entropy_05_amd import binding

    if not os.path.exists(binding.LIB_PATH):
        from linear_cross_entropy_05_amd import build

        build.build()
    return binding.load_library()


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size == 0:
        return 0.0
    den = float(np.max(np.abs(b)))
    num = float(np.max(np.abs(a - b)))
    return num / den if den > 0 else num


def to_np(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_gpu(w: si.Workload, chunk_tokens=None, inputs=None):
    """Run flce_fwd_bwd on a workload; returns (inputs on CPU, outputs on CPU)."""
    import linear_cross_entropy_05_amd as flce

    X, W, y = inputs if inputs is not None else si.make_inputs(w)
    dev = torch.device("cuda", 0)
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    C = w.chunk_tokens if chunk_tokens is None else chunk_tokens
    say(f"[gpu] flce_fwd_bwd {w.name} BT={w.BT} H={w.H} V={w.V} {w.dtype} chunk={C}")
    loss, dX, dW, rl = flce.flce_fwd_bwd(Xd, Wd, yd, w.ignore_index, C, row_loss=True)
    torch.cuda.synchronize()
    out = {"loss": float(loss.item()), "dX": dX.cpu(), "dW": dW.cpu(), "row_loss": rl.cpu()}
    return (X, W, y), out
