"""Seeded synthetic inputs for the FLCE workloads.

This module only draws random numbers and rounds them to the storage dtype;
it holds none of the loss arithmetic, so that the CPU oracle and the HIP path
can both be fed from it without sharing any of the method.

The workloads stand in for the language-model heads the Liger-Kernel pages
benchmark (LLaMA 3-8B, Qwen2, Gemma, Mistral: "[論文レビュー] Liger Kernel:
Efficient Triton Kernels for LLM Training", 主な発見; "Liger-Kernel 項目詳細介紹",
支持的模型 and 性能基準測試).  No dataset or trained weight is used: hidden
states are N(0, 1) (times a scale), weights N(0, 0.02^2), targets uniform or
Zipf(1.1) over vocabulary ids, with a share of positions set to the ignore
index.  Draw order per workload: X, W, targets, ignore positions, all from one
``torch.Generator`` seeded with the workload's seed, in float32, then rounded
to bfloat16 (round-to-nearest-even) where the workload is bf16.
"""

from __future__ import annotations

import dataclasses
import hashlib
import math

import numpy as np
import torch

IGNORE_INDEX = -100


@dataclasses.dataclass
class Workload:
    name: str
    BT: int
    H: int
    V: int
    dtype: str  # "fp32" or "bf16"
    seed: int
    x_scale: float = 1.0
    w_std: float = 0.02
    targets: str = "uniform"  # "uniform" | "zipf1.1"
    ignore: tuple = ("random_frac", 0.05)  # ("index", i) | ("random_frac", f) | ("tail_frac", f) | ("none",) | ("all",)
    chunk_tokens: int = 0  # 0 = library's automatic choice
    ignore_index: int = IGNORE_INDEX

    @property
    def torch_dtype(self):
        return {"fp32": torch.float32, "bf16": torch.bfloat16}[self.dtype]


# The five workloads: a tiny fp32 case, then four bf16 heads shaped like the
# pages' model families (Mistral/Llama-2, Llama-3-8B, Qwen2-7B at 16K context,
# Gemma's 256K vocabulary).
WORKLOADS = {
    "tiny": Workload("tiny", 8, 128, 256, "fp32", 0, ignore=("index", 3), chunk_tokens=8),
    "mistral": Workload("mistral", 2048, 2048, 32000, "bf16", 1, chunk_tokens=1024),
    "llama3": Workload("llama3", 8192, 4096, 128256, "bf16", 2, targets="zipf1.1"),
    "qwen2": Workload("qwen2", 16384, 3584, 152064, "bf16", 3, ignore=("tail_frac", 0.10)),
    "gemma": Workload("gemma", 8192, 3072, 256000, "bf16", 4, x_scale=3.0),
}


def workload(name: str, **overrides) -> Workload:
    return dataclasses.replace(WORKLOADS[name], **overrides)


def _zipf_targets(g: torch.Generator, BT: int, V: int, s: float = 1.1) -> torch.Tensor:
    # id r in [0, V) drawn with probability proportional to (r + 1)^-s, by inverse CDF
    ranks = torch.arange(1, V + 1, dtype=torch.float64)
    cdf = torch.cumsum(ranks.pow(-s), 0)
    cdf = cdf / cdf[-1]
    u = torch.rand(BT, generator=g, dtype=torch.float64)
    return torch.searchsorted(cdf, u, right=True).clamp_(max=V - 1).to(torch.int64)


def make_inputs(w: Workload):
    """Return (X [BT,H], W [V,H], y [BT] int64) as CPU tensors of the workload's dtype."""
    g = torch.Generator().manual_seed(w.seed)
    X = torch.randn(w.BT, w.H, generator=g, dtype=torch.float32)
    if w.x_scale != 1.0:
        X.mul_(w.x_scale)
    X = X.to(w.torch_dtype)
    W = torch.randn(w.V, w.H, generator=g, dtype=torch.float32).mul_(w.w_std).to(w.torch_dtype)
    if w.targets == "uniform":
        y = torch.randint(0, w.V, (w.BT,), generator=g, dtype=torch.int64)
    elif w.targets == "zipf1.1":
        y = _zipf_targets(g, w.BT, w.V, 1.1)
    else:
        raise ValueError(w.targets)
    kind = w.ignore[0]
    if kind == "index":
        if w.ignore[1] < w.BT:
            y[w.ignore[1]] = w.ignore_index
    elif kind == "random_frac":
        n = int(round(w.ignore[1] * w.BT))
        y[torch.randperm(w.BT, generator=g)[:n]] = w.ignore_index
    elif kind == "tail_frac":
        n = int(math.floor(w.ignore[1] * w.BT))
        if n:
            y[w.BT - n:] = w.ignore_index
    elif kind == "all":
        y[:] = w.ignore_index
    elif kind != "none":
        raise ValueError(kind)
    return X, W, y


def small(BT: int, H: int, V: int, dtype: str = "bf16", seed: int = 0, **kw) -> Workload:
    """An ad-hoc workload for tests (ragged shapes, edge cases)."""
    return Workload(f"small_{BT}x{H}x{V}_{dtype}_{seed}", BT, H, V, dtype, seed, **kw)


def fingerprint(*tensors) -> str:
    """Short hash of a strided sample of each tensor's bytes (checks reproducibility)."""
    h = hashlib.sha256()
    for t in tensors:
        a = t.detach().cpu()
        if a.dtype == torch.bfloat16:
            a = a.view(torch.int16)
        a = a.reshape(-1)
        n = a.numel()
        step = max(1, n // 65536)
        h.update(np.ascontiguousarray(a[::step].numpy()).tobytes())
        h.update(np.ascontiguousarray(a[-4096:].numpy()).tobytes())
        h.update(str((tuple(t.shape), str(t.dtype))).encode())
    return h.hexdigest()[:16]
