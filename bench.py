"""Benchmark: fused linear + cross-entropy forward+backward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config llama3] [--no-cpu-baseline]

One step = one flce_fwd_bwd call over the whole batch of the workload (all
token chunks: logits GEMM with the softmax-statistics epilogue, log-sum-exp,
in-place gradient, dX and dW GEMMs, final mean).  Inputs are seeded synthetic
tensors already resident in HBM when the timed region starts.  Prints one JSON
line on stdout (progress goes to stderr).

The default workload is the Llama-3-8B-shaped head: BT=8192 tokens (batch 8 x
sequence 1024), H=4096, V=128256, bf16 inputs, fp32 accumulation, Zipf(1.1)
targets with 5% ignored, one 4096-token chunk (<= 1 GiB) at a time.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published (no sparsity)
PEAK_HBM_GBS = 8000.0
METRIC = "FLCE fwd+bwd tokens/s and % bf16 MFMA peak at H=4096, V=128256"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def gpu_bench(w, steps, warmup, forward=True):
    import torch

    import linear_cross_entropy_05_amd as flce
    import synth_inputs as si

    dev = torch.device("cuda", 0)
    props = torch.cuda.get_device_properties(dev)
    log(f"[bench] device {props.name} {getattr(props, 'gcnArchName', '?')} CUs={props.multi_processor_count}")
    log(f"[bench] inputs {w.name}: BT={w.BT} H={w.H} V={w.V} {w.dtype}")
    X, W, y = si.make_inputs(w)
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    n_valid = int((y != w.ignore_index).sum())  # the tokens the products compute (ignored ones are skipped)
    del X, W
    C = flce.flce_chunk_tokens(w.BT, w.H, w.V, w.chunk_tokens, w.torch_dtype)
    ws_bytes = flce.flce_workspace_bytes(w.BT, w.H, w.V, w.chunk_tokens, w.torch_dtype)
    out = (
        torch.empty((), dtype=torch.float32, device=dev),
        torch.empty_like(Xd),
        torch.empty((w.V, w.H), dtype=torch.float32, device=dev),
        torch.empty((1,), dtype=torch.int32, device=dev),
    )
    torch.cuda.synchronize()

    # peak extra memory of one call: everything it allocates beyond inputs/outputs
    torch.cuda.reset_peak_memory_stats(dev)
    base = torch.cuda.memory_allocated(dev)
    flce.flce_fwd_bwd(Xd, Wd, yd, w.ignore_index, w.chunk_tokens, out=out, check=True)
    torch.cuda.synchronize()
    peak_extra = torch.cuda.max_memory_allocated(dev) - base
    log(f"[bench] chunk={C} workspace={ws_bytes / 2**30:.3f} GiB peak_extra={peak_extra / 2**30:.3f} GiB "
        f"loss={out[0].item():.6f}")

    workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
    for _ in range(warmup):
        flce.flce_fwd_bwd(Xd, Wd, yd, w.ignore_index, w.chunk_tokens, out=out, workspace=workspace, check=False)
    torch.cuda.synchronize()
    log(f"[bench] warmup {warmup} done; timing {steps} steps")

    # the headline: K whole calls with nothing else on the stream between them
    stream = torch.cuda.current_stream(dev)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    marks[0].record(stream)
    for i in range(steps):
        flce.flce_fwd_bwd(Xd, Wd, yd, w.ignore_index, w.chunk_tokens, out=out, workspace=workspace, check=False)
        marks[i + 1].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    wall1 = time.perf_counter()
    ms = t0.elapsed_time(t1) / steps
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))
    wall_ms = (wall1 - wall0) * 1e3 / steps

    # per-kernel times from a second loop of K calls with the library's event
    # hooks on (two event records around every launch, on its stream)
    with flce.KernelTimer(max_launches=64 * steps + 64) as kt:
        h0 = torch.cuda.Event(enable_timing=True)
        h1 = torch.cuda.Event(enable_timing=True)
        h0.record(stream)
        for i in range(steps):
            flce.flce_fwd_bwd(Xd, Wd, yd, w.ignore_index, w.chunk_tokens, out=out, workspace=workspace, check=False)
        h1.record(stream)
        torch.cuda.synchronize()
    hooked_ms = h0.elapsed_time(h1) / steps

    # forward only (evaluation path), timed separately and reported as context
    fwd_ms = orpo = eager = lib = None
    if forward:
        fwd_ms = time_forward(flce, w, Xd, Wd, yd, steps, stream, float(out[0].item()))
        orpo = time_orpo(flce, w, Xd, Wd, yd, stream)
        eager = time_torch_eager(w, Xd, Wd, yd, stream, float(out[0].item()))
        lib = time_library_gemms(w, Xd, Wd, C, stream)
    err = int(out[3].item())
    if err != 0:
        raise RuntimeError(f"device reported error flag {err}")
    loss = float(out[0].item())
    kernels = {k: {"avg_ms": kt.ms[k] / kt.launches[k], "launches_per_step": kt.launches[k] / steps,
                   "ms_per_step": kt.ms[k] / steps}
               for k in kt.ms if kt.launches[k]}
    log(f"[bench] {ms:.3f} ms/step (wall {wall_ms:.3f}); with kernel hooks {hooked_ms:.3f}; kernels: "
        + ", ".join(f"{k} {v['ms_per_step']:.3f}" for k, v in kernels.items()))
    return {"ms": ms, "ms_min": per_step[0], "ms_median": per_step[len(per_step) // 2], "fwd_ms": fwd_ms,
            "hooked_ms": hooked_ms,
            "orpo": orpo, "eager": eager, "lib": lib, "C": C, "n_valid": n_valid, "ws_bytes": ws_bytes,
            "peak_extra": peak_extra,
            "loss": loss,
            "kernels": kernels,
            "cus": props.multi_processor_count, "arch": getattr(props, "gcnArchName", "?")}


def time_forward(flce, w, Xd, Wd, yd, steps, stream, loss_fwd_bwd):
    """Forward-only calls (no gradients, no logits chunk) on the same inputs:
    ms per call; its loss must equal the fwd+bwd loss to the bit."""
    import torch

    dev = Xd.device
    fwd_out = (torch.empty((), dtype=torch.float32, device=dev), torch.empty((1,), dtype=torch.int32, device=dev))
    fwd_ws = torch.empty((flce.flce_fwd_workspace_bytes(w.BT, w.H, w.V, 0, w.torch_dtype),), dtype=torch.uint8,
                         device=dev)
    for _ in range(2):
        flce.flce_forward(Xd, Wd, yd, w.ignore_index, 0, out=fwd_out, workspace=fwd_ws, check=False)
    torch.cuda.synchronize()
    f0 = torch.cuda.Event(enable_timing=True)
    f1 = torch.cuda.Event(enable_timing=True)
    f0.record(stream)
    for _ in range(steps):
        flce.flce_forward(Xd, Wd, yd, w.ignore_index, 0, out=fwd_out, workspace=fwd_ws, check=False)
    f1.record(stream)
    torch.cuda.synchronize()
    fwd_ms = f0.elapsed_time(f1) / steps
    if float(fwd_out[0].item()) != loss_fwd_bwd:
        raise RuntimeError("forward-only loss differs from the fwd+bwd loss")
    log(f"[bench] forward only: {fwd_ms:.3f} ms/step")
    return fwd_ms


def time_torch_eager(w, Xd, Wd, yd, stream, loss_flce, reps=3):
    """The unfused composition in plain PyTorch on the GPU (context only, the
    analogue of the unfused baseline the pages compare against): full logits
    X W^T in the input dtype, cross-entropy in fp32, autograd backward.
    ms per fwd+bwd, peak extra bytes over the inputs, and its loss."""
    import torch
    import torch.nn.functional as F

    Xr = Xd.detach().clone().requires_grad_(True)
    Wr = Wd.detach().clone().requires_grad_(True)

    def step():
        Xr.grad = None
        Wr.grad = None
        logits = torch.mm(Xr, Wr.t())  # one 2-D product, no batched path
        loss = F.cross_entropy(logits.float(), yd, ignore_index=w.ignore_index)
        loss.backward()
        return loss

    step()
    torch.cuda.synchronize()
    Xr.grad = None
    Wr.grad = None
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    loss = step()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        loss = step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    le = float(loss.item())
    del Xr, Wr, loss
    torch.cuda.empty_cache()
    log(f"[bench] torch eager (unfused) fwd+bwd: {ms:.3f} ms/step, peak extra {peak / 2**30:.2f} GiB, "
        f"loss {le:.6f} (fused {loss_flce:.6f})")
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(w.BT / (ms * 1e-3), 1),
            "peak_extra_bytes": int(peak), "loss": le,
            "what": "torch.mm(X, W.t()) in the input dtype + F.cross_entropy(fp32 logits) + autograd backward"}


def time_library_gemms(w, Xd, Wd, C, stream, reps=5):
    """The three products of one chunk done by the vendor GEMM (torch.mm, i.e.
    hipBLASLt) on the same shapes (context only): logits X_c W^T, dX = G W and
    dW = G^T X_c, each with a plain output in the input dtype (no softmax
    statistics, no fp32 dW read-modify-write).  ms per product and TFLOP/s."""
    import torch

    if Xd.dtype != torch.bfloat16:
        return None
    Xc = Xd[:C]
    G = torch.mm(Xc, Wd.t())  # [C, V], reused as the gradient operand
    shapes = {
        "logits": lambda: torch.mm(Xc, Wd.t()),
        "dx": lambda: torch.mm(G, Wd),
        "dw": lambda: torch.mm(G.t(), Xc),
    }
    out = {}
    flops = 2.0 * C * w.H * w.V
    for name, f in shapes.items():
        for _ in range(2):
            r = f()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            r = f()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}
        del r
    del G
    torch.cuda.empty_cache()
    log("[bench] vendor GEMMs per chunk: " + ", ".join(f"{k} {v['ms']:.3f} ms" for k, v in out.items()))
    out["what"] = (f"torch.mm (hipBLASLt) on one {C}-token chunk: X_c W^T, G W, G^T X_c, bf16 outputs; "
                   "this library's products also compute the softmax statistics (logits) and accumulate dW in fp32, "
                   "its dX and dW products run as one launch (dx_dw, against the vendor's dx + dw), and its chunks "
                   "hold only the non-ignored tokens (this_library_tokens_per_launch on average)")
    return out


def time_orpo(flce, w, Xd, Wd, yd, stream, seq_len=1024, reps=3):
    """Fused-linear ORPO on the same tokens read as BT / seq_len sequences
    (first half chosen, second half rejected): ms per call (context)."""
    import torch

    n_seq = w.BT // seq_len
    if n_seq < 2 or n_seq % 2 or n_seq * seq_len != w.BT:
        return None
    y2 = yd.view(n_seq, seq_len)
    flce.flce_orpo(Xd, Wd, y2, 0.1, w.ignore_index)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        flce.flce_orpo(Xd, Wd, y2, 0.1, w.ignore_index, check=False)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    log(f"[bench] ORPO ({n_seq} sequences of {seq_len}): {ms:.3f} ms/call")
    return {"ms_per_call": round(ms, 4), "sequences": n_seq, "seq_len": seq_len, "beta": 0.1,
            "tokens_per_s": round(w.BT / (ms * 1e-3), 1)}


def time_ce_inplace(reps=5, BT=8192, V=256000, H=3072, seed=4):
    """Logits-only cross-entropy (ce_fwd_bwd_inplace) on the Gemma shape:
    fp32 logits [8192, 256000] = X W^T prepared by torch on the GPU (input
    preparation, not timed; X ~ 3 N(0,1), W ~ N(0, 0.02^2) in bf16 as in the
    Gemma workload, drawn on the GPU), then `reps` timed in-place calls (each
    call works on the previous call's output; the traffic is the same).
    Returns ms per call and GB/s against the algorithmic bytes: one read and
    one write of the logits, 2 x 4 B x BT x V."""
    import torch

    import linear_cross_entropy_05_amd as flce

    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev).manual_seed(seed)
    X = (3.0 * torch.randn(BT, H, generator=g, device=dev)).to(torch.bfloat16).float()
    W = (0.02 * torch.randn(V, H, generator=g, device=dev)).to(torch.bfloat16).float()
    logits = X @ W.T
    del X, W
    y = torch.randint(0, V, (BT,), generator=g, device=dev)
    flce.ce_fwd_bwd_inplace(logits, y)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        flce.ce_fwd_bwd_inplace(logits, y, check=False)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    alg = 2.0 * 4 * BT * V
    del logits
    torch.cuda.empty_cache()
    log(f"[bench] CE in place, fp32 logits {BT}x{V}: {ms:.3f} ms/call, {alg / (ms * 1e-3) / 1e9:.0f} GB/s algorithmic")
    return {"workload": f"gemma logits {BT}x{V} fp32", "ms_per_call": round(ms, 4),
            "algorithmic_bytes": int(alg), "achieved_gbs": round(alg / (ms * 1e-3) / 1e9, 1),
            "peak_gbs": PEAK_HBM_GBS, "frac": round(alg / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def copy_calibration(nbytes=256 << 20, reps=3):
    """A plain device-to-device copy of known size, so that profiler byte
    counters (FETCH_SIZE, WRITE_SIZE) can be scaled against it."""
    import torch

    dev = torch.device("cuda", 0)
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: {reps} x {nbytes} bytes read + written")


def profiled(kernel: str):
    """The committed rocprofv3 counter record of `kernel`
    (profiles/hbm_traffic.json), or None if the kernel sources changed since
    the counters were taken (hash of linear_cross_entropy_05_amd/csrc)."""
    import glob
    import hashlib

    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "linear_cross_entropy_05_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(f.read())
    if h.hexdigest()[:16] != t.get("source_sha256"):
        return None
    return t.get("kernels", {}).get(kernel)


def measured_traffic(kernel: str):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy)."""
    k = profiled(kernel)
    return int(k["bytes_per_launch"]) if k else None


PEAK_CLOCK_GHZ = 2.4  # the clock the published MFMA peak assumes


def measured_mfma(kernel: str, achieved_tflops=None):
    """MFMA busy fraction and the clock the kernel ran at, from the
    SQ_VALU_MFMA_BUSY_CYCLES / GRBM_GUI_ACTIVE counter pass, and the dense
    bf16 peak scaled to that clock (the achieved rate against it when given)."""
    k = profiled(kernel)
    if not k or "mfma_busy_pct" not in k:
        return None
    peak_at_clock = PEAK_BF16_TFLOPS * k["clock_ghz"] / PEAK_CLOCK_GHZ
    out = {"kernel": kernel, "mfma_busy_pct": k["mfma_busy_pct"], "clock_ghz": k["clock_ghz"],
           "peak_at_clock_tflops": round(peak_at_clock, 1),
           "source": "profiles/hbm_traffic.json (rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE)"}
    if achieved_tflops is not None:
        out["frac_at_clock"] = round(achieved_tflops / peak_at_clock, 4)
    return out


def roofline(w, r):
    """Dominant kernel (largest time per step) against its own roofline."""
    name, k = max(r["kernels"].items(), key=lambda kv: kv[1]["ms_per_step"])
    C = r["C"]
    nchunks = -(-w.BT // C)
    # The chunks hold only the non-ignored tokens (N of them), so the launches
    # of one call cover N tokens in all: N / nchunks per launch on average.
    n = r.get("n_valid", w.BT)
    per_launch_flops = {
        # each GEMM launch covers one chunk: 2 * tokens * H * V per product
        # (dX and dW share one launch)
        "logits": 2.0 * n * w.H * w.V / nchunks,
        "dx_dw": 4.0 * n * w.H * w.V / nchunks,
    }
    esz = 2 if w.dtype == "bf16" else 4
    per_launch_bytes = {
        # one chunk of logits read + gradient written, in place
        "grad_inplace": 2.0 * (n / nchunks) * w.V * esz,
    }
    if name in per_launch_flops:
        achieved = per_launch_flops[name] / (k["avg_ms"] * 1e-3) / 1e12
        return name, {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                      "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(name)}
    achieved = per_launch_bytes.get(name, 0.0) / (k["avg_ms"] * 1e-3) / 1e9
    return name, {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                  "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic(name)}


def cpu_baseline(w, sample_tokens):
    """The float64 oracle on the host cores, on the first `sample_tokens` tokens
    of the same workload (full W), as tokens/s."""
    import oracle
    import synth_inputs as si

    from threadpoolctl import threadpool_info, threadpool_limits

    cores = len(os.sched_getaffinity(0))
    X, W, y = si.make_inputs(w)
    S = min(sample_tokens, w.BT)
    Xs, ys = X[:S].clone(), y[:S].clone()
    log(f"[bench] cpu oracle on {S} tokens, {cores} cores")
    with threadpool_limits(limits=cores):
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = int(blas[0].get("num_threads", cores)) if blas else cores
        t0 = time.perf_counter()
        ref = oracle.flce_ref(Xs, W, ys, w.ignore_index)
        dt = time.perf_counter() - t0
    log(f"[bench] cpu oracle {dt:.2f} s (loss on sample {ref['loss']:.5f})")
    import resource

    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    rss_gb = resource.getrusage(resource.RUSAGE_SELF).ru_maxrss / 2**20  # KiB -> GiB
    return {"value": round(S / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {S} of {w.BT} tokens of the {w.name} workload with the full W "
                      f"[{w.V}, {w.H}]; NumPy float64 fwd+bwd, {dt:.2f} s",
            "cpu_model": model, "blas": blas[0].get("internal_api") if blas else None,
            "peak_rss_gib": round(rss_gb, 1)}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="llama3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-forward", action="store_true",
                    help="skip the context timings (forward only, ORPO, unfused torch, logits-only CE)")
    ap.add_argument("--ce-only", action="store_true",
                    help="time only the logits-only CE on the Gemma shape (for its profile)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=8192)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for HBM byte counters)")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {a.gpus}); this library has no multi-GPU path.",
              file=sys.stderr)
        return 2

    import synth_inputs as si

    w = si.workload(a.config)
    if a.copy_calibration:
        copy_calibration()
    if a.ce_only:
        print(json.dumps({"ce_inplace": time_ce_inplace()}), flush=True)
        return 0
    r = gpu_bench(w, a.steps, a.warmup, forward=not a.no_forward)
    ce = None if a.no_forward else time_ce_inplace()
    tokens_per_s = w.BT / (r["ms"] * 1e-3)
    tflops = 6.0 * w.BT * w.H * w.V / (r["ms"] * 1e-3) / 1e12
    dom, roof = roofline(w, r)
    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(r["ms"], 4),
        "ms_per_step_min": round(r["ms_min"], 4),
        "ms_per_step_median": round(r["ms_median"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}-head", "tokens": w.BT, "hidden": w.H, "vocab": w.V,
                   "chunk_tokens": r["C"], "ignore_frac": w.ignore[1] if len(w.ignore) > 1 else 0,
                   "targets": w.targets},
        "tflops": round(tflops, 2),
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        # the same rate counting only the flops the products compute: the
        # ignored tokens do not enter them (6 N H V instead of 6 BT H V)
        "tokens_computed": r["n_valid"],
        "tflops_computed": round(6.0 * r["n_valid"] * w.H * w.V / (r["ms"] * 1e-3) / 1e12, 2),
        "peak_extra_bytes": int(r["peak_extra"]),
        "workspace_bytes": int(r["ws_bytes"]),
        "dominant_kernel": dom,
        "roofline": roof,
        "mfma_counters": measured_mfma(dom, roof["achieved"] if roof["unit"] == "TFLOP/s" else None),
        "kernels_ms_per_step": {k: round(v["ms_per_step"], 4) for k, v in r["kernels"].items()},
        "kernels_sum_ms_per_step": round(sum(v["ms_per_step"] for v in r["kernels"].values()), 4),
        "kernels_loop_ms_per_step": round(r["hooked_ms"], 4),
        "orpo": r["orpo"],
        "torch_eager": r["eager"],
        "vendor_gemm_per_chunk": None if r["lib"] is None else dict(
            r["lib"], this_library_ms={k: round(r["kernels"][k]["avg_ms"], 4) for k in ("logits", "dx_dw")
                                       if k in r["kernels"]},
            this_library_tokens_per_launch=round(r["n_valid"] / -(-w.BT // r["C"]), 1)),
        "ce_inplace": ce,
        "forward_only": None if r["fwd_ms"] is None else {
            "ms_per_step": round(r["fwd_ms"], 4), "tokens_per_s": round(w.BT / (r["fwd_ms"] * 1e-3), 1),
            "tflops": round(2.0 * w.BT * w.H * w.V / (r["fwd_ms"] * 1e-3) / 1e12, 2)},
        "device": {"arch": r["arch"], "cus": r["cus"]},
        "loss": r["loss"],
    }
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, a.cpu_sample_tokens)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
