"""bench.py's host-side arithmetic on the CPU: the roofline of the dominant
kernel, the refusal of more than one GPU, and the committed counter record
being dropped once the kernel sources no longer match it."""
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth_inputs as si  # noqa: E402


def _r(kernels, C):
    return {"C": C, "kernels": {k: {"avg_ms": v[0], "ms_per_step": v[1]} for k, v in kernels.items()}}


def test_roofline_of_an_mfma_kernel():
    w = si.workload("llama3")
    # dX + dW dominant: 6.8 ms per launch, two launches per step of 2 chunks of 4096 tokens
    name, roof = bench.roofline(w, _r({"logits": (3.3, 6.6), "dx_dw": (6.8, 13.6), "grad_inplace": (0.4, 0.8)},
                                       4096))
    assert name == "dx_dw" and roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s"
    flops = 4.0 * 4096 * 4096 * 128256  # one chunk, two products: 4 C H V
    assert roof["achieved"] == pytest.approx(flops / 6.8e-3 / 1e12, rel=1e-4)
    assert roof["frac"] == pytest.approx(roof["achieved"] / 2500.0, rel=1e-3)
    assert roof["peak"] == 2500.0


def test_roofline_counts_only_the_computed_tokens():
    # with 410 of 8192 tokens ignored the two dW launches cover 7782 tokens:
    # 3891 per launch on average
    w = si.workload("llama3")
    r = _r({"logits": (3.3, 6.6)}, 4096)
    r["n_valid"] = 8192 - 410
    _, roof = bench.roofline(w, r)
    assert roof["achieved"] == pytest.approx(2.0 * 3891 * 4096 * 128256 / 3.3e-3 / 1e12, rel=1e-4)


def test_roofline_of_an_hbm_kernel():
    w = si.workload("llama3")
    name, roof = bench.roofline(w, _r({"grad_inplace": (0.4, 19.0), "dx_dw": (6.8, 13.6)}, 4096))
    assert name == "grad_inplace" and roof["bound"] == "hbm" and roof["unit"] == "GB/s"
    # one chunk of bf16 logits read and its gradient written: 2 x 4096 x 128256 x 2 bytes
    assert roof["achieved"] == pytest.approx(2 * 4096 * 128256 * 2 / 0.4e-3 / 1e9, rel=1e-4)


def test_more_than_one_gpu_is_refused():
    assert bench.main(["--gpus", "2"]) == 2


def test_counter_record_follows_the_sources(tmp_path, monkeypatch):
    # the committed record is used only while its hash matches the kernel sources
    rec = bench.profiled("dx_dw")
    if rec is None:
        pytest.skip("counter record does not match the current sources")
    assert bench.measured_traffic("dx_dw") == int(rec["bytes_per_launch"])
    m = bench.measured_mfma("dx_dw", 1000.0)
    assert m["peak_at_clock_tflops"] == pytest.approx(2500.0 * rec["clock_ghz"] / 2.4, rel=1e-3)
    # a copy of the repository whose record names other sources: both fields drop to None
    fake = tmp_path / "repo"
    (fake / "profiles").mkdir(parents=True)
    (fake / "linear_cross_entropy_05_amd" / "csrc").mkdir(parents=True)
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
        t = json.load(f)
    (fake / "profiles" / "hbm_traffic.json").write_text(json.dumps(t))
    (fake / "linear_cross_entropy_05_amd" / "csrc" / "k.hip").write_text("// changed")
    monkeypatch.setattr(bench, "ROOT", str(fake))
    assert bench.profiled("dx_dw") is None
    assert bench.measured_traffic("dx_dw") is None and bench.measured_mfma("dx_dw") is None
