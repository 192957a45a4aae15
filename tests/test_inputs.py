"""The seeded input generator: reproducible, right shapes, right ignore pattern (CPU)."""
import math

import torch

import synth_inputs as si


def test_tiny_workload_shape_and_ignore():
    w = si.workload("tiny")
    X, W, y = si.make_inputs(w)
    assert X.shape == (8, 128) and W.shape == (256, 128) and y.shape == (8,)
    assert X.dtype == torch.float32 and y.dtype == torch.int64
    assert y[3].item() == -100 and int((y == -100).sum()) == 1
    assert int(y[y != -100].min()) >= 0 and int(y.max()) < 256


def test_reproducible():
    w = si.small(64, 32, 100, "bf16", seed=9)
    a = si.make_inputs(w)
    b = si.make_inputs(w)
    for s, t in zip(a, b):
        assert torch.equal(s, t)
    assert si.fingerprint(*a) == si.fingerprint(*b)


def test_ignore_patterns():
    X, W, y = si.make_inputs(si.small(2048, 8, 64, "bf16", seed=1))
    assert int((y == -100).sum()) == 102  # round(0.05 * 2048)
    X, W, y = si.make_inputs(si.small(100, 8, 64, "bf16", seed=1, ignore=("tail_frac", 0.10)))
    assert torch.all(y[90:] == -100) and torch.all(y[:90] != -100)


def test_zipf_targets_favour_low_ids():
    X, W, y = si.make_inputs(si.small(20000, 8, 5000, "bf16", seed=2, targets="zipf1.1", ignore=("none",)))
    counts = torch.bincount(y, minlength=5000).double()
    # p(0)/p(1) = 2^1.1
    assert abs(counts[0] / counts[1] - 2 ** 1.1) < 0.25
    assert counts[0] / 20000 > 0.05


def test_scales():
    X, W, y = si.make_inputs(si.small(512, 256, 300, "bf16", seed=3, x_scale=3.0))
    assert abs(X.float().std().item() - 3.0) < 0.1
    assert abs(W.float().std().item() - 0.02) < 0.002
    assert X.dtype == torch.bfloat16 and W.dtype == torch.bfloat16
