"""Per-token gradient scales (token_scale) and the module's reductions on the
GPU, against the float64 oracle: gradients of sum_i s_i * loss_i."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_helpers import TOL, ensure_built, rel_err, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return ensure_built()


def _scales(BT, seed):
    r = np.random.default_rng(seed)
    return torch.tensor(r.uniform(-1.0, 2.0, BT), dtype=torch.float32)


@pytest.mark.parametrize("dtype,chunk", [("fp32", 256), ("bf16", 256), ("bf16", 0)])
def test_token_scale_matches_oracle(dtype, chunk):
    import linear_cross_entropy_05_amd as flce

    w = si.small(700, 200, 1000, dtype, seed=51, w_std=0.05)
    X, W, y = si.make_inputs(w)
    s = _scales(w.BT, 52)
    dev = torch.device("cuda", 0)
    say(f"[gpu] flce_fwd_bwd token_scale {w.name} chunk={chunk}")
    loss, dX, dW = flce.flce_fwd_bwd(X.to(dev), W.to(dev), y.to(dev), w.ignore_index, chunk, token_scale=s.to(dev))
    torch.cuda.synchronize()
    ref = oracle.flce_ref(X, W, y, w.ignore_index, token_scale=s)
    tl, tg = TOL[w.dtype]
    ex, ew = rel_err(to_np(dX), ref["dX"]), rel_err(to_np(dW), ref["dW"])
    el = abs(loss.item() - ref["loss"]) / ref["loss"]
    say(f"  loss err {el:.2e}; dX {ex:.2e}; dW {ew:.2e}")
    assert el <= tl and ex <= tg and ew <= tg


def test_token_scale_one_over_n_is_bitwise_the_mean():
    import linear_cross_entropy_05_amd as flce

    w = si.small(300, 136, 700, "bf16", seed=53)
    Xd, Wd, yd = [t.to(torch.device("cuda", 0)) for t in si.make_inputs(w)]
    n = int((yd != w.ignore_index).sum())
    s = torch.full((w.BT,), 1.0 / n, dtype=torch.float32, device=Xd.device)
    a = flce.flce_fwd_bwd(Xd, Wd, yd, w.ignore_index)
    b = flce.flce_fwd_bwd(Xd, Wd, yd, w.ignore_index, token_scale=s)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])


def test_module_reduction_none():
    """reduction='none': per-token losses from the forward-only path; backward
    with random upstream gradients equals the oracle with those as scales."""
    import linear_cross_entropy_05_amd as flce

    w = si.small(400, 128, 900, "bf16", seed=54, w_std=0.05)
    X, W, y = si.make_inputs(w)
    dev = torch.device("cuda", 0)
    Wg = W.to(dev).requires_grad_(True)
    Xg = X.to(dev).requires_grad_(True)
    mod = flce.FusedLinearCrossEntropyLoss(ignore_index=w.ignore_index, reduction="none")
    rows = mod(Wg, Xg, y.to(dev))
    g = _scales(w.BT, 55)
    rows.backward(g.to(dev))
    torch.cuda.synchronize()
    ref = oracle.flce_ref(X, W, y, w.ignore_index, token_scale=g)
    tl, tg = TOL["bf16"]
    er = rel_err(to_np(rows), ref["row_loss"])
    ex, ew = rel_err(to_np(Xg.grad), ref["dX"]), rel_err(to_np(Wg.grad), ref["dW"])
    say(f"  rows {er:.2e}; dX {ex:.2e}; dW {ew:.2e}")
    assert rows.shape == (w.BT,) and Wg.grad.dtype == torch.bfloat16
    assert er <= tl and ex <= tg and ew <= tg


def test_module_mean_upstream_scale():
    """reduction='mean': an upstream gradient of 1 hands on the fused
    gradients unchanged; 2.5 scales them."""
    import linear_cross_entropy_05_amd as flce

    w = si.small(300, 64, 500, "fp32", seed=56)
    X, W, y = si.make_inputs(w)
    dev = torch.device("cuda", 0)
    mod = flce.FusedLinearCrossEntropyLoss(ignore_index=w.ignore_index)
    _, dX, dW = flce.flce_fwd_bwd(X.to(dev), W.to(dev), y.to(dev), w.ignore_index)
    for scale in (1.0, 2.5):
        Wg = W.to(dev).requires_grad_(True)
        Xg = X.to(dev).requires_grad_(True)
        (mod(Wg, Xg, y.to(dev)) * scale).backward()
        torch.cuda.synchronize()
        if scale == 1.0:
            assert torch.equal(Xg.grad, dX) and torch.equal(Wg.grad, dW)
        else:
            assert rel_err(to_np(Xg.grad), 2.5 * to_np(dX)) <= 1e-6
            assert rel_err(to_np(Wg.grad), 2.5 * to_np(dW)) <= 1e-6
