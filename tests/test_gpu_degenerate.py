"""Smallest shapes on the HIP path (needs a gfx950 GPU): one token, the
smallest hidden sizes the boundary accepts (4 for fp32, 8 for bf16), a
vocabulary of one or two entries, one-token chunks.

With V = 1 the softmax is exactly 1 on the only entry, so the loss and both
gradients are exactly 0 (the oracle returns zeros); the GPU takes the target
logit from its own fp32 dot product, so its loss agrees to rounding, and is
held to an absolute bound.  V = 2 is the logistic loss and goes through the
usual relative comparison against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_helpers import TOL, ensure_built, rel_err, run_gpu, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return ensure_built()


@pytest.mark.parametrize("BT,H,dtype,chunk", [(1, 4, "fp32", 0), (5, 4, "fp32", 2), (1, 8, "bf16", 0),
                                              (9, 8, "bf16", 1)])
def test_single_entry_vocabulary(BT, H, dtype, chunk):
    w = si.small(BT, H, 1, dtype, seed=40 + BT, ignore=("none",))
    (X, W, y), out = run_gpu(w, chunk)
    ref = oracle.flce_ref(X, W, y, w.ignore_index)
    assert ref["loss"] == 0.0 and not ref["dX"].any() and not ref["dW"].any()
    say(f"  loss {out['loss']:.3e}; max|dX| {float(out['dX'].abs().max()):.3e}; "
        f"max|dW| {float(out['dW'].abs().max()):.3e}")
    assert abs(out["loss"]) <= 1e-6
    assert float(out["dX"].float().abs().max()) <= 1e-6
    assert float(out["dW"].abs().max()) <= 1e-6
    assert float(out["row_loss"].abs().max()) <= 1e-6


@pytest.mark.parametrize("BT,H,V,dtype,chunk", [(1, 4, 2, "fp32", 0), (3, 4, 2, "fp32", 1), (1, 8, 2, "bf16", 0),
                                                (6, 8, 3, "bf16", 4), (2, 16, 5, "fp32", 0)])
def test_tiny_shapes_match_oracle(BT, H, V, dtype, chunk):
    w = si.small(BT, H, V, dtype, seed=50 + BT + V, ignore=("none",), w_std=0.5)
    (X, W, y), out = run_gpu(w, chunk)
    ref = oracle.flce_ref(X, W, y, w.ignore_index)
    tl, tg = TOL[dtype]
    el = abs(out["loss"] - ref["loss"]) / abs(ref["loss"])
    ex = rel_err(to_np(out["dX"]), ref["dX"])
    ew = rel_err(to_np(out["dW"]), ref["dW"])
    say(f"  loss {out['loss']:.7f} ref {ref['loss']:.7f} err {el:.2e}; dX {ex:.2e}; dW {ew:.2e}")
    assert el <= tl and ex <= tg and ew <= tg
    if V == 2:
        # logistic loss: l_i = softplus(z_other - z_target)
        Z = X.double().numpy() @ W.double().numpy().T
        yi = y.numpy()
        other = Z[np.arange(BT), 1 - yi]
        tgt = Z[np.arange(BT), yi]
        assert abs(out["loss"] - float(np.mean(np.logaddexp(0.0, other - tgt)))) <= tl * abs(ref["loss"])


def test_single_token_forward_only_equals_fwd_bwd():
    import linear_cross_entropy_05_amd as flce

    w = si.small(1, 8, 300, "bf16", seed=60, ignore=("none",))
    X, W, y = si.make_inputs(w)
    dev = torch.device("cuda", 0)
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    lf = flce.flce_forward(Xd, Wd, yd, w.ignore_index, 0)
    lb = flce.flce_fwd_bwd(Xd, Wd, yd, w.ignore_index, 0)[0]
    torch.cuda.synchronize()
    assert float(lf.item()) == float(lb.item())
