"""Properties of the HIP path's outputs that hold at any size (needs a gfx950
GPU): ignored tokens are inert, and the gradient rows of a softmax
cross-entropy sum to zero, so the columns of dW sum to zero too.

Bounds come from the arithmetic: a gradient entry stored in bf16 is off by at
most 2^-9 of itself, and a token's gradient row has sum_v |G_iv| <= 2/N (the
softmax minus the one-hot, over N), so sum_v dW[v, h] = sum_i X_ih sum_v G_iv
is at most 2^-9 (2/N) sum_i |X_ih| away from 0, plus fp32 accumulation error
(fp32 chunks: the shared error of the token's lse, ~2^-18, takes the place of 2^-9).
"""
import numpy as np
import pytest
import torch

import synth_inputs as si
from gpu_helpers import ensure_built, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return ensure_built()


def _run(X, W, y, ign, chunk):
    import linear_cross_entropy_05_amd as flce

    dev = torch.device("cuda", 0)
    loss, dX, dW = flce.flce_fwd_bwd(X.to(dev), W.to(dev), y.to(dev), ign, chunk)
    torch.cuda.synchronize()
    return loss.item(), dX.cpu(), dW.cpu()


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_ignored_tokens_are_inert(dtype):
    # 20% of 600 tokens ignored, three chunks (the last ragged), V over several tiles
    w = si.small(600, 256, 2000, dtype, seed=70, ignore=("random_frac", 0.2))
    X, W, y = si.make_inputs(w)
    ign = (y == w.ignore_index)
    say(f"[gpu] inert ignored tokens {dtype}: {int(ign.sum())} of {w.BT} ignored")
    loss, dX, dW = _run(X, W, y, w.ignore_index, 256)
    assert torch.count_nonzero(dX[ign]) == 0
    # other hidden states on the ignored tokens change nothing, bit for bit
    g = torch.Generator().manual_seed(71)
    X2 = X.clone()
    X2[ign] = (torch.randn(int(ign.sum()), w.H, generator=g) * 5).to(X.dtype)
    loss2, dX2, dW2 = _run(X2, W, y, w.ignore_index, 256)
    assert loss2 == loss
    assert torch.equal(dX2, dX)
    assert torch.equal(dW2, dW)


@pytest.mark.parametrize("dtype,chunk", [("fp32", 128), ("bf16", 256), ("bf16", 0)])
def test_dw_columns_sum_to_zero(dtype, chunk):
    w = si.small(700, 200, 3000, dtype, seed=72, w_std=0.2)
    X, W, y = si.make_inputs(w)
    _, _, dW = _run(X, W, y, w.ignore_index, chunk)
    valid = (y != w.ignore_index)
    N = int(valid.sum())
    xabs = X[valid].double().abs().sum(0).numpy()
    col = dW.double().sum(0).numpy()
    colabs = dW.double().abs().sum(0).numpy()
    # bf16 chunk: 2^-9 per entry; fp32 chunk: the entries share the error of
    # their token's lse (a few fp32 ulps of a value ~10, ~1e-6 relative)
    rel = 2.0 ** -9 if dtype == "bf16" else 2.0 ** -18
    bound = rel * (2.0 / N) * xabs + 1e-6 * colabs
    worst = float(np.max(np.abs(col) / bound))
    say(f"  max |column sum| / bound = {worst:.3f} (max |column sum| {np.max(np.abs(col)):.3e})")
    assert worst <= 1.0


def test_ce_inplace_rows_sum_to_zero():
    import linear_cross_entropy_05_amd as flce

    g = torch.Generator().manual_seed(73)
    BT, V = 64, 50257
    logits = (torch.randn(BT, V, generator=g) * 4).cuda()
    y = torch.randint(0, V, (BT,), generator=g)
    y[::9] = -100
    flce.ce_fwd_bwd_inplace(logits, y.cuda(), -100)
    torch.cuda.synchronize()
    G = logits.double().cpu()
    N = int((y != -100).sum())
    rows = G.sum(1).abs()
    # fp32: each entry is off by a few ulps of itself, and sum_v |G_iv| <= 2/N
    say(f"  max |row sum| {float(rows.max()):.3e} (2/N = {2.0 / N:.3e})")
    assert float(rows.max()) <= 1e-5 * (2.0 / N)
    assert torch.count_nonzero(G[::9]) == 0
