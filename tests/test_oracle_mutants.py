"""Plant mistakes in a copy of the oracle's definition (CPU only) and check
that the pins catch every one of them.  This guards the pins themselves:
a pin set that passes a broken oracle would not pin anything."""
import numpy as np
import pytest

from oracle_pins import PINS


def _flce(X, W, y, ig, mistake=None):
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    y = np.asarray(y, dtype=np.int64)
    Z = X @ (W if mistake == "transposed_weight" else W.T)
    BT, V = Z.shape
    keep = y != ig
    if mistake == "ignore_not_masked":
        keep = np.ones(BT, bool)
    N = keep.sum()
    denom = {"batch_mean": BT, "sum_reduction": 1}.get(mistake, max(N, 1))
    if mistake == "no_max_shift":
        lse = np.log(np.exp(Z).sum(1))
    elif mistake == "max_instead_of_lse":
        lse = Z.max(1)
    else:
        m = Z.max(1, keepdims=True)
        lse = (m + np.log(np.exp(Z - m).sum(1, keepdims=True)))[:, 0]
    yy = np.where(y == ig, 0, y) if mistake != "ignore_not_masked" else y % V
    if mistake == "target_off_by_one":
        yy = (yy + 1) % V
    rl = np.where(keep, lse - Z[np.arange(BT), yy], 0.0)
    loss = rl.sum() / denom
    P = np.exp(Z - lse[:, None])
    if mistake == "column_softmax":
        P = np.exp(Z - Z.max(0)) / np.exp(Z - Z.max(0)).sum(0)
    sign = -1.0 if mistake == "flipped_sign" else 1.0
    if mistake != "no_onehot":
        P[np.arange(BT)[keep], yy[keep]] -= 1.0
    P[~keep] = 0.0
    G = sign * P / (1.0 if mistake == "grad_not_normalised" else denom)
    dX = G @ W
    if mistake == "dX_transposed_weight" and W.shape[0] == W.shape[1]:
        dX = G @ W.T  # only type-checks on square weights; falls back otherwise
    dW = G.T @ X
    return {"loss": float(loss), "dX": dX, "dW": dW, "dlogits": G}


MISTAKES = [
    "transposed_weight",
    "ignore_not_masked",
    "batch_mean",
    "sum_reduction",
    "no_max_shift",
    "max_instead_of_lse",
    "target_off_by_one",
    "column_softmax",
    "flipped_sign",
    "no_onehot",
    "grad_not_normalised",
    "dX_transposed_weight",
]


def test_unmutated_copy_passes_every_pin():
    for pin in PINS:
        pin(lambda X, W, y, ig: _flce(X, W, y, ig))


@pytest.mark.parametrize("mistake", MISTAKES)
def test_pins_catch_planted_mistake(mistake):
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(lambda X, W, y, ig: _flce(X, W, y, ig, mistake))
        except (AssertionError, ValueError, IndexError, RuntimeError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {mistake!r}"
