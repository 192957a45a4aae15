"""The oracle against its pins (CPU only)."""
import math

import numpy as np
import pytest

import oracle
from oracle_pins import PINS


def impl(X, W, y, ignore_index):
    return oracle.flce_ref(X, W, y, ignore_index)


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_flce_oracle_pin(pin):
    pin(impl)


def test_out_of_range_target_raises():
    X = np.ones((3, 2))
    W = np.ones((4, 2))
    with pytest.raises(ValueError):
        oracle.flce_ref(X, W, np.array([0, 4, 1]), -100)
    with pytest.raises(ValueError):
        oracle.flce_ref(X, W, np.array([0, -1, 1]), -100)
    oracle.flce_ref(X, W, np.array([0, -100, 3]), -100)  # ignored index is fine


def test_ce_ref_equal_logits_is_ln_v():
    for V in (256, 32000):
        Z = np.full((3, V), 2.5)
        out = oracle.ce_ref(Z, np.array([0, 5, V - 1]))
        assert abs(out["loss"] - math.log(V)) <= 1e-15 * math.log(V)
        assert np.max(np.abs(out["dlogits"].sum(1))) <= 1e-15


def test_ce_ref_matches_flce_ref_on_projected_logits():
    r = np.random.default_rng(3)
    X, W = r.standard_normal((9, 5)), r.standard_normal((12, 5))
    y = r.integers(0, 12, 9)
    y[2] = -100
    a = oracle.flce_ref(X, W, y)
    b = oracle.ce_ref(X @ W.T, y)
    assert a["loss"] == b["loss"]
    assert np.array_equal(a["dlogits"], b["dlogits"])


def test_ce_ref_against_torch():
    import torch
    import torch.nn.functional as F

    r = np.random.default_rng(5)
    Z = r.standard_normal((17, 33)) * 4
    y = r.integers(0, 33, 17)
    y[[0, 9]] = -100
    Zt = torch.tensor(Z, requires_grad=True)
    loss = F.cross_entropy(Zt, torch.tensor(y), ignore_index=-100)
    loss.backward()
    out = oracle.ce_ref(Z, y)
    assert abs(out["loss"] - loss.item()) <= 1e-13 * loss.item()
    assert np.max(np.abs(out["dlogits"] - Zt.grad.numpy())) <= 1e-15


def test_rows_ref_matches_full_oracle():
    r = np.random.default_rng(4)
    X, W = r.standard_normal((10, 6)), r.standard_normal((15, 6)) * 0.5
    y = r.integers(0, 15, 10)
    y[[1, 7]] = -100
    full = oracle.flce_ref(X, W, y)
    rows = [0, 1, 5, 9]
    part = oracle.flce_rows_ref(X, W, y, rows, n_valid=full["n_valid"])
    assert np.allclose(part["row_loss"], full["row_loss"][rows], rtol=1e-14, atol=0)
    assert np.allclose(part["lse"], full["lse"][rows], rtol=1e-14, atol=0)
    assert np.allclose(part["dX"], full["dX"][rows], rtol=1e-13, atol=1e-16)


def test_oracle_upcasts_bf16_exactly():
    import torch

    x = torch.tensor([[1.0 + 2 ** -7, -3.0]], dtype=torch.bfloat16)
    w = torch.tensor([[0.5, 0.25], [2.0 ** -9, 1.0]], dtype=torch.bfloat16)
    out = oracle.flce_ref(x, w, torch.tensor([1]))
    z = np.array([(1 + 2 ** -7) * 0.5 - 0.75, (1 + 2 ** -7) * 2 ** -9 - 3.0])
    lse = z.max() + math.log(np.exp(z - z.max()).sum())
    assert out["loss"] == pytest.approx(lse - z[1], rel=1e-15)


def test_ce_rows_ref_matches_full_batch():
    r = np.random.default_rng(6)
    Z = r.standard_normal((12, 40)) * 3
    y = r.integers(0, 40, 12)
    y[[2, 5]] = -100
    full = oracle.ce_ref(Z, y)
    rows = [0, 2, 7, 11]
    part = oracle.ce_rows_ref(Z[rows], y[rows], n_valid=full["n_valid"])
    assert np.allclose(part["row_loss"], full["row_loss"][rows], rtol=1e-14, atol=0)
    assert np.allclose(part["dlogits"], full["dlogits"][rows], rtol=1e-13, atol=1e-18)


def test_row_lse_closed_form():
    Z = np.log(np.array([[1.0, 2.0, 3.0, 4.0], [0.5, 0.5, 0.5, 0.5]]))
    assert np.allclose(oracle.row_lse(Z), [np.log(10.0), np.log(2.0)], rtol=1e-15)
