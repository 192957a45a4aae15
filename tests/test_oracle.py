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


# ---- per-token gradient scales (token_scale): gradients of sum_i s_i * loss_i ----

def _weighted_case(seed, BT=6, H=4, V=7):
    r = np.random.default_rng(seed)
    X = r.standard_normal((BT, H))
    W = r.standard_normal((V, H)) * 0.4
    y = r.integers(0, V, BT)
    y[2] = -100
    s = r.uniform(-1.0, 2.0, BT)  # any real weights, negative ones included
    return X, W, y, s


def test_token_scale_finite_differences():
    """dX and dW with token_scale s are the central differences of
    f = sum_i s_i * loss_i, where loss_i are the oracle's token losses (pinned
    on their own by the definition pins)."""
    X, W, y, s = _weighted_case(41)
    out = oracle.flce_ref(X, W, y, -100, token_scale=s)
    h = 1e-6

    def f(Xa, Wa):
        return float(np.dot(s, oracle.flce_ref(Xa, Wa, y, -100)["row_loss"]))

    for name, A in (("dX", X), ("dW", W)):
        num = np.zeros_like(A)
        for i in range(A.shape[0]):
            for j in range(A.shape[1]):
                P, M = A.copy(), A.copy()
                P[i, j] += h
                M[i, j] -= h
                num[i, j] = (f(P, W) - f(M, W)) / (2 * h) if name == "dX" else (f(X, P) - f(X, M)) / (2 * h)
        err = float(np.max(np.abs(out[name] - num))) / float(np.max(np.abs(num)))
        assert err <= 1e-7, (name, err)
    # the loss itself is still the mean over non-ignored tokens
    assert out["loss"] == oracle.flce_ref(X, W, y, -100)["loss"]


def test_token_scale_against_torch():
    """torch CPU float64: cross_entropy(reduction='none') weighted by s, summed, autograd."""
    import torch
    import torch.nn.functional as F

    X, W, y, s = _weighted_case(42, BT=9, H=5, V=11)
    Xt = torch.tensor(X, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    rows = F.cross_entropy(Xt @ Wt.T, torch.tensor(y), ignore_index=-100, reduction="none")
    (rows * torch.tensor(s)).sum().backward()
    out = oracle.flce_ref(X, W, y, -100, token_scale=s)
    assert float(np.max(np.abs(out["dX"] - Xt.grad.numpy()))) <= 1e-12 * float(np.max(np.abs(Xt.grad.numpy())))
    assert float(np.max(np.abs(out["dW"] - Wt.grad.numpy()))) <= 1e-12 * float(np.max(np.abs(Wt.grad.numpy())))
    assert np.allclose(out["row_loss"], rows.detach().numpy(), rtol=1e-13, atol=0)


def test_token_scale_one_over_n_is_the_mean():
    X, W, y, _ = _weighted_case(43)
    n = int((y != -100).sum())
    a = oracle.flce_ref(X, W, y, -100)
    b = oracle.flce_ref(X, W, y, -100, token_scale=np.full(len(y), 1.0 / n))
    assert float(np.max(np.abs(a["dX"] - b["dX"]))) <= 1e-15 * float(np.max(np.abs(a["dX"])))
    assert float(np.max(np.abs(a["dW"] - b["dW"]))) <= 1e-15 * float(np.max(np.abs(a["dW"])))


def test_rowblock_oracle_equals_whole_oracle():
    """The row-blocked form (for hosts short of memory) against the whole
    definition, with blocks that do not divide the batch and ignored rows in
    several blocks; also the all-ignored batch."""
    import synth_inputs as si

    w = si.small(37, 24, 50, "fp32", seed=11, ignore=("random_frac", 0.2))
    X, W, y = si.make_inputs(w)
    full = oracle.flce_ref(X, W, y, w.ignore_index)
    for block in (1, 5, 16, 37, 100):
        part = oracle.flce_ref_rowblocks(X, W, y, w.ignore_index, block=block)
        assert abs(part["loss"] - full["loss"]) <= 1e-14 * abs(full["loss"])
        for k in ("dX", "dW", "row_loss", "lse"):
            assert np.max(np.abs(part[k] - full[k])) <= 1e-13 * np.max(np.abs(full[k])), (block, k)
        assert part["n_valid"] == full["n_valid"]
    y2 = y.clone()
    y2[:] = w.ignore_index
    part = oracle.flce_ref_rowblocks(X, W, y2, w.ignore_index, block=8)
    assert part["loss"] == 0.0 and not part["dX"].any() and not part["dW"].any()
