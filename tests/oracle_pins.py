"""Pins for the FLCE oracle: properties fixed by mathematics, not by the oracle itself.

Each pin takes an implementation ``impl(X, W, y, ignore_index) -> dict`` with
keys ``loss``, ``dX``, ``dW``, ``dlogits`` (all float64) and raises
AssertionError if the implementation violates the property.  The same pins
run against the real oracle (all must pass) and against deliberately broken
copies of it (each copy must fail at least one pin), so that a plausible
mistake anywhere in the oracle -- a dropped term, a wrong sign or index, a
transposed operand, a wrong normaliser -- cannot go unnoticed.

Sources of truth: closed forms of softmax cross-entropy (W = 0 gives ln V;
V = 2 gives the logistic loss), invariances of the definition (row sums of
the softmax gradient, a common shift of the logits, permutations), central
finite differences, a pure-Python brute force, and torch's CPU float64
``cross_entropy`` with autograd as an independent library routine.
"""

from __future__ import annotations

import math

import numpy as np

IGN = -100


def _rng(seed):
    return np.random.default_rng(seed)


def _case(seed, BT, H, V, n_ignore=1, scale=1.0, wstd=0.3):
    r = _rng(seed)
    X = r.standard_normal((BT, H)) * scale
    W = r.standard_normal((V, H)) * wstd
    y = r.integers(0, V, BT)
    if n_ignore:
        y[r.choice(BT, n_ignore, replace=False)] = IGN
    return X, W, y


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(float(np.max(np.abs(b))) if b.size else 0.0, 1e-300)
    return float(np.max(np.abs(a - b))) / den if a.size else 0.0


def pin_zero_weight(impl):
    """W = 0: every logit is 0, so loss = ln V exactly, dX = 0 and
    dW[v] = (1/N) * ((1/V) * sum_valid x_i - sum_{valid, y_i = v} x_i)."""
    r = _rng(11)
    BT, H, V = 12, 5, 7
    X = r.standard_normal((BT, H))
    W = np.zeros((V, H))
    y = np.array([0, 3, 3, IGN, 6, 1, 3, 0, IGN, 2, 5, 6])
    out = impl(X, W, y, IGN)
    assert abs(out["loss"] - math.log(V)) <= 1e-15 * math.log(V), out["loss"]
    assert np.all(out["dX"] == 0.0)
    keep = y != IGN
    N = keep.sum()
    expect = np.tile(X[keep].sum(0) / V, (V, 1))
    for i in np.flatnonzero(keep):
        expect[y[i]] -= X[i]
    expect /= N
    assert _rel(out["dW"], expect) <= 1e-14


def pin_row_sums(impl):
    """Each row of dlogits (softmax - onehot)/N sums to 0."""
    X, W, y = _case(1, 9, 6, 13, n_ignore=2)
    G = impl(X, W, y, IGN)["dlogits"]
    assert G.shape == (9, 13)
    assert np.max(np.abs(G.sum(1))) <= 1e-15 * 13


def pin_dw_column_sums(impl):
    """Summing dW over the vocabulary gives 0 for every hidden unit."""
    X, W, y = _case(2, 10, 4, 9)
    dW = impl(X, W, y, IGN)["dW"]
    assert np.max(np.abs(dW.sum(0))) <= 1e-14 * max(1.0, np.max(np.abs(dW)))


def pin_ignored_rows(impl):
    """Ignored rows have zero dlogits and dX, and their hidden state does not
    move the loss or dW."""
    X, W, y = _case(3, 8, 5, 11, n_ignore=3)
    out = impl(X, W, y, IGN)
    ign = y == IGN
    assert np.all(out["dlogits"][ign] == 0.0)
    assert np.all(out["dX"][ign] == 0.0)
    X2 = X.copy()
    X2[ign] += 7.0
    out2 = impl(X2, W, y, IGN)
    assert abs(out2["loss"] - out["loss"]) <= 1e-14 * abs(out["loss"])
    assert _rel(out2["dW"], out["dW"]) <= 1e-13


def pin_shift_invariance(impl):
    """Adding the same vector u to every row of W shifts row i's logits by
    x_i . u: loss, dX and dW are unchanged."""
    X, W, y = _case(4, 7, 6, 10)
    u = _rng(40).standard_normal(6)
    a = impl(X, W, y, IGN)
    b = impl(X, W + u[None, :], y, IGN)
    assert abs(a["loss"] - b["loss"]) <= 1e-13 * abs(a["loss"])
    assert _rel(b["dX"], a["dX"]) <= 1e-12
    assert _rel(b["dW"], a["dW"]) <= 1e-12


def pin_two_class(impl):
    """V = 2: each loss term is softplus(z_other - z_target)."""
    X, W, y = _case(5, 16, 3, 2, n_ignore=2, wstd=1.5)
    out = impl(X, W, y, IGN)
    Z = X @ W.T
    keep = y != IGN
    terms = [math.log1p(math.exp(Z[i, 1 - y[i]] - Z[i, y[i]])) for i in np.flatnonzero(keep)]
    expect = math.fsum(terms) / keep.sum()
    assert abs(out["loss"] - expect) <= 1e-14 * expect


def pin_finite_differences(impl):
    """dX and dW agree with central differences of the loss (step 1e-6, float64)."""
    X, W, y = _case(6, 5, 4, 6, n_ignore=1)
    out = impl(X, W, y, IGN)
    h = 1e-6

    def loss(Xa, Wa):
        return impl(Xa, Wa, y, IGN)["loss"]

    num_dX = np.zeros_like(X)
    for i in range(X.shape[0]):
        for j in range(X.shape[1]):
            P, M = X.copy(), X.copy()
            P[i, j] += h
            M[i, j] -= h
            num_dX[i, j] = (loss(P, W) - loss(M, W)) / (2 * h)
    num_dW = np.zeros_like(W)
    for i in range(W.shape[0]):
        for j in range(W.shape[1]):
            P, M = W.copy(), W.copy()
            P[i, j] += h
            M[i, j] -= h
            num_dW[i, j] = (loss(X, P) - loss(X, M)) / (2 * h)
    assert _rel(out["dX"], num_dX) <= 1e-7, _rel(out["dX"], num_dX)
    assert _rel(out["dW"], num_dW) <= 1e-7, _rel(out["dW"], num_dW)


def pin_torch_library(impl):
    """Independent library routine: torch CPU float64 cross_entropy (mean over
    non-ignored targets) with autograd, on a square H = V case (so that a
    transposed weight would still type-check) and a rectangular one."""
    import torch
    import torch.nn.functional as F

    for seed, (BT, H, V) in ((7, (11, 9, 9)), (8, (13, 6, 17))):
        X, W, y = _case(seed, BT, H, V, n_ignore=2)
        Xt = torch.tensor(X, requires_grad=True)
        Wt = torch.tensor(W, requires_grad=True)
        loss = F.cross_entropy(Xt @ Wt.T, torch.tensor(y), ignore_index=IGN, reduction="mean")
        loss.backward()
        out = impl(X, W, y, IGN)
        assert abs(out["loss"] - loss.item()) <= 1e-13 * abs(loss.item())
        assert _rel(out["dX"], Xt.grad.numpy()) <= 1e-12
        assert _rel(out["dW"], Wt.grad.numpy()) <= 1e-12


def pin_permutations(impl):
    """Permuting tokens permutes dX rows and leaves loss and dW; relabelling
    vocabulary ids permutes dW rows and leaves loss and dX."""
    X, W, y = _case(9, 10, 5, 8, n_ignore=2)
    a = impl(X, W, y, IGN)
    p = _rng(90).permutation(10)
    b = impl(X[p], W, y[p], IGN)
    assert abs(a["loss"] - b["loss"]) <= 1e-14 * abs(a["loss"])
    assert _rel(b["dX"], a["dX"][p]) <= 1e-13
    assert _rel(b["dW"], a["dW"]) <= 1e-13
    q = _rng(91).permutation(8)  # new id k holds old id q[k]
    inv = np.argsort(q)
    y2 = np.where(y == IGN, IGN, inv[np.where(y == IGN, 0, y)])
    c = impl(X, W[q], y2, IGN)
    assert abs(a["loss"] - c["loss"]) <= 1e-14 * abs(a["loss"])
    assert _rel(c["dX"], a["dX"]) <= 1e-13
    assert _rel(c["dW"], a["dW"][q]) <= 1e-13


def pin_large_logits(impl):
    """Logits of size ~1000 stay finite (max-shifted log-sum-exp).  With one
    logit 1000 above the rest the loss is ~0 when it is the target and
    ~1000 + (z_dominant - z_target) otherwise."""
    H, V = 2, 4
    W = np.array([[1000.0, 0.0], [0.0, 0.0], [0.0, 1.0], [0.0, -1.0]])
    X = np.array([[1.0, 0.0], [1.0, 0.0], [1.0, 0.5]])
    y = np.array([0, 1, 2])
    out = impl(X, W, y, IGN)
    assert np.isfinite(out["loss"]) and np.all(np.isfinite(out["dX"])) and np.all(np.isfinite(out["dW"]))
    # row 0: target is the dominant logit -> term ~ 3 e^-1000 = 0; row 1: 1000 - 0; row 2: 1000 - 0.5
    expect = (0.0 + 1000.0 + 999.5) / 3
    assert abs(out["loss"] - expect) <= 1e-12 * expect


def pin_brute_force(impl):
    """Pure-Python loops (math.fsum/exp/log, explicit dot products)."""
    from oracle import flce_brute_force

    X, W, y = _case(12, 6, 4, 9, n_ignore=2)
    out = impl(X, W, y, IGN)
    ref = flce_brute_force(X, W, y, IGN)
    assert abs(out["loss"] - ref["loss"]) <= 1e-14 * abs(ref["loss"])
    assert _rel(out["dX"], ref["dX"]) <= 1e-13
    assert _rel(out["dW"], ref["dW"]) <= 1e-13


def pin_batch_duplication(impl):
    """Repeating the batch twice keeps the mean loss and dW, halves dX rows
    (N doubles): fixes the 1/N normaliser to the count of valid tokens."""
    X, W, y = _case(13, 6, 3, 5, n_ignore=2)
    a = impl(X, W, y, IGN)
    b = impl(np.vstack([X, X]), W, np.concatenate([y, y]), IGN)
    assert abs(a["loss"] - b["loss"]) <= 1e-14 * abs(a["loss"])
    assert _rel(b["dW"], a["dW"]) <= 1e-13
    assert _rel(b["dX"][:6], a["dX"] / 2) <= 1e-13


def pin_all_ignored(impl):
    """N = 0 (every target ignored): loss 0 and zero gradients (reading of a
    case the pages leave open; the mean would otherwise be 0/0)."""
    X, W, y = _case(14, 4, 3, 5, n_ignore=0)
    y[:] = IGN
    out = impl(X, W, y, IGN)
    assert out["loss"] == 0.0
    assert np.all(out["dX"] == 0.0) and np.all(out["dW"] == 0.0)


def pin_ignore_index_value(impl):
    """The ignore index is the caller's: with ignore_index = 3, class 3 rows
    drop out and -100 is not special (it would then be out of range)."""
    X, W, y = _case(15, 7, 3, 6, n_ignore=0)
    y[[1, 4]] = 3
    out = impl(X, W, y, 3)
    keep = y != 3
    ref = impl(X[keep], W, y[keep], IGN)
    assert abs(out["loss"] - ref["loss"]) <= 1e-14 * abs(ref["loss"])
    assert _rel(out["dW"], ref["dW"]) <= 1e-13


PINS = [
    pin_zero_weight,
    pin_row_sums,
    pin_dw_column_sums,
    pin_ignored_rows,
    pin_shift_invariance,
    pin_two_class,
    pin_finite_differences,
    pin_torch_library,
    pin_permutations,
    pin_large_logits,
    pin_brute_force,
    pin_batch_duplication,
    pin_all_ignored,
    pin_ignore_index_value,
]
