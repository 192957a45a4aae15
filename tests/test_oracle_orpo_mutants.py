"""Plant mistakes in a copy of the ORPO definition (CPU only) and check that
the ORPO pins catch every one of them, as tests/test_oracle_mutants.py does
for the cross-entropy oracle: a pin set that passes a broken definition
would not pin anything.

The pins here are the ones of tests/test_oracle_orpo.py, written against a
function argument: a two-class closed form, beta = 0 (the chosen-token
cross-entropy of the pinned cross-entropy oracle), identical chosen and
rejected halves (log odds ratio 0, odds-ratio term beta log 2), and central
finite differences of the loss."""
import math

import numpy as np
import pytest

import oracle
from oracle.orpo_oracle import orpo_ref

IGN = -100


def _softplus(x):
    return max(x, 0.0) + math.log1p(math.exp(-abs(x)))


def _sigmoid(x):
    return 1.0 / (1.0 + math.exp(-x)) if x >= 0 else math.exp(x) / (1.0 + math.exp(x))


def _orpo(X, W, y, n_seq, beta, mistake=None, loss_only=False):
    """The ORPO loss and gradients from the plain definition, with an
    optional planted mistake."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    y = np.asarray(y, dtype=np.int64)
    Z = X @ W.T
    m = Z.max(axis=1)
    lse = m + np.log(np.exp(Z - m[:, None]).sum(axis=1))
    keep = y != IGN
    yy = np.where(keep, y, 0)
    rl = np.where(keep, lse - Z[np.arange(len(y)), yy], 0.0)
    T = len(y) // n_seq
    B = n_seq // 2
    kp = keep.reshape(n_seq, T)
    L = rl.reshape(n_seq, T)
    n = kp.sum(axis=1)
    if mistake == "sum_not_mean_logp":
        a = -np.where(kp, L, 0.0).sum(axis=1)
    else:
        a = np.where(n > 0, -np.where(kp, L, 0.0).sum(axis=1) / np.maximum(n, 1), 0.0)
    nll_rows = n_seq if mistake == "nll_all_sequences" else B
    n_nll = int(n[:nll_rows].sum())
    nll = float(np.where(kp[:nll_rows], L[:nll_rows], 0.0).sum() / max(n_nll, 1))
    w = np.zeros((n_seq, T))
    w[:nll_rows] = np.where(kp[:nll_rows], 1.0 / max(n_nll, 1), 0.0)
    scale = beta if mistake == "beta_not_over_B" else beta / B
    or_sum = 0.0
    for p in range(B):
        sw, sl = p, B + p
        if n[sw] == 0 or n[sl] == 0:
            continue
        aw, al = a[sw], a[sl]
        if mistake == "no_log1m":
            r = aw - al
            dr_daw, dr_dal = 1.0, -1.0
        else:
            r = (aw - al) - (math.log(-math.expm1(aw)) - math.log(-math.expm1(al)))
            dr_daw, dr_dal = 1.0 / (-math.expm1(aw)), -1.0 / (-math.expm1(al))
        if mistake == "r_sign":
            r, dr_daw, dr_dal = -r, -dr_daw, -dr_dal
        if mistake == "softplus_positive":
            or_sum += _softplus(r)
            g = _sigmoid(r) * scale
        else:
            or_sum += _softplus(-r)
            g = -_sigmoid(-r) * scale
        if mistake == "grad_wrong_sign_rejected":
            dr_dal = -dr_dal
        nw = 1.0 if mistake in ("grad_missing_1_over_n", "sum_not_mean_logp") else float(n[sw])
        nl = 1.0 if mistake in ("grad_missing_1_over_n", "sum_not_mean_logp") else float(n[sl])
        w[sw] += np.where(kp[sw], g * dr_daw * (-1.0 / nw), 0.0)
        w[sl] += np.where(kp[sl], g * dr_dal * (-1.0 / nl), 0.0)
    loss = nll + scale * or_sum
    if loss_only:
        return loss
    P = np.exp(Z - lse[:, None])
    P[np.arange(len(y))[keep], yy[keep]] -= 1.0
    P[~keep] = 0.0
    G = P * w.reshape(-1)[:, None]
    return {"loss": loss, "dX": G @ W, "dW": G.T @ X, "seq_logp": a}


def _case(seed, n_seq=4, T=3, H=4, V=6, n_ignore=2):
    r = np.random.default_rng(seed)
    X = r.standard_normal((n_seq * T, H))
    W = r.standard_normal((V, H)) * 0.5
    y = r.integers(0, V, n_seq * T)
    y[r.choice(n_seq * T, n_ignore, replace=False)] = IGN
    return X, W, y


def pin_two_class(f):
    c = np.array([1.3, -0.4, 0.2, 2.0, 0.7, -1.1])
    X = np.stack([c, np.zeros_like(c)], axis=1)
    W = np.array([[0.0, 0.0], [1.0, 0.0]])
    y = np.ones(6, dtype=np.int64)
    beta = 0.25
    out = f(X, W, y, 6, beta)
    nll = sum(_softplus(-c[p]) for p in range(3)) / 3
    orr = sum(_softplus(-(c[p] - c[3 + p])) for p in range(3)) / 3
    assert abs(out["loss"] - (nll + beta * orr)) <= 1e-12 * (nll + beta * orr)
    assert np.allclose(out["seq_logp"], [-_softplus(-v) for v in c], rtol=1e-12, atol=0)
    # every token twice plus one ignored token per sequence: means over the
    # valid tokens are unchanged, so the same closed form holds
    X3 = np.repeat(X, 3, axis=0)
    y3 = np.tile(np.array([1, 1, IGN]), 6)
    out3 = f(X3, W, y3, 6, beta)
    assert abs(out3["loss"] - (nll + beta * orr)) <= 1e-12 * (nll + beta * orr)
    assert np.allclose(out3["seq_logp"], [-_softplus(-v) for v in c], rtol=1e-12, atol=0)


def pin_beta_zero(f):
    X, W, y = _case(61)
    out = f(X, W, y, 4, 0.0)
    half = X.shape[0] // 2
    ref = oracle.flce_ref(X[:half], W, y[:half], IGN)
    assert abs(out["loss"] - ref["loss"]) <= 1e-12 * ref["loss"]
    assert np.max(np.abs(out["dW"] - ref["dW"])) <= 1e-12 * np.max(np.abs(ref["dW"]))
    assert np.all(out["dX"][half:] == 0.0)


def pin_identical_halves(f):
    Xh, W, yh = _case(62, n_seq=2, T=4)
    X = np.concatenate([Xh, Xh])
    y = np.concatenate([yh, yh])
    beta = 0.3
    out = f(X, W, y, 4, beta)
    ref = oracle.flce_ref(Xh, W, yh, IGN)
    assert abs(out["loss"] - (ref["loss"] + beta * math.log(2))) <= 1e-12
    assert np.max(np.abs(out["dW"] - ref["dW"])) <= 1e-12 * np.max(np.abs(ref["dW"]))


def pin_finite_differences(f, loss_fn):
    X, W, y = _case(63, n_seq=6, T=3, H=3, V=5, n_ignore=1)
    y[15:18] = IGN
    beta = 0.7
    out = f(X, W, y, 6, beta)
    assert abs(out["loss"] - loss_fn(X, W, y, 6, beta)) <= 1e-12 * abs(out["loss"])
    h = 1e-6
    for name, A in (("dX", X), ("dW", W)):
        num = np.zeros_like(A)
        for i in range(A.shape[0]):
            for j in range(A.shape[1]):
                P, M = A.copy(), A.copy()
                P[i, j] += h
                M[i, j] -= h
                if name == "dX":
                    num[i, j] = (loss_fn(P, W, y, 6, beta) - loss_fn(M, W, y, 6, beta)) / (2 * h)
                else:
                    num[i, j] = (loss_fn(X, P, y, 6, beta) - loss_fn(X, M, y, 6, beta)) / (2 * h)
        err = float(np.max(np.abs(out[name] - num))) / float(np.max(np.abs(num)))
        assert err <= 1e-6, (name, err)


def _pins(f, loss_fn):
    return [
        ("two_class", lambda: pin_two_class(f)),
        ("beta_zero", lambda: pin_beta_zero(f)),
        ("identical_halves", lambda: pin_identical_halves(f)),
        ("finite_differences", lambda: pin_finite_differences(f, loss_fn)),
    ]


MISTAKES = [
    "r_sign",
    "no_log1m",
    "nll_all_sequences",
    "beta_not_over_B",
    "sum_not_mean_logp",
    "grad_missing_1_over_n",
    "grad_wrong_sign_rejected",
    "softplus_positive",
]


def test_oracle_passes_the_pins():
    # the oracle itself, through the same pins
    f = lambda X, W, y, n, b: orpo_ref(X, W, y, n_seq=n, beta=b)  # noqa: E731
    for _, pin in _pins(f, lambda X, W, y, n, b: oracle.orpo_loss_only(X, W, y, n, b)):
        pin()


def test_unmutated_copy_passes_the_pins():
    f = lambda X, W, y, n, b: _orpo(X, W, y, n, b)  # noqa: E731
    for _, pin in _pins(f, lambda X, W, y, n, b: _orpo(X, W, y, n, b, loss_only=True)):
        pin()


@pytest.mark.parametrize("mistake", MISTAKES)
def test_pins_catch_planted_mistake(mistake):
    f = lambda X, W, y, n, b: _orpo(X, W, y, n, b, mistake)  # noqa: E731
    lf = lambda X, W, y, n, b: _orpo(X, W, y, n, b, mistake, loss_only=True)  # noqa: E731
    caught = []
    for name, pin in _pins(f, lf):
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, FloatingPointError, OverflowError):
            caught.append(name)
    assert caught, f"no pin catches the planted mistake {mistake!r}"
