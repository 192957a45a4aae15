"""The ORPO oracle against closed forms and finite differences (CPU only)."""
import math

import numpy as np

from oracle.orpo_oracle import orpo_loss_only, orpo_ref
import oracle

IGN = -100


def test_two_class_closed_form():
    """V = 2, one token per sequence, logits (0, c): P = sigmoid(c), so the
    sequence log odds are exactly c and r = c_w - c_l."""
    c = np.array([1.3, -0.4, 0.2, 2.0, 0.7, -1.1])  # B = 3 pairs: chosen 0..2, rejected 3..5
    X = np.stack([c, np.zeros_like(c)], axis=1)     # x_i = (c_i, 0)
    W = np.array([[0.0, 0.0], [1.0, 0.0]])          # logits (0, c_i)
    y = np.ones(6, dtype=np.int64)
    beta = 0.25
    out = orpo_ref(X, W, y, n_seq=6, beta=beta)
    sp = lambda x: math.log1p(math.exp(-abs(x))) + max(x, 0.0)  # noqa: E731
    nll = sum(sp(-c[p]) for p in range(3)) / 3                 # -log sigmoid(c) = softplus(-c)
    orr = sum(sp(-(c[p] - c[3 + p])) for p in range(3)) / 3
    expect = nll + beta * orr
    assert abs(out["loss"] - expect) <= 1e-14 * expect, (out["loss"], expect)
    assert np.allclose(out["seq_logp"], [-sp(-v) for v in c], rtol=1e-14, atol=0)


def test_two_class_repeated_tokens():
    """The same closed form with every token repeated and an ignored token
    added to each sequence: sequence scores are means over the valid tokens
    and the NLL a mean over the chosen valid tokens, so nothing changes (a
    sum in place of either mean would)."""
    c = np.array([1.3, -0.4, 0.2, 2.0, 0.7, -1.1])
    X = np.repeat(np.stack([c, np.zeros_like(c)], axis=1), 3, axis=0)
    W = np.array([[0.0, 0.0], [1.0, 0.0]])
    y = np.tile(np.array([1, 1, IGN]), 6)
    beta = 0.25
    out = orpo_ref(X, W, y, n_seq=6, beta=beta)
    sp = lambda x: math.log1p(math.exp(-abs(x))) + max(x, 0.0)  # noqa: E731
    expect = sum(sp(-c[p]) for p in range(3)) / 3 + beta * sum(sp(-(c[p] - c[3 + p])) for p in range(3)) / 3
    assert abs(out["loss"] - expect) <= 1e-14 * expect, (out["loss"], expect)
    assert np.allclose(out["seq_logp"], [-sp(-v) for v in c], rtol=1e-14, atol=0)


def test_two_class_near_certain_chosen():
    """The two-class closed form where one chosen sequence is near certain
    (logit 20: a = log sigmoid(20) ~ -2e-9), the regime where log(1 - e^a)
    is steep.  Loss and the per-token factors dL/dl_i against closed forms:
    with one token per sequence e^{a_s} = sigmoid(c_s), r_p = c_w - c_l and
    dL/dl_w = 1/B + beta/B sigmoid(-r_p) / sigmoid(-c_w),
    dL/dl_l = -beta/B sigmoid(-r_p) / sigmoid(-c_l)."""
    c = np.array([20.0, -0.4, 2.0, 0.7])  # B = 2: chosen 0, 1; rejected 2, 3
    X = np.stack([c, np.zeros_like(c)], axis=1)
    W = np.array([[0.0, 0.0], [1.0, 0.0]])
    y = np.ones(4, dtype=np.int64)
    beta = 0.5
    out = orpo_ref(X, W, y, n_seq=4, beta=beta)
    sp = lambda x: math.log1p(math.exp(-abs(x))) + max(x, 0.0)  # noqa: E731
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))  # noqa: E731
    r = [c[0] - c[2], c[1] - c[3]]
    expect = (sp(-c[0]) + sp(-c[1])) / 2 + beta * (sp(-r[0]) + sp(-r[1])) / 2
    assert abs(out["loss"] - expect) <= 1e-12 * expect, (out["loss"], expect)
    w = [1 / 2 + beta / 2 * sig(-r[p]) / sig(-c[p]) for p in range(2)]
    w += [-beta / 2 * sig(-r[p]) / sig(-c[2 + p]) for p in range(2)]
    # a_w is resolved to ~1e-6 relative in float64 (lse - z at |z| = 20)
    assert np.allclose(out["weights"], w, rtol=1e-5, atol=0), (out["weights"], w)


def _case(seed, n_seq=4, T=3, H=4, V=6, n_ignore=2):
    r = np.random.default_rng(seed)
    X = r.standard_normal((n_seq * T, H))
    W = r.standard_normal((V, H)) * 0.5
    y = r.integers(0, V, n_seq * T)
    y[r.choice(n_seq * T, n_ignore, replace=False)] = IGN
    return X, W, y


def test_beta_zero_is_chosen_cross_entropy():
    X, W, y = _case(61)
    out = orpo_ref(X, W, y, n_seq=4, beta=0.0)
    half = X.shape[0] // 2
    ref = oracle.flce_ref(X[:half], W, y[:half], IGN)
    assert abs(out["loss"] - ref["loss"]) <= 1e-14 * ref["loss"]
    assert np.max(np.abs(out["dW"] - ref["dW"])) <= 1e-14 * np.max(np.abs(ref["dW"]))
    assert np.max(np.abs(out["dX"][:half] - ref["dX"])) <= 1e-14 * np.max(np.abs(ref["dX"]))
    assert np.all(out["dX"][half:] == 0.0)


def test_identical_halves_give_log_two():
    """Chosen == rejected: every log odds ratio is 0, the odds-ratio term is
    beta log 2, and its dW contributions cancel between the two halves."""
    Xh, W, yh = _case(62, n_seq=2, T=4)
    X = np.concatenate([Xh, Xh])
    y = np.concatenate([yh, yh])
    beta = 0.3
    out = orpo_ref(X, W, y, n_seq=4, beta=beta)
    ref = oracle.flce_ref(Xh, W, yh, IGN)
    assert abs(out["loss"] - (ref["loss"] + beta * math.log(2))) <= 1e-13
    assert np.max(np.abs(out["dW"] - ref["dW"])) <= 1e-13 * np.max(np.abs(ref["dW"]))


def test_finite_differences():
    """dX and dW are the central differences of the loss (written from the
    logits directly, not through the gradient code), including a pair whose
    rejected sequence has no valid token."""
    X, W, y = _case(63, n_seq=6, T=3, H=3, V=5, n_ignore=1)
    y[5 * 3:6 * 3] = IGN  # sequence 5 (rejected of pair 2) fully ignored
    beta = 0.7
    out = orpo_ref(X, W, y, n_seq=6, beta=beta)
    assert abs(out["loss"] - orpo_loss_only(X, W, y, 6, beta)) <= 1e-14 * out["loss"]
    h = 1e-6
    for name, A in (("dX", X), ("dW", W)):
        num = np.zeros_like(A)
        for i in range(A.shape[0]):
            for j in range(A.shape[1]):
                P, M = A.copy(), A.copy()
                P[i, j] += h
                M[i, j] -= h
                if name == "dX":
                    num[i, j] = (orpo_loss_only(P, W, y, 6, beta) - orpo_loss_only(M, W, y, 6, beta)) / (2 * h)
                else:
                    num[i, j] = (orpo_loss_only(X, P, y, 6, beta) - orpo_loss_only(X, M, y, 6, beta)) / (2 * h)
        err = float(np.max(np.abs(out[name] - num))) / float(np.max(np.abs(num)))
        assert err <= 1e-7, (name, err)
