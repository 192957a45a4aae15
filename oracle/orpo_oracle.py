"""CPU oracle for the chunked fused-linear ORPO loss (odds-ratio preference loss).

TEST INFRASTRUCTURE ONLY, like ``flce_oracle``: nothing on the product path
imports or calls it, and it shares no code with the HIP library.

What the pages fix
------------------
"Liger-Kernel 項目詳細介紹" (aibars.net) lists ``LigerFusedLinearORPOLoss`` among
the post-training losses (section 主要功能, ORPO 損失) and, in section 使用方法,
item 4 (後訓練損失使用示例), shows the call ``orpo_loss(lm_head.weight, x,
target)``: the LM-head weight first, then hidden states and targets, exactly
like the fused linear cross-entropy.  The pages give no formula.

Reading (the published ORPO objective, restated here, as the plainest reading
of "ORPO loss" on top of the same LM head):

* The batch holds 2B sequences of T tokens: sequences 0..B-1 are the chosen
  responses, B..2B-1 the rejected ones, pair p = (p, B + p).  Hidden states
  X [2B*T, H] row-major (sequence-major), targets y [2B*T], ignore_index as in
  the cross-entropy.
* Token log-probability logp_i = -(lse_i - Z_{i, y_i}) with Z = X W^T; the
  sequence score is the mean log-probability over its non-ignored tokens,
  a_s = (1/n_s) sum_{i in s, valid} logp_i.
* Log odds of a sequence: log(P / (1 - P)) with P = exp(a_s), i.e.
  a_s - log(1 - exp(a_s)); the pair's log odds ratio is
  r_p = (a_w - a_l) - (log(1 - e^{a_w}) - log(1 - e^{a_l})).
* loss = NLL + beta * (1/B) * sum_p softplus(-r_p), where NLL is the mean
  token loss over the non-ignored tokens of the chosen sequences and
  softplus(-r) = -log sigmoid(r).
* A pair in which either sequence has no non-ignored token contributes 0 to
  the odds-ratio term (its score is undefined); N_chosen = 0 gives NLL = 0.

Gradients are the chain rule through the token losses: the loss depends on Z
only through l_i, so dL/dZ_i = (softmax_i - onehot_i) * w_i with
w_i = dL/dl_i, and dX = G W, dW = G^T X (``flce_oracle.flce_ref`` with
``token_scale = w``).  Pinned in ``tests/test_oracle_orpo.py`` by a two-class
closed form (also with every token repeated and an ignored token added, which
leaves means over valid tokens unchanged), beta = 0 (plain chosen-token
cross-entropy), identical chosen and rejected sequences (r = 0), and central
finite differences of the loss; ``tests/test_oracle_orpo_mutants.py`` checks
that these pins catch eight planted mistakes in a copy of the definition.
"""

from __future__ import annotations

import math

import numpy as np

from .flce_oracle import _as_f64, _as_i64, flce_ref


def _softplus(x: float) -> float:
    return max(x, 0.0) + math.log1p(math.exp(-abs(x)))


def _sigmoid(x: float) -> float:
    return 1.0 / (1.0 + math.exp(-x)) if x >= 0 else math.exp(x) / (1.0 + math.exp(x))


def orpo_terms(row_loss, y, n_seq: int, beta: float, ignore_index: int = -100):
    """Loss and per-token weights dL/dl_i from the token losses l_i.

    row_loss [2B*T] (0 on ignored tokens), y [2B*T].  Returns a dict with
    ``loss``, ``weights`` [2B*T] (0 on ignored tokens), ``seq_logp`` [2B]
    (a_s; 0 for a sequence without valid tokens), ``nll`` and ``or_term``.
    """
    rl = np.asarray(row_loss, dtype=np.float64)
    y = _as_i64(y)
    if n_seq < 2 or n_seq % 2 or rl.size % n_seq:
        raise ValueError("need an even number of sequences of equal length")
    T = rl.size // n_seq
    B = n_seq // 2
    keep = (y != ignore_index).reshape(n_seq, T)
    L = rl.reshape(n_seq, T)
    n = keep.sum(axis=1)
    a = np.where(n > 0, -np.where(keep, L, 0.0).sum(axis=1) / np.maximum(n, 1), 0.0)
    n_chosen = int(n[:B].sum())
    nll = float(np.where(keep[:B], L[:B], 0.0).sum() / max(n_chosen, 1))
    w = np.zeros((n_seq, T))
    w[:B] = np.where(keep[:B], 1.0 / max(n_chosen, 1), 0.0)
    or_sum = 0.0
    for p in range(B):
        sw, sl = p, B + p
        if n[sw] == 0 or n[sl] == 0:
            continue
        aw, al = a[sw], a[sl]
        # log(1 - e^a) with a <= 0, as log(-expm1(a))
        r = (aw - al) - (math.log(-math.expm1(aw)) - math.log(-math.expm1(al)))
        or_sum += _softplus(-r)
        g = -_sigmoid(-r) * beta / B  # d (beta/B softplus(-r)) / dr
        dr_daw = 1.0 / (-math.expm1(aw))
        dr_dal = -1.0 / (-math.expm1(al))
        # a_s = -(1/n_s) sum l_i: da_s/dl_i = -1/n_s
        w[sw] += np.where(keep[sw], g * dr_daw * (-1.0 / n[sw]), 0.0)
        w[sl] += np.where(keep[sl], g * dr_dal * (-1.0 / n[sl]), 0.0)
    or_term = beta * or_sum / B
    return {"loss": nll + or_term, "weights": w.reshape(-1), "seq_logp": a, "nll": nll, "or_term": or_term}


def orpo_ref(X, W, y, n_seq: int, beta: float = 0.1, ignore_index: int = -100):
    """ORPO loss and gradients by the definition above, in float64.

    Returns ``loss``, ``dX`` [2B*T, H], ``dW`` [V, H], ``seq_logp`` [2B],
    ``nll``, ``or_term`` and the per-token ``weights``.
    """
    base = flce_ref(X, W, y, ignore_index)  # token losses l_i (gradients unused)
    t = orpo_terms(base["row_loss"], y, n_seq, beta, ignore_index)
    g = flce_ref(X, W, y, ignore_index, token_scale=t["weights"])
    return {"loss": t["loss"], "dX": g["dX"], "dW": g["dW"], "seq_logp": t["seq_logp"], "nll": t["nll"],
            "or_term": t["or_term"], "weights": t["weights"], "row_loss": base["row_loss"]}


def orpo_loss_only(X, W, y, n_seq: int, beta: float = 0.1, ignore_index: int = -100) -> float:
    """The loss alone (for finite differences)."""
    Z = _as_f64(X) @ _as_f64(W).T
    y = _as_i64(y)
    m = Z.max(axis=1)
    lse = m + np.log(np.exp(Z - m[:, None]).sum(axis=1))
    keep = y != ignore_index
    rl = np.where(keep, lse - Z[np.arange(len(y)), np.where(keep, y, 0)], 0.0)
    return orpo_terms(rl, y, n_seq, beta, ignore_index)["loss"]
