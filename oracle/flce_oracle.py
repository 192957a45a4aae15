"""CPU oracle for fused linear + cross-entropy (FLCE) and logits-only cross-entropy.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.  It shares
no code, constant or helper with the HIP library; its inputs come from the
seeded generator module ``synth_inputs`` (which computes nothing of the method)
or from the tests themselves.

What it computes
----------------
The Liger-Kernel pages describe the method only in words:

* "[論文レビュー] Liger Kernel: Efficient Triton Kernels for LLM Training"
  (nubint.ai), section 提案手法: a chunked fused Linear+CrossEntropy (FLCE)
  that avoids holding the large-vocabulary logits; section 主な発見: the
  CrossEntropy kernel uses an online softmax and replaces the logits by their
  gradient in place.
* "Liger-Kernel 項目詳細介紹" (aibars.net), section 技術實現: the computation is
  exact (no approximation) and forward and backward are unit-tested; section
  使用方法, item 3 (低級 API): the call is ``loss_fn(weight, input, target)``
  with ``weight`` an ``nn.Linear(H, V).weight`` of shape [V, H], ``input``
  [BT, H] and integer ``target`` [BT], followed by ``loss.backward()``.

Because the method is exact, chunking, online softmax and in-place gradients
only reorder the same arithmetic.  The oracle is therefore the plain textbook
definition of mean softmax cross-entropy of the projected logits, evaluated in
float64 with the full BT x V logits materialised:

    Z      = X W^T                                  [BT, V]
    lse_i  = m_i + ln sum_v exp(Z_iv - m_i),  m_i = max_v Z_iv
    l_i    = lse_i - Z_{i, y_i}          for rows with y_i != ignore_index
    N      = #{i : y_i != ignore_index}
    loss   = sum_i l_i / N
    G_iv   = (exp(Z_iv - lse_i) - [v == y_i]) / N  (0 for ignored rows)
    dX     = G W,   dW = G^T X

Readings where the pages are silent:
the reduction is the mean over non-ignored tokens of the whole call; no bias
term (the usage example passes only ``model.weight``); N = 0 gives loss 0 and
zero gradients; a valid target outside [0, V) is an error, never clamped;
inputs are upcast exactly to float64 before any arithmetic.

Every function is pinned by tests under ``tests/test_oracle.py`` against
closed forms, invariants, finite differences, a pure-Python brute force and
an independent library routine (torch CPU float64 ``cross_entropy``).
"""

from __future__ import annotations

import numpy as np


def _as_f64(a) -> np.ndarray:
    """Exact upcast to float64 (bf16/fp32 values are all representable)."""
    if hasattr(a, "detach"):  # torch tensor: go through float32, which holds bf16 exactly
        a = a.detach().cpu()
        if a.dtype.is_floating_point:
            a = a.float()
        a = a.numpy()
    return np.asarray(a, dtype=np.float64)


def _as_i64(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.asarray(a, dtype=np.int64)


def check_targets(y, V: int, ignore_index: int = -100) -> None:
    """Raise ValueError if a non-ignored target lies outside [0, V)."""
    y = _as_i64(y)
    keep = y != ignore_index
    bad = keep & ((y < 0) | (y >= V))
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise ValueError(f"target {int(y[i])} at row {i} outside [0, {V})")


def row_lse(Z: np.ndarray) -> np.ndarray:
    """Row-wise log-sum-exp, shifted by the row maximum for range safety."""
    Z = _as_f64(Z)
    m = Z.max(axis=1, keepdims=True)
    return (m + np.log(np.exp(Z - m).sum(axis=1, keepdims=True)))[:, 0]


def ce_ref(logits, y, ignore_index: int = -100):
    """Mean softmax cross-entropy on given logits and its gradient.

    Oracle of the logits-only CrossEntropy kernel (nubint.ai review, 主な発見:
    online softmax with the gradient written over the logits).  Returns a dict
    with ``loss`` (float), ``dlogits`` [BT, V] float64 (what the in-place
    kernel leaves in the logits buffer), ``row_loss`` [BT] (0 on ignored rows),
    ``lse`` [BT] and ``n_valid``.
    """
    return _ce(np.array(_as_f64(logits), dtype=np.float64, copy=True), y, ignore_index)


def _ce(Z: np.ndarray, y, ignore_index: int, n_valid=None, token_scale=None):
    """ce_ref on a float64 logits array it overwrites (Z becomes dlogits).

    ``n_valid`` overrides N (the count of non-ignored rows) when Z holds only
    some rows of a larger batch.  ``token_scale`` [BT], when given, replaces
    the 1/N factor of each row's gradient: dlogits_i = (softmax_i - onehot_i)
    * token_scale[i], the gradient of sum_i token_scale[i] * loss_i (the loss
    itself stays the mean).
    """
    y = _as_i64(y)
    BT, V = Z.shape
    check_targets(y, V, ignore_index)
    keep = y != ignore_index
    n = int(keep.sum()) if n_valid is None else int(n_valid)
    denom = float(max(n, 1))
    rows = np.arange(BT)
    z_target = Z[rows, np.where(keep, y, 0)].copy()
    # log-sum-exp shifted by the row maximum: Z <- exp(Z - m), s = row sums
    m = Z.max(axis=1) if BT else np.zeros(0)
    Z -= m[:, None]
    np.exp(Z, out=Z)
    s = Z.sum(axis=1)
    lse = m + np.log(s)
    row_loss = np.where(keep, lse - z_target, 0.0)
    loss = float(row_loss.sum() / denom)
    # softmax = exp(Z - m) / s; minus the one-hot target; over N; ignored rows 0
    Z /= s[:, None]
    Z[rows[keep], y[keep]] -= 1.0
    Z[~keep, :] = 0.0
    if token_scale is None:
        Z /= denom
    else:
        Z *= np.asarray(token_scale, dtype=np.float64).reshape(BT, 1)
    return {"loss": loss, "dlogits": Z, "row_loss": row_loss, "lse": lse, "n_valid": n}


def ce_rows_ref(logits_rows, y_rows, n_valid: int, ignore_index: int = -100):
    """ce_ref for a subset of rows of a larger batch whose N is ``n_valid``.

    Every row's loss term and gradient depend only on that row and on N, so
    selected rows can be checked one by one at sizes where the whole batch is
    too large for the CPU.  Returns ``row_loss``, ``lse`` and ``dlogits`` of
    those rows (the latter divided by the batch's N).
    """
    Z = np.array(_as_f64(logits_rows), dtype=np.float64, copy=True)
    out = _ce(Z, y_rows, ignore_index, n_valid=n_valid)
    out.pop("loss")
    return out


def flce_ref(X, W, y, ignore_index: int = -100, token_scale=None):
    """Fused linear + cross-entropy, forward and backward, by the plain definition.

    X [BT, H], W [V, H] (nn.Linear weight layout, no bias), y [BT] integer.
    Returns a dict with ``loss``, ``dX`` [BT, H], ``dW`` [V, H], ``row_loss``,
    ``lse``, ``n_valid`` and the full ``dlogits`` [BT, V], all float64.
    With ``token_scale`` [BT] the gradients are those of
    sum_i token_scale[i] * loss_i instead of the mean (see ``_ce``).
    """
    X64 = _as_f64(X)
    W64 = _as_f64(W)
    if X64.ndim != 2 or W64.ndim != 2 or X64.shape[1] != W64.shape[1]:
        raise ValueError(f"shape mismatch X{X64.shape} W{W64.shape}")
    Z = X64 @ W64.T
    ts = None if token_scale is None else _as_f64(token_scale)
    out = _ce(Z, y, ignore_index, token_scale=ts)  # Z is overwritten by dlogits
    G = out["dlogits"]
    out["dX"] = G @ W64
    out["dW"] = G.T @ X64
    return out


def flce_ref_rowblocks(X, W, y, ignore_index: int = -100, block: int = 1024):
    """``flce_ref`` for hosts without room for the whole BT x V logits.

    The same definition with the token axis cut into blocks of ``block``
    rows: each row's loss term and gradient row depend only on that row and
    on the batch's N, so block b's logits Z_b = X_b W^T, its gradient rows
    G_b and dX_b = G_b W are exactly those rows of the whole computation;
    dW = G^T X is the sum over blocks of G_b^T X_b (the product's sum over
    tokens, split).  Returns ``loss``, ``dX``, ``dW``, ``row_loss``, ``lse``
    and ``n_valid`` (no ``dlogits``), all float64.
    """
    X64 = _as_f64(X)
    W64 = _as_f64(W)
    y = _as_i64(y)
    if X64.ndim != 2 or W64.ndim != 2 or X64.shape[1] != W64.shape[1]:
        raise ValueError(f"shape mismatch X{X64.shape} W{W64.shape}")
    BT = X64.shape[0]
    check_targets(y, W64.shape[0], ignore_index)
    n = int((y != ignore_index).sum())
    dX = np.zeros_like(X64)
    dW = np.zeros_like(W64)
    row_loss = np.zeros(BT)
    lse = np.zeros(BT)
    for b in range(0, BT, block):
        e = min(b + block, BT)
        out = _ce(X64[b:e] @ W64.T, y[b:e], ignore_index, n_valid=n)
        G = out["dlogits"]
        dX[b:e] = G @ W64
        dW += G.T @ X64[b:e]
        row_loss[b:e] = out["row_loss"]
        lse[b:e] = out["lse"]
    loss = float(row_loss.sum() / max(n, 1))
    return {"loss": loss, "dX": dX, "dW": dW, "row_loss": row_loss, "lse": lse, "n_valid": n}


def flce_rows_ref(X, W, y, rows, n_valid: int, ignore_index: int = -100):
    """Per-row quantities for selected rows only, one row at a time.

    For full-size checks where the whole oracle would be too slow: row i's
    loss term, log-sum-exp and dX row depend only on row i (and on the batch's
    N, passed in as ``n_valid``), so each is computed from that row's own
    logits ``Z_i = W x_i``.  Returns dict of arrays indexed like ``rows``:
    ``row_loss`` [R], ``lse`` [R], ``dX`` [R, H].
    """
    W64 = _as_f64(W)
    y = _as_i64(y)
    V = W64.shape[0]
    denom = float(max(int(n_valid), 1))
    rows = [int(r) for r in rows]
    lse = np.zeros(len(rows))
    row_loss = np.zeros(len(rows))
    dX = np.zeros((len(rows), W64.shape[1]))
    for j, r in enumerate(rows):
        x = _as_f64(X[r])
        z = W64 @ x
        m = z.max()
        lse[j] = m + np.log(np.exp(z - m).sum())
        if int(y[r]) == ignore_index:
            continue
        t = int(y[r])
        if not 0 <= t < V:
            raise ValueError(f"target {t} at row {r} outside [0, {V})")
        row_loss[j] = lse[j] - z[t]
        g = np.exp(z - lse[j])
        g[t] -= 1.0
        dX[j] = (g / denom) @ W64
    return {"row_loss": row_loss, "lse": lse, "dX": dX}


def flce_brute_force(X, W, y, ignore_index: int = -100):
    """Pure-Python loops over Python floats, for tiny inputs only.

    Independent of NumPy's matmul/exp: every logit is an explicit dot product
    and every exponential goes through ``math.exp``.  Used to pin ``flce_ref``.
    """
    import math

    X = _as_f64(X).tolist()
    W = _as_f64(W).tolist()
    y = _as_i64(y).tolist()
    BT, V, H = len(X), len(W), len(W[0]) if W else 0
    n = sum(1 for t in y if t != ignore_index)
    denom = float(max(n, 1))
    dX = [[0.0] * H for _ in range(BT)]
    dW = [[0.0] * H for _ in range(V)]
    total = 0.0
    for i in range(BT):
        if y[i] == ignore_index:
            continue
        z = [math.fsum(X[i][h] * W[v][h] for h in range(H)) for v in range(V)]
        m = max(z)
        s = math.fsum(math.exp(zv - m) for zv in z)
        lse = m + math.log(s)
        total += lse - z[y[i]]
        for v in range(V):
            g = (math.exp(z[v] - lse) - (1.0 if v == y[i] else 0.0)) / denom
            for h in range(H):
                dX[i][h] += g * W[v][h]
                dW[v][h] += g * X[i][h]
    return {"loss": total / denom, "dX": np.array(dX), "dW": np.array(dW)}
