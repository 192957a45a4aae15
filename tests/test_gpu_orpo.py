"""Fused-linear ORPO (flce_orpo) on the GPU against the float64 ORPO oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_helpers import TOL, ensure_built, rel_err, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return ensure_built()


def _inputs(n_seq, T, H, V, dtype, seed, ignore_seq=None, w_std=0.05):
    w = si.small(n_seq * T, H, V, dtype, seed=seed, w_std=w_std)
    X, W, y = si.make_inputs(w)
    y = y.clone()
    if ignore_seq is not None:
        y[ignore_seq * T:(ignore_seq + 1) * T] = w.ignore_index
    return w, X, W, y


def _run(n_seq, T, H, V, dtype, seed, beta=0.1, chunk=0, ignore_seq=None):
    import linear_cross_entropy_05_amd as flce

    w, X, W, y = _inputs(n_seq, T, H, V, dtype, seed, ignore_seq)
    dev = torch.device("cuda", 0)
    say(f"[gpu] flce_orpo n_seq={n_seq} T={T} H={H} V={V} {dtype} beta={beta} chunk={chunk}")
    loss, dX, dW, sl = flce.flce_orpo(X.to(dev), W.to(dev), y.to(dev).view(n_seq, T), beta, w.ignore_index, chunk,
                                      seq_logp=True)
    torch.cuda.synchronize()
    ref = oracle.orpo_ref(X, W, y, n_seq, beta, w.ignore_index)
    tl, tg = TOL[dtype]
    el = abs(loss.item() - ref["loss"]) / abs(ref["loss"])
    es = rel_err(to_np(sl), ref["seq_logp"])
    ex, ew = rel_err(to_np(dX), ref["dX"]), rel_err(to_np(dW), ref["dW"])
    say(f"  loss {loss.item():.7f} ref {ref['loss']:.7f} err {el:.2e}; seq logp {es:.2e}; dX {ex:.2e}; dW {ew:.2e}")
    assert el <= tl and es <= tl and ex <= tg and ew <= tg
    return (X, W, y), (loss, dX, dW, sl), ref


def test_orpo_fp32_ragged():
    _run(4, 37, 64, 300, "fp32", seed=71)


def test_orpo_bf16_multi_tile():
    _run(6, 130, 200, 1000, "bf16", seed=72, beta=0.2)


def test_orpo_bf16_chunked_with_empty_sequence():
    # rejected sequence of pair 1 has no valid token; several token chunks
    _run(4, 160, 136, 700, "bf16", seed=73, beta=0.5, chunk=200, ignore_seq=3)


def test_orpo_one_pass_several_chunks_ragged():
    # 5 pairs of 96-token sequences, chunks of 400 tokens: 2 pairs per chunk,
    # so three chunks, the last with one pair; the rejected sequence of pair 3
    # has no valid token
    _run(10, 96, 136, 700, "bf16", seed=77, beta=0.3, chunk=400, ignore_seq=8)


def test_orpo_one_pass_fp32_several_chunks():
    # 3 pairs, 2 per 160-token chunk
    _run(6, 40, 64, 300, "fp32", seed=78, chunk=160)


def test_orpo_one_and_two_pass_agree():
    """The same inputs through chunks of whole pairs (one pass) and through
    chunks too short for a pair (forward pass, sequence terms, fused pass)."""
    import linear_cross_entropy_05_amd as flce

    n_seq, T, H, V = 4, 60, 72, 500
    w, X, W, y = _inputs(n_seq, T, H, V, "fp32", seed=79)
    dev = torch.device("cuda", 0)
    args = (X.to(dev), W.to(dev), y.to(dev).view(n_seq, T), 0.2, w.ignore_index)
    one = flce.flce_orpo(*args, 0, seq_logp=True)    # a 240-token chunk holds both pairs
    two = flce.flce_orpo(*args, 100, seq_logp=True)  # a pair needs 120 tokens
    torch.cuda.synchronize()
    assert flce.flce_orpo_workspace_bytes(n_seq, T, H, V, 0, torch.float32) != \
        flce.flce_orpo_workspace_bytes(n_seq, T, H, V, 100, torch.float32)
    assert abs(one[0].item() - two[0].item()) <= 1e-6 * abs(two[0].item())
    assert torch.equal(one[3], two[3])  # sequence scores from the same token losses, same order
    assert rel_err(to_np(one[1]), to_np(two[1])) <= 1e-5 and rel_err(to_np(one[2]), to_np(two[2])) <= 1e-5


def test_orpo_beta_zero_is_chosen_cross_entropy():
    import linear_cross_entropy_05_amd as flce

    n_seq, T, H, V = 4, 64, 128, 500
    w, X, W, y = _inputs(n_seq, T, H, V, "fp32", seed=74)
    dev = torch.device("cuda", 0)
    loss, dX, dW = flce.flce_orpo(X.to(dev), W.to(dev), y.to(dev).view(n_seq, T), 0.0, w.ignore_index)
    half = n_seq * T // 2
    l2, dX2, dW2 = flce.flce_fwd_bwd(X[:half].to(dev), W.to(dev), y[:half].to(dev), w.ignore_index)
    torch.cuda.synchronize()
    assert abs(loss.item() - l2.item()) <= 1e-6 * abs(l2.item())
    assert torch.equal(dX[:half], dX2) and float(dX[half:].abs().max()) == 0.0
    assert rel_err(to_np(dW), to_np(dW2)) <= 1e-6


def test_orpo_module_autograd():
    import linear_cross_entropy_05_amd as flce

    n_seq, T, H, V = 4, 50, 96, 400
    w, X, W, y = _inputs(n_seq, T, H, V, "bf16", seed=75)
    dev = torch.device("cuda", 0)
    Wg = W.to(dev).requires_grad_(True)
    Xg = X.to(dev).view(n_seq, T, H).clone().requires_grad_(True)
    mod = flce.FusedLinearORPOLoss(ignore_index=w.ignore_index, beta=0.1)
    loss = mod(Wg, Xg, y.to(dev).view(n_seq, T))
    (2.0 * loss).backward()
    torch.cuda.synchronize()
    ref = oracle.orpo_ref(X, W, y, n_seq, 0.1, w.ignore_index)
    tl, tg = TOL["bf16"]
    assert abs(loss.item() - ref["loss"]) / ref["loss"] <= tl
    assert Xg.grad.shape == (n_seq, T, H) and Wg.grad.dtype == torch.bfloat16
    assert rel_err(to_np(Xg.grad).reshape(-1, H), 2.0 * ref["dX"]) <= tg
    assert rel_err(to_np(Wg.grad), 2.0 * ref["dW"]) <= tg


def test_orpo_near_certain_chosen_sequence():
    """A chosen sequence with one valid token whose target logit exceeds all
    others by 25: its loss in fp32 rounds to 0 (or just below), so its mean
    log-probability is 0 where the float64 oracle has ~-2e-10.  The odds term
    must stay finite and the results match the oracle (its limits as a -> 0
    are finite)."""
    import linear_cross_entropy_05_amd as flce

    n_seq, T, H, V = 4, 8, 8, 16
    w, X, W, y = _inputs(n_seq, T, H, V, "fp32", seed=76)
    t = int(y[0]) if int(y[0]) != w.ignore_index else 3
    y[0] = t
    y[1:T] = w.ignore_index               # sequence 0: one valid token
    X[0] = 0.0
    X[0, 0] = 25.0                        # x_0 = 25 e_0
    W[:, 0] = 0.0
    W[t, 0] = 1.0                         # z_{0,t} = 25, every other logit of token 0 is 0
    dev = torch.device("cuda", 0)
    say(f"[gpu] flce_orpo near-certain chosen sequence n_seq={n_seq} T={T} H={H} V={V} fp32")
    loss, dX, dW, sl = flce.flce_orpo(X.to(dev), W.to(dev), y.to(dev).view(n_seq, T), 0.1, w.ignore_index,
                                      seq_logp=True)
    torch.cuda.synchronize()
    ref = oracle.orpo_ref(X, W, y, n_seq, 0.1, w.ignore_index)
    assert -1e-9 < ref["seq_logp"][0] < 0.0  # float64 resolves the near-certain score
    assert bool(torch.isfinite(loss)) and bool(torch.isfinite(dX).all()) and bool(torch.isfinite(dW).all())
    tl, tg = TOL["fp32"]
    el = abs(loss.item() - ref["loss"]) / abs(ref["loss"])
    ex, ew = rel_err(to_np(dX), ref["dX"]), rel_err(to_np(dW), ref["dW"])
    say(f"  loss {loss.item():.7f} ref {ref['loss']:.7f} err {el:.2e}; dX {ex:.2e}; dW {ew:.2e}; "
        f"a_0 gpu {float(sl[0]):.3e} ref {ref['seq_logp'][0]:.3e}")
    assert el <= tl and ex <= tg and ew <= tg
