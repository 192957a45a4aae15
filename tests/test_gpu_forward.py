"""Forward-only FLCE (flce_fwd) on the GPU: against the float64 oracle, and
bitwise against the loss of the forward+backward call on the same inputs
(both take the same logits, statistics and reductions; only the chunk
buffer and the backward products are left out)."""
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


def _dev(*ts):
    dev = torch.device("cuda", 0)
    return [t.to(dev) for t in ts]


def forward_vs_oracle(w, chunk_tokens=0):
    import linear_cross_entropy_05_amd as flce

    X, W, y = si.make_inputs(w)
    Xd, Wd, yd = _dev(X, W, y)
    say(f"[gpu] flce_forward {w.name} BT={w.BT} H={w.H} V={w.V} {w.dtype} chunk={chunk_tokens}")
    loss, rl = flce.flce_forward(Xd, Wd, yd, w.ignore_index, chunk_tokens, row_loss=True)
    torch.cuda.synchronize()
    ref = oracle.flce_ref(X, W, y, w.ignore_index)
    tl, _ = TOL[w.dtype]
    el = abs(loss.item() - ref["loss"]) / max(abs(ref["loss"]), 1e-30)
    er = rel_err(to_np(rl), ref["row_loss"])
    say(f"  loss {loss.item():.7f} ref {ref['loss']:.7f} err {el:.2e}; token losses {er:.2e}")
    assert el <= tl and er <= tl
    return loss, rl


def test_tiny_fp32_forward():
    forward_vs_oracle(si.workload("tiny"))


@pytest.mark.parametrize("chunk", [1, 3, 5])
def test_tiny_fp32_forward_chunks(chunk):
    forward_vs_oracle(si.workload("tiny"), chunk)


def test_fp32_ragged_forward():
    forward_vs_oracle(si.small(700, 200, 1000, "fp32", seed=21, w_std=0.05), 256)


def test_bf16_ragged_forward():
    forward_vs_oracle(si.small(700, 200, 1000, "bf16", seed=22, w_std=0.05))


def test_bf16_large_logits_forward():
    forward_vs_oracle(si.small(512, 768, 3000, "bf16", seed=24, x_scale=3.0, w_std=0.04))


@pytest.mark.parametrize("dtype,chunk_fwd,chunk_bwd", [("fp32", 0, 256), ("bf16", 0, 256), ("bf16", 300, 0),
                                                       ("bf16", 1, 700)])
def test_forward_equals_fwd_bwd_loss_bitwise(dtype, chunk_fwd, chunk_bwd):
    """Per-token losses do not depend on the chunking, so the two entry points
    agree to the bit for any pair of chunk sizes."""
    import linear_cross_entropy_05_amd as flce

    w = si.small(700, 200, 1000, dtype, seed=31, w_std=0.05)
    Xd, Wd, yd = _dev(*si.make_inputs(w))
    lf, rf = flce.flce_forward(Xd, Wd, yd, w.ignore_index, chunk_fwd, row_loss=True)
    lb, _, _, rb = flce.flce_fwd_bwd(Xd, Wd, yd, w.ignore_index, chunk_bwd, row_loss=True)
    torch.cuda.synchronize()
    say(f"  forward {lf.item():.9f} fwd+bwd {lb.item():.9f}")
    assert torch.equal(rf, rb)
    assert torch.equal(lf, lb)


def test_forward_mistral_head_full_size():
    """Mistral/Llama-2 head (2048 x 2048 x 32000, bf16): loss and every token
    loss against the oracle."""
    forward_vs_oracle(si.workload("mistral"))


def test_forward_edge_cases():
    import linear_cross_entropy_05_amd as flce

    w = si.small(40, 64, 300, "bf16", seed=32)
    X, W, y = si.make_inputs(w)
    Xd, Wd, yd = _dev(X, W, y)
    # every target ignored: loss 0, token losses 0
    allign = torch.full_like(yd, w.ignore_index)
    loss, rl = flce.flce_forward(Xd, Wd, allign, w.ignore_index, row_loss=True)
    assert loss.item() == 0.0 and float(rl.abs().max()) == 0.0
    # empty batch
    loss = flce.flce_forward(Xd[:0], Wd, yd[:0], w.ignore_index)
    assert loss.item() == 0.0
    # a target outside [0, V) that is not ignore_index is reported
    bad = yd.clone()
    bad[5] = w.V
    with pytest.raises(flce.FlceError):
        flce.flce_forward(Xd, Wd, bad, w.ignore_index)


def test_module_no_grad_uses_forward_path():
    """Under torch.no_grad the module returns the forward-only loss, which
    equals the training-mode loss to the bit."""
    import linear_cross_entropy_05_amd as flce

    w = si.small(300, 128, 700, "bf16", seed=33)
    Xd, Wd, yd = _dev(*si.make_inputs(w))
    mod = flce.FusedLinearCrossEntropyLoss(ignore_index=w.ignore_index)
    with torch.no_grad():
        l0 = mod(Wd, Xd, yd)
    Wg = Wd.clone().requires_grad_(True)
    l1 = mod(Wg, Xd, yd)
    torch.cuda.synchronize()
    assert not l0.requires_grad and l1.requires_grad
    assert torch.equal(l0, l1.detach())
    ref = oracle.flce_ref(*si.make_inputs(w), w.ignore_index)
    assert abs(l0.item() - ref["loss"]) / ref["loss"] <= TOL["bf16"][0]
