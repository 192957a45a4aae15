"""Calls on two streams at once: every piece of per-call state (statistics,
chunk buffer, tile-queue counters, valid-token count) lives in the caller's
workspace, so concurrent calls with their own workspaces must give exactly the
results they give one at a time."""
import pytest
import torch

import synth_inputs as si
from gpu_helpers import ensure_built, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return ensure_built()


def _inputs(BT, H, V, seed):
    w = si.small(BT, H, V, "bf16", seed=seed, w_std=0.05)
    X, W, y = si.make_inputs(w)
    dev = torch.device("cuda", 0)
    return w, X.to(dev), W.to(dev), y.to(dev)


def test_fwd_bwd_on_two_streams_matches_one_at_a_time():
    import linear_cross_entropy_05_amd as flce

    w1, X1, W1, y1 = _inputs(1536, 512, 20000, 81)
    w2, X2, W2, y2 = _inputs(1280, 768, 15000, 82)
    ref1 = flce.flce_fwd_bwd(X1, W1, y1, w1.ignore_index, 512)
    ref2 = flce.flce_fwd_bwd(X2, W2, y2, w2.ignore_index, 384)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(4):
        say(f"[gpu] two streams, repetition {rep}")
        torch.cuda.synchronize()
        with torch.cuda.stream(sa):
            o1 = flce.flce_fwd_bwd(X1, W1, y1, w1.ignore_index, 512, check=False)
        with torch.cuda.stream(sb):
            o2 = flce.flce_fwd_bwd(X2, W2, y2, w2.ignore_index, 384, check=False)
        torch.cuda.synchronize()
        for got, ref in ((o1, ref1), (o2, ref2)):
            assert torch.equal(got[0], ref[0])
            assert torch.equal(got[1], ref[1]) and torch.equal(got[2], ref[2])


def test_logits_ce_on_two_streams_matches_one_at_a_time():
    import linear_cross_entropy_05_amd as flce

    dev = torch.device("cuda", 0)
    g = torch.Generator().manual_seed(83)
    a = (torch.randn(300, 40000, generator=g) * 2).to(dev)
    b = (torch.randn(200, 50257, generator=g) * 2).to(dev)
    ya = torch.randint(0, 40000, (300,), generator=g).to(dev)
    yb = torch.randint(0, 50257, (200,), generator=g).to(dev)
    ra, rb = a.clone(), b.clone()
    la = flce.ce_fwd_bwd_inplace(ra, ya)
    lb = flce.ce_fwd_bwd_inplace(rb, yb)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    ga, gb = a.clone(), b.clone()
    torch.cuda.synchronize()
    with torch.cuda.stream(sa):
        l1 = flce.ce_fwd_bwd_inplace(ga, ya, check=False)
    with torch.cuda.stream(sb):
        l2 = flce.ce_fwd_bwd_inplace(gb, yb, check=False)
    torch.cuda.synchronize()
    assert torch.equal(l1, la) and torch.equal(l2, lb)
    assert torch.equal(ga, ra) and torch.equal(gb, rb)
