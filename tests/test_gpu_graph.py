"""The library's calls inside a captured HIP graph (torch.cuda.CUDAGraph):
every replay must reproduce the eager call bit for bit.  The library only
launches kernels on the caller's stream (no allocation, no memset), which is
what makes it capturable; between replays the outputs are overwritten with
NaN by eager work, so each replay has to write all of them again."""
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


def _outs(X, W):
    dev = X.device
    return (torch.empty((), dtype=torch.float32, device=dev), torch.empty_like(X),
            torch.empty((W.shape[0], W.shape[1]), dtype=torch.float32, device=dev),
            torch.empty((1,), dtype=torch.int32, device=dev))


def test_fwd_bwd_replays_in_a_graph():
    import linear_cross_entropy_05_amd as flce

    w = si.small(700, 200, 1000, "bf16", seed=31, w_std=0.05)
    X, W, y = si.make_inputs(w)
    dev = torch.device("cuda", 0)
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    chunk = 256  # three chunks: the dW read-modify-write and the ragged last chunk are in the graph
    need = flce.flce_workspace_bytes(w.BT, w.H, w.V, chunk, Xd.dtype)
    ref = _outs(Xd, Wd)
    flce.flce_fwd_bwd(Xd, Wd, yd, w.ignore_index, chunk, out=ref,
                      workspace=torch.empty((need,), dtype=torch.uint8, device=dev), check=True)
    out = _outs(Xd, Wd)
    ws = torch.empty((need,), dtype=torch.uint8, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the side stream, as torch recommends before capture
        flce.flce_fwd_bwd(Xd, Wd, yd, w.ignore_index, chunk, out=out, workspace=ws, check=False)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        flce.flce_fwd_bwd(Xd, Wd, yd, w.ignore_index, chunk, out=out, workspace=ws, check=False)
    for r in range(4):
        for t in out[:3]:
            t.fill_(float("nan"))
        out[3].fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"  replay {r}: loss {out[0].item():.7f} (eager {ref[0].item():.7f})")
        assert int(out[3].item()) == 0
        for a, b in zip(out[:3], ref[:3]):
            assert torch.equal(a, b)


def test_ce_inplace_replays_in_a_graph():
    import linear_cross_entropy_05_amd as flce

    dev = torch.device("cuda", 0)
    g0 = torch.Generator().manual_seed(32)
    BT, V = 37, 50257
    logits0 = (torch.randn(BT, V, generator=g0) * 3).to(dev)
    y = torch.randint(0, V, (BT,), generator=g0).to(dev)
    y[5] = -100
    ref_logits = logits0.clone()
    ref_loss = flce.ce_fwd_bwd_inplace(ref_logits, y, check=True).clone()
    buf = logits0.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        flce.ce_fwd_bwd_inplace(buf, y, check=False)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    buf.copy_(logits0)
    with torch.cuda.graph(g):
        loss = flce.ce_fwd_bwd_inplace(buf, y, check=False)
    for r in range(3):
        buf.copy_(logits0)  # eager work between replays: fresh logits
        loss.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"  replay {r}: loss {loss.item():.7f} (eager {ref_loss.item():.7f})")
        assert torch.equal(loss, ref_loss)
        assert torch.equal(buf, ref_logits)
