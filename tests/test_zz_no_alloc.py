"""ce_fwd_bwd_inplace_noalloc (static device scratch, no allocation) through
the C ABI against the workspace entry point ce_fwd_bwd_inplace on the same
inputs: two calls in a row, the second with fewer rows and a shorter
vocabulary, so the scratch still holds the first call's values when the
second starts.  The two entry points run the same kernels, so their results
must agree bit for bit (stronger than the fp32 bound); both are also held to
the float64 oracle at that bound."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL, ensure_built, rel_err, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return ensure_built()


def _logits(BT, V, seed):
    g = torch.Generator().manual_seed(seed)
    z = 3.0 * torch.randn(BT, V, generator=g, dtype=torch.float32)
    y = torch.randint(0, V, (BT,), generator=g, dtype=torch.int64)
    y[torch.randperm(BT, generator=g)[: BT // 10]] = -100
    return z, y


def test_noalloc_matches_workspace_entry_point():
    import linear_cross_entropy_05_amd as flce

    dev = torch.device("cuda", 0)
    cases = [(1000, 5000, 81, False), (300, 777, 82, True)]  # (BT, V, seed, caller's row_loss)
    for BT, V, seed, with_rows in cases:
        z, y = _logits(BT, V, seed)
        yd = y.to(dev)
        a = z.to(dev)
        b = z.to(dev)
        say(f"[gpu] ce_fwd_bwd_inplace_noalloc BT={BT} V={V} row_loss={'caller' if with_rows else 'scratch'}")
        la, rla = flce.ce_fwd_bwd_inplace(a, yd, -100, row_loss=True)
        loss_b = torch.empty((), dtype=torch.float32, device=dev)
        err_b = torch.full((1,), -1, dtype=torch.int32, device=dev)
        rlb = torch.empty((BT,), dtype=torch.float32, device=dev) if with_rows else None
        lb = flce.ce_fwd_bwd_inplace_noalloc(b, yd, -100, out=(loss_b, err_b), row_loss=rlb)
        torch.cuda.synchronize()
        assert int(err_b.item()) == 0
        assert torch.equal(a, b), "dlogits differ between the two entry points"
        assert la.item() == lb.item(), (la.item(), lb.item())
        if with_rows:
            assert torch.equal(rla, rlb)
        ref = oracle.ce_ref(z, y, -100)
        tl, tg = TOL["fp32"]
        el = abs(lb.item() - ref["loss"]) / abs(ref["loss"])
        ed = rel_err(to_np(b), ref["dlogits"])
        say(f"  loss {lb.item():.7f} (workspace entry {la.item():.7f}, oracle {ref['loss']:.7f}) err {el:.2e}; "
            f"dlogits {ed:.2e}")
        assert el <= tl and ed <= tg
        assert np.isfinite(to_np(b)).all()
