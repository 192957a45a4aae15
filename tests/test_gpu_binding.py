"""The Python binding's argument checks with device tensors (needs a GPU):
every case is rejected on the host, before any kernel launch."""
import pytest
import torch

import synth_inputs as si
from gpu_helpers import ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return ensure_built()


def _inputs():
    w = si.small(64, 128, 500, "bf16", seed=80)
    X, W, y = si.make_inputs(w)
    dev = torch.device("cuda", 0)
    return w, X.to(dev), W.to(dev), y.to(dev), dev


def test_outputs_of_the_wrong_shape_or_type_are_refused():
    import linear_cross_entropy_05_amd as flce

    w, X, W, y, dev = _inputs()
    good = (torch.empty((), dtype=torch.float32, device=dev), torch.empty_like(X),
            torch.empty((w.V, w.H), dtype=torch.float32, device=dev), torch.empty((1,), dtype=torch.int32, device=dev))
    bad = [
        (good[0], good[1], torch.empty((w.V - 1, w.H), dtype=torch.float32, device=dev), good[3]),  # short dW
        (good[0], good[1], torch.empty((w.V, w.H), dtype=torch.bfloat16, device=dev), good[3]),     # bf16 dW
        (good[0], torch.empty((w.BT, w.H), dtype=torch.float32, device=dev), good[2], good[3]),     # fp32 dX
        (good[0], good[1], torch.empty((w.H, w.V), dtype=torch.float32, device=dev).t(), good[3]),  # strided dW
        (good[0], good[1], good[2], torch.empty((2,), dtype=torch.int32, device=dev)),              # err shape
    ]
    for out in bad:
        with pytest.raises((ValueError, TypeError)):
            flce.flce_fwd_bwd(X, W, y, w.ignore_index, 0, out=out)
    loss, dX, dW = flce.flce_fwd_bwd(X, W, y, w.ignore_index, 0, out=good)
    assert torch.isfinite(loss).item()


def test_small_workspace_and_host_operands_are_refused():
    import linear_cross_entropy_05_amd as flce

    w, X, W, y, dev = _inputs()
    need = flce.flce_workspace_bytes(w.BT, w.H, w.V, 0, X.dtype)
    with pytest.raises(flce.FlceError):
        flce.flce_fwd_bwd(X, W, y, w.ignore_index, 0, workspace=torch.empty((need - 256,), dtype=torch.uint8,
                                                                               device=dev))
    with pytest.raises(ValueError):
        flce.flce_fwd_bwd(X, W, y.cpu(), w.ignore_index, 0)
    with pytest.raises(ValueError):
        flce.flce_forward(X, W.cpu(), y, w.ignore_index, 0)
    with pytest.raises(ValueError):
        flce.flce_forward(X, W, y, w.ignore_index, 0, out=(torch.empty((1,), dtype=torch.float32, device=dev),
                                                            torch.empty((1,), dtype=torch.int32, device=dev)))
    # a workspace given in another element type counts its bytes
    ws = torch.empty(((need + 3) // 4,), dtype=torch.float32, device=dev)
    loss, _, _ = flce.flce_fwd_bwd(X, W, y, w.ignore_index, 0, workspace=ws)
    assert torch.isfinite(loss).item()
