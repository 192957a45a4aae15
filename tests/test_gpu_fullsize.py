"""Full-size workloads on the GPU, in the launch configuration bench.py times
(automatic chunk size), checked element by element against the float64
oracle run here on the host.

FLCE heads (Llama-3-8B, Qwen2-7B at 16K context, Gemma 256K vocabulary):
  * a fast pre-check against stored oracle values (tests/golden/<name>.json,
    written by make_full_size_golden.py from the same seeded inputs, whose
    fingerprint is checked first): the loss, 64 token losses, 4096 random dX
    entries and 4096 + 4 H dW entries;
  * then the whole oracle (oracle.flce_ref, float64 with the full logits;
    oracle.flce_ref_rowblocks when the host is short of memory, said in the
    output): the loss and EVERY token loss, dX entry and dW entry, with
    max |gpu - ref| / max |ref| per tensor against the bf16 bound.
Forward only (flce_fwd) on the same three heads: the loss and every token
loss against the same oracle run.
Logits-only cross-entropy on the Gemma shape (fp32 logits 8192 x 256000,
8.4 GB): every token loss and every dlogits row, pulled back and compared
block by block against the per-row oracle.
"""
import gc
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_helpers import TOL, ensure_built, rel_err, say, to_np

# each test runs the float64 oracle over a whole head on the host (up to a
# minute or two of CPU time), beyond the per-test limit used for GPU runs
pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# oracle loss and token losses of each workload, kept for the forward-only test
_ORACLE_ROWS = {}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return ensure_built()


def _mem_available() -> int:
    try:
        with open("/proc/meminfo") as f:
            for ln in f:
                if ln.startswith("MemAvailable:"):
                    return int(ln.split()[1]) * 1024
    except OSError:
        pass
    return 0


def _oracle(w, X, W, y):
    """The whole float64 oracle if the host has room for its logits, else
    the row-blocked form of the same definition."""
    need = 8 * (w.BT * w.V + 3 * w.V * w.H + 3 * w.BT * w.H)  # logits, W, dW (+ copy), X, dX
    avail = _mem_available()
    if avail >= 1.3 * need:
        say(f"  oracle: whole float64 definition ({need / 2**30:.1f} GiB of {avail / 2**30:.1f} GiB available)")
        ref = oracle.flce_ref(X, W, y, w.ignore_index)
        ref.pop("dlogits")
    else:
        say(f"  oracle: row blocks of 512 tokens (whole form needs {need / 2**30:.1f} GiB, "
            f"{avail / 2**30:.1f} GiB available)")
        ref = oracle.flce_ref_rowblocks(X, W, y, w.ignore_index, block=512)
    return ref


def _max_err(got_t, ref, rows=4096):
    """max |got - ref| over all entries, block by block (got on the GPU)."""
    e = 0.0
    for b in range(0, ref.shape[0], rows):
        g = got_t[b:b + rows].float().cpu().numpy().astype(np.float64)
        e = max(e, float(np.max(np.abs(g - ref[b:b + rows]))))
    return e


@pytest.mark.parametrize("name", ["llama3", "qwen2", "gemma"])
def test_flce_full_size(name):
    import linear_cross_entropy_05_amd as flce

    with open(os.path.join(GOLDEN, f"{name}.json")) as f:
        g = json.load(f)
    w = si.workload(name)
    X, W, y = si.make_inputs(w)
    assert si.fingerprint(X, W, y) == g["fingerprint"], "seeded inputs differ from the ones the oracle saw"
    dev = torch.device("cuda", 0)
    say(f"[gpu] flce_fwd_bwd {name} BT={w.BT} H={w.H} V={w.V} chunk=auto")
    loss, dX, dW, rl = flce.flce_fwd_bwd(X.to(dev), W.to(dev), y.to(dev), w.ignore_index, w.chunk_tokens,
                                         row_loss=True)
    torch.cuda.synchronize()
    tl, tg = TOL[w.dtype]

    # fast pre-check: stored samples
    el = abs(loss.item() - g["loss"]) / abs(g["loss"])
    rows = torch.tensor(g["rows"])
    er = rel_err(to_np(rl[rows.to(dev)]), g["row_loss"])
    xi = torch.tensor(g["dX_idx"], device=dev)
    wi = torch.tensor(g["dW_idx"], device=dev)
    ex = float(np.max(np.abs(to_np(dX[xi[:, 0], xi[:, 1]]) - np.array(g["dX_val"])))) / g["max_abs_dX"]
    ew = float(np.max(np.abs(to_np(dW[wi[:, 0], wi[:, 1]]) - np.array(g["dW_val"])))) / g["max_abs_dW"]
    say(f"  stored samples: loss err {el:.2e}; rows {er:.2e}; dX {ex:.2e}; dW {ew:.2e}")
    assert el <= tl and er <= tl and ex <= tg and ew <= tg

    # every entry against the oracle run here
    ref = _oracle(w, X, W, y)
    assert ref["n_valid"] == g["n_valid"]
    _ORACLE_ROWS[name] = (ref["loss"], ref["row_loss"].copy())
    el = abs(loss.item() - ref["loss"]) / abs(ref["loss"])
    er = rel_err(to_np(rl), ref["row_loss"])
    ex = _max_err(dX, ref["dX"]) / float(np.max(np.abs(ref["dX"])))
    ew = _max_err(dW, ref["dW"]) / float(np.max(np.abs(ref["dW"])))
    nx, nw = ref["dX"].size, ref["dW"].size
    say(f"  every entry: loss {loss.item():.7f} ref {ref['loss']:.7f} err {el:.2e}; {w.BT} token losses {er:.2e}; "
        f"dX ({nx} entries) {ex:.2e}; dW ({nw} entries) {ew:.2e}")
    del ref, dX, dW, rl
    gc.collect()
    torch.cuda.empty_cache()
    assert el <= tl and er <= tl and ex <= tg and ew <= tg


@pytest.mark.parametrize("name", ["llama3", "qwen2", "gemma"])
def test_flce_forward_full_size(name):
    """Forward only, automatic pass size: the loss and every token loss
    against the oracle (the run of the fwd+bwd test, or a new one)."""
    import linear_cross_entropy_05_amd as flce

    w = si.workload(name)
    X, W, y = si.make_inputs(w)
    dev = torch.device("cuda", 0)
    say(f"[gpu] flce_forward {name} BT={w.BT} H={w.H} V={w.V} chunk=auto")
    loss, rl = flce.flce_forward(X.to(dev), W.to(dev), y.to(dev), w.ignore_index, row_loss=True)
    torch.cuda.synchronize()
    if name not in _ORACLE_ROWS:
        ref = _oracle(w, X, W, y)
        _ORACLE_ROWS[name] = (ref["loss"], ref["row_loss"].copy())
        del ref
        gc.collect()
    ref_loss, ref_rl = _ORACLE_ROWS[name]
    tl, _ = TOL[w.dtype]
    el = abs(loss.item() - ref_loss) / abs(ref_loss)
    er = rel_err(to_np(rl), ref_rl)
    say(f"  loss {loss.item():.7f} ref {ref_loss:.7f} err {el:.2e}; all {w.BT} token losses {er:.2e}")
    assert el <= tl and er <= tl


def test_ce_inplace_gemma_shape():
    import linear_cross_entropy_05_amd as flce

    w = si.workload("gemma")
    X, W, y = si.make_inputs(w)
    dev = torch.device("cuda", 0)
    # input preparation (not the path under test): fp32 logits of the Gemma head
    logits = X.to(dev).float() @ W.to(dev).float().T
    del W
    logits_cpu = logits.cpu()
    say(f"[gpu] ce_fwd_bwd_inplace gemma BT={w.BT} V={w.V} fp32")
    loss, rl = flce.ce_fwd_bwd_inplace(logits, y.to(dev), w.ignore_index, row_loss=True)
    torch.cuda.synchronize()
    got_rl = to_np(rl)
    n_valid = int((y != w.ignore_index).sum())
    ref_rl = np.zeros(w.BT)
    err_d, max_ref = 0.0, 0.0
    B = 512
    for b in range(0, w.BT, B):
        ref = oracle.ce_rows_ref(logits_cpu[b:b + B], y[b:b + B], n_valid, w.ignore_index)
        ref_rl[b:b + B] = ref["row_loss"]
        got = logits[b:b + B].cpu().numpy().astype(np.float64)  # the gradient the call left in place
        err_d = max(err_d, float(np.max(np.abs(got - ref["dlogits"]))))
        max_ref = max(max_ref, float(np.max(np.abs(ref["dlogits"]))))
        del ref, got
    del logits
    torch.cuda.empty_cache()
    ref_loss = float(ref_rl.sum() / n_valid)
    el = abs(loss.item() - ref_loss) / ref_loss
    er = rel_err(got_rl, ref_rl)
    ed = err_d / max_ref
    say(f"  loss {loss.item():.7f} ref {ref_loss:.7f} err {el:.2e}; token losses {er:.2e}; "
        f"every dlogits entry ({w.BT * w.V}) {ed:.2e}")
    tl, tg = TOL["fp32"]
    assert el <= tl and er <= tl and ed <= tg
