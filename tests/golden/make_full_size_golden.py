"""Write oracle values for the three full-size FLCE workloads (CPU, float64).

    python tests/golden/make_full_size_golden.py [llama3 qwen2 gemma]

For each workload the seeded inputs come from ``synth_inputs`` and the whole
float64 oracle ``oracle.flce_ref`` runs once (minutes per workload, ~30 GB of
host memory at the largest).  Stored per workload, in ``<name>.json``: the
input fingerprint (the GPU test regenerates the inputs and checks it), the
loss, N, max |dX| and max |dW| over all entries, and sampled entries -- the
per-token losses of 64 tokens, 4096 random dX entries, 4096 random dW entries
plus every hidden unit of the dW rows of the 4 most frequent targets (the
largest dW values).  Only ``oracle`` and ``synth_inputs`` are used here.
"""

import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth_inputs as si  # noqa: E402


def sample(name: str, seed: int = 1234):
    w = si.workload(name)
    X, W, y = si.make_inputs(w)
    fp = si.fingerprint(X, W, y)
    t0 = time.time()
    ref = oracle.flce_ref(X, W, y, w.ignore_index)
    dt = time.time() - t0
    r = np.random.default_rng(seed)
    rows = np.sort(r.choice(w.BT, 64, replace=False))
    dx_idx = np.stack([r.integers(0, w.BT, 4096), r.integers(0, w.H, 4096)], 1)
    dw_idx = np.stack([r.integers(0, w.V, 4096), r.integers(0, w.H, 4096)], 1)
    yv = y.numpy()
    counts = np.bincount(yv[yv != w.ignore_index], minlength=w.V)
    top = np.argsort(-counts)[:4]
    hot = np.stack([np.repeat(top, w.H), np.tile(np.arange(w.H), len(top))], 1)
    dw_idx = np.concatenate([dw_idx, hot])
    out = {
        "workload": name,
        "shape": [w.BT, w.H, w.V],
        "fingerprint": fp,
        "oracle_seconds": round(dt, 1),
        "loss": ref["loss"],
        "n_valid": ref["n_valid"],
        "max_abs_dX": float(np.max(np.abs(ref["dX"]))),
        "max_abs_dW": float(np.max(np.abs(ref["dW"]))),
        "rows": rows.tolist(),
        "row_loss": ref["row_loss"][rows].tolist(),
        "dX_idx": dx_idx.tolist(),
        "dX_val": ref["dX"][dx_idx[:, 0], dx_idx[:, 1]].tolist(),
        "dW_idx": dw_idx.tolist(),
        "dW_val": ref["dW"][dw_idx[:, 0], dw_idx[:, 1]].tolist(),
    }
    with open(os.path.join(HERE, f"{name}.json"), "w") as f:
        json.dump(out, f)
    print(f"{name}: loss {ref['loss']:.8f} N {ref['n_valid']} oracle {dt:.0f} s", flush=True)


if __name__ == "__main__":
    for n in sys.argv[1:] or ["llama3", "qwen2", "gemma"]:
        sample(n)
