"""HIP path vs the float64 oracle, element by element (needs a gfx950 GPU).

Sizes are chosen so the oracle finishes in seconds while the GEMMs still span
several 256-wide tiles with ragged tails in every dimension, several token
chunks with a ragged last chunk, and the K (hidden) extent ends mid-stage.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_helpers import TOL, ensure_built, rel_err, run_gpu, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return ensure_built()


def check_against_oracle(w, chunk_tokens=None, inputs=None):
    (X, W, y), out = run_gpu(w, chunk_tokens, inputs)
    ref = oracle.flce_ref(X, W, y, w.ignore_index)
    tl, tg = TOL[w.dtype]
    el = abs(out["loss"] - ref["loss"]) / max(abs(ref["loss"]), 1e-30)
    ex = rel_err(to_np(out["dX"]), ref["dX"])
    ew = rel_err(to_np(out["dW"]), ref["dW"])
    er = rel_err(to_np(out["row_loss"]), ref["row_loss"])
    say(f"  loss {out['loss']:.7f} ref {ref['loss']:.7f} err {el:.2e}; dX {ex:.2e}; dW {ew:.2e}; rows {er:.2e}")
    assert el <= tl
    assert ex <= tg
    assert ew <= tg
    assert er <= max(tl, tg / 10)
    return out, ref


def test_tiny_fp32_matches_oracle():
    check_against_oracle(si.workload("tiny"))


@pytest.mark.parametrize("chunk", [1, 3, 5])
def test_tiny_fp32_other_chunk_sizes(chunk):
    check_against_oracle(si.workload("tiny"), chunk)


def test_fp32_ragged_multi_tile():
    # V = 1000: 4 vocabulary tiles, last one 232 wide; H = 200: 7 K stages, last 8 wide;
    # BT = 700 in chunks of 256: 3 chunks, last 188 tokens; H tiles ragged too.
    check_against_oracle(si.small(700, 200, 1000, "fp32", seed=21, w_std=0.05), 256)


def test_bf16_ragged_multi_tile():
    check_against_oracle(si.small(700, 200, 1000, "bf16", seed=22, w_std=0.05), 256)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_wide_hidden_split_dx(dtype):
    # few token tiles and a long vocabulary: the dX product is split along V
    # (9 splits in bf16, 16 in fp32), and the split sum reads the fp32
    # partials four at a time
    check_against_oracle(si.small(300, 520, 5000, dtype, seed=23), 300)


@pytest.mark.parametrize("BT,H,V,chunk", [(130, 72, 300, 64), (257, 136, 777, 100), (65, 520, 1300, 0),
                                           (513, 40, 5000, 200)])
def test_bf16_shape_sweep(BT, H, V, chunk):
    # hidden sizes and chunk lengths that are not multiples of 64 (the
    # transposed token chunk of the dW product pads both), tiny and long
    # vocabularies, several chunks with a ragged last one
    check_against_oracle(si.small(BT, H, V, "bf16", seed=BT + H + V, w_std=0.05), chunk)


@pytest.mark.parametrize("BT,H,V,chunk", [(2600, 200, 1000, 1100), (2200, 264, 515, 1088), (2000, 200, 1000, 700),
                                           (2560, 136, 777, 1024)])
def test_bf16_long_chunks_fold_old_dw(BT, H, V, chunk):
    # on chunks after the first the old dW rows are added into the
    # accumulators during the K loop of the dW product instead of being read
    # back at the end: one 32 x 32 block per stage for chunks of >= 1025
    # tokens (>= 17 K stages: 1100, 1088), two per stage for 513 .. 1024
    # tokens (9 .. 16 stages: 700 and the ragged 600, 1024); ragged last
    # chunks too short for either (400 / 24 / 512 tokens) take the
    # read-modify-write epilogue; partial vocabulary and hidden tiles in all
    check_against_oracle(si.small(BT, H, V, "bf16", seed=BT + V, w_std=0.05), chunk)


@pytest.mark.parametrize("chunk", [1050, 600])
def test_bf16_long_chunks_deterministic(chunk):
    # both fold paths are as deterministic as the store path
    w = si.small(2100, 136, 700, "bf16", seed=29)
    inputs = si.make_inputs(w)
    a = run_gpu(w, chunk, inputs)[1]
    b = run_gpu(w, chunk, inputs)[1]
    assert a["loss"] == b["loss"]
    assert torch.equal(a["dX"], b["dX"]) and torch.equal(a["dW"], b["dW"])


def test_bf16_large_logits():
    # hidden states x3, as in the huge-vocabulary config: logits std ~3
    check_against_oracle(si.small(512, 768, 3000, "bf16", seed=24, x_scale=3.0, w_std=0.04), 0)


def test_chunk_size_invariance_fp32():
    w = si.small(40, 64, 300, "fp32", seed=25)
    inputs = si.make_inputs(w)
    outs = [run_gpu(w, c, inputs)[1] for c in (1, 7, 40)]
    for o in outs[1:]:
        assert abs(o["loss"] - outs[0]["loss"]) <= 1e-6 * abs(outs[0]["loss"])
        assert rel_err(to_np(o["dX"]), to_np(outs[0]["dX"])) <= 1e-6
        assert rel_err(to_np(o["dW"]), to_np(outs[0]["dW"])) <= 1e-6


def test_bitwise_deterministic():
    w = si.small(600, 256, 2000, "bf16", seed=26)
    inputs = si.make_inputs(w)
    a = run_gpu(w, 256, inputs)[1]
    b = run_gpu(w, 256, inputs)[1]
    assert a["loss"] == b["loss"]
    assert torch.equal(a["dX"], b["dX"]) and torch.equal(a["dW"], b["dW"])


def test_all_ignored_gives_zero():
    w = si.small(64, 64, 500, "bf16", seed=27, ignore=("all",))
    (_, _, _), out = run_gpu(w, 32)
    assert out["loss"] == 0.0
    assert torch.count_nonzero(out["dX"]) == 0 and torch.count_nonzero(out["dW"]) == 0


def test_empty_batch():
    import linear_cross_entropy_05_amd as flce

    dev = torch.device("cuda", 0)
    X = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    W = torch.randn((100, 64), device=dev).to(torch.bfloat16)
    y = torch.empty((0,), dtype=torch.int64, device=dev)
    loss, dX, dW = flce.flce_fwd_bwd(X, W, y)
    assert loss.item() == 0.0 and dX.shape == (0, 64)
    assert torch.count_nonzero(dW) == 0


def test_out_of_range_target_raises():
    import linear_cross_entropy_05_amd as flce

    w = si.small(16, 64, 100, "bf16", seed=28)
    X, W, y = si.make_inputs(w)
    y[5] = 100  # == V
    dev = torch.device("cuda", 0)
    with pytest.raises(flce.FlceError) as e:
        flce.flce_fwd_bwd(X.to(dev), W.to(dev), y.to(dev))
    assert e.value.status == 6


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_compaction_leaves_later_chunks_empty(dtype):
    # only the non-ignored tokens fill the chunks: 70% ignored leaves 360
    # tokens, chunk 0 full (256), chunk 1 with 104 rows, chunks 2-4 empty
    check_against_oracle(si.small(1200, 136, 777, dtype, seed=41, ignore=("random_frac", 0.7), w_std=0.05), 256)


def test_compaction_tokens_kept_only_at_the_end():
    # the first 900 positions ignored: the kept tokens all come from the last
    # chunk's positions, and the ignored dX rows and losses are exact zeros
    w = si.small(1000, 200, 1000, "bf16", seed=42, w_std=0.05)
    X, W, y = si.make_inputs(w)
    y[:900] = w.ignore_index
    out, _ = check_against_oracle(w, 256, (X, W, y))
    assert torch.count_nonzero(out["dX"][:900]) == 0 and torch.count_nonzero(out["row_loss"][:900]) == 0


def test_compaction_over_several_scan_passes():
    # 9000 targets: the position list is built in three passes of 4096 (the
    # last ragged), 30% ignored at random; nine chunks of 1000 kept tokens
    check_against_oracle(si.small(9000, 64, 300, "fp32", seed=44, ignore=("random_frac", 0.3)), 1000)


def test_compaction_with_split_dx():
    # 40% ignored and a split dX product: split partials in chunk order, summed
    # rows written back to the tokens' positions
    check_against_oracle(si.small(300, 520, 5000, "bf16", seed=43, ignore=("random_frac", 0.4)), 300)


def test_custom_ignore_index():
    w = si.small(128, 64, 300, "fp32", seed=29, ignore_index=7, ignore=("random_frac", 0.2))
    check_against_oracle(w, 64)


def test_module_autograd_matches_oracle():
    import linear_cross_entropy_05_amd as flce

    w = si.small(96, 128, 700, "fp32", seed=30)
    X, W, y = si.make_inputs(w)
    dev = torch.device("cuda", 0)
    Wd = W.to(dev).requires_grad_(True)
    Xd = X.to(dev).requires_grad_(True)
    loss = flce.FusedLinearCrossEntropyLoss()(Wd, Xd, y.to(dev))
    (2.5 * loss).backward()
    ref = oracle.flce_ref(X, W, y)
    assert abs(loss.item() - ref["loss"]) <= 1e-5 * ref["loss"]
    assert rel_err(to_np(Xd.grad), 2.5 * ref["dX"]) <= 1e-5
    assert rel_err(to_np(Wd.grad), 2.5 * ref["dW"]) <= 1e-5


def test_mistral_head_full_size():
    # BT=2048, H=2048, V=32000, chunk 1024: the whole oracle fits in seconds
    out, ref = check_against_oracle(si.workload("mistral"))
    assert ref["n_valid"] == 2048 - 102


# ---- logits-only cross-entropy, in place ------------------------------------------


def run_ce(logits_cpu, y, ignore_index=-100):
    import linear_cross_entropy_05_amd as flce

    dev = torch.device("cuda", 0)
    L = logits_cpu.to(dev)
    say(f"[gpu] ce_fwd_bwd_inplace BT={L.shape[0]} V={L.shape[1]}")
    loss, rl = flce.ce_fwd_bwd_inplace(L, y.to(dev), ignore_index, row_loss=True)
    torch.cuda.synchronize()
    return float(loss.item()), L.cpu(), rl.cpu()


@pytest.mark.parametrize("V", [1, 7, 1001, 4096, 50257, 65539, 102401, 150001])
def test_ce_inplace_matches_oracle(V):
    g = torch.Generator().manual_seed(V)
    BT = 37
    logits = torch.randn(BT, V, generator=g) * 3
    y = torch.randint(0, V, (BT,), generator=g)
    y[[0, 11]] = -100
    loss, dl, rl = run_ce(logits, y)
    ref = oracle.ce_ref(logits, y)
    assert abs(loss - ref["loss"]) <= 1e-5 * abs(ref["loss"])
    assert rel_err(to_np(dl), ref["dlogits"]) <= 1e-5
    assert rel_err(to_np(rl), ref["row_loss"]) <= 1e-5
    assert torch.count_nonzero(dl[[0, 11]]) == 0


def test_ce_inplace_out_of_range_raises():
    import linear_cross_entropy_05_amd as flce

    logits = torch.randn(4, 10).cuda()
    y = torch.tensor([1, 2, -3, 4]).cuda()
    with pytest.raises(flce.FlceError):
        flce.ce_fwd_bwd_inplace(logits, y)
