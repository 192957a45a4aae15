"""The C-ABI library on the CPU: it loads, exports what include/flce.h declares,
sizes workspaces, and rejects bad arguments before touching any device.
No call here reaches a kernel launch."""
import ctypes

import pytest

from gpu_helpers import ensure_built

F32, BF16 = 0, 1


@pytest.fixture(scope="module")
def lib():
    return ensure_built()


def test_exports_every_declared_function(lib):
    from linear_cross_entropy_05_amd import header_functions

    names = header_functions()
    assert set(names) >= {
        "flce_fwd_bwd",
        "flce_fwd",
        "flce_fwd_workspace_bytes",
        "flce_orpo",
        "flce_orpo_workspace_bytes",
        "ce_fwd_bwd_inplace",
        "flce_workspace_bytes",
        "ce_workspace_bytes",
        "flce_chunk_tokens",
        "flce_status_str",
        "flce_device_supported",
        "ce_fwd_bwd_inplace_noalloc",
        "ce_noalloc_max_rows",
    }
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in range(10):
        assert lib.flce_status_str(s)
    assert b"unknown" in lib.flce_status_str(99)


def test_chunk_rule(lib):
    # fewest chunks with C x round_up(V, 256) elements <= 1 GiB, equal, rounded up to 256 tokens
    assert lib.flce_chunk_tokens(8192, 4096, 128256, 0, BF16) == 4096  # 2 chunks
    assert lib.flce_chunk_tokens(16384, 3584, 152064, 0, BF16) == 3328  # 5 chunks (at most 3530 tokens fit)
    assert lib.flce_chunk_tokens(8192, 3072, 256000, 0, BF16) == 2048  # 4 chunks
    assert lib.flce_chunk_tokens(4000, 4096, 128256, 0, BF16) == 4000  # fits whole
    assert lib.flce_chunk_tokens(5000, 4096, 128256, 0, BF16) == 2560  # 2 chunks of 2500 -> 2560
    assert lib.flce_chunk_tokens(2048, 2048, 32000, 1024, BF16) == 1024
    assert lib.flce_chunk_tokens(8, 128, 256, 8, F32) == 8
    assert lib.flce_chunk_tokens(100, 128, 256, 0, F32) == 100
    assert lib.flce_chunk_tokens(100, 128, 256, 1000, F32) == 100
    assert lib.flce_chunk_tokens(-1, 128, 256, 0, F32) == 0


def test_workspace_bound_by_one_chunk(lib):
    for BT, H, V, C in ((8192, 4096, 128256, 0), (16384, 3584, 152064, 0), (8192, 3072, 256000, 0)):
        c = lib.flce_chunk_tokens(BT, H, V, C, BF16)
        ldz = (V + 255) // 256 * 256
        chunk = c * ldz * 2
        ws = lib.flce_workspace_bytes(BT, H, V, C, BF16)
        assert chunk <= ws <= chunk * 1.5, (BT, H, V, ws / chunk)
    assert lib.flce_workspace_bytes(8, 0, 256, 0, F32) == 0
    assert lib.flce_workspace_bytes(8, 128, 256, 0, 7) == 0
    assert lib.ce_workspace_bytes(8192, 256000) >= 8192 * 4


# Default (fake, never dereferenced) arguments of each entry point and the
# cases that must be rejected on the host with the given status.  The same
# tables drive the sanitizer build of the host checks (test_host_sanitize.py).
FWD_BWD_DEFAULTS = dict(X=16, W=16, t=16, s=None, BT=8, H=128, V=256, ign=-100, C=0, dt=F32, loss=16, rl=None, dX=16,
                        dW=16, ws=256, wsb=1 << 20, err=16, stream=None)


def _call(lib, **kw):
    a = dict(FWD_BWD_DEFAULTS)
    a.update(kw)
    vp = ctypes.c_void_p
    return lib.flce_fwd_bwd(vp(a["X"]), vp(a["W"]), vp(a["t"]), vp(a["s"]), a["BT"], a["H"], a["V"], a["ign"], a["C"],
                            a["dt"], vp(a["loss"]), vp(a["rl"]), vp(a["dX"]), vp(a["dW"]), vp(a["ws"]), a["wsb"],
                            vp(a["err"]), vp(a["stream"]))


FWD_BWD_CASES = [
    (dict(dt=5), 2),
    (dict(H=0), 1),
    (dict(V=0), 1),
    (dict(BT=-1), 1),
    (dict(W=None), 1),
    (dict(X=None), 1),
    (dict(t=None), 1),
    (dict(loss=None), 1),
    (dict(dX=None), 1),
    (dict(dW=None), 1),
    (dict(ws=None), 1),
    (dict(err=None), 1),
    (dict(H=130), 7),
    (dict(H=132, dt=BF16), 7),
    (dict(X=24), 8),
    (dict(W=8), 8),
    (dict(ws=128), 8),
    (dict(t=20), 8),
    (dict(s=18), 8),
    # the products store 16-byte (fp32) or 8-byte (bf16) pieces of dX and dW rows
    (dict(dX=20), 8),
    (dict(dX=24, dt=BF16, H=128), 8),
    (dict(dW=20), 8),
    (dict(wsb=16), 3),
    # a 256-row tile of the logits chunk past 2^31 bytes (V = 4.2 M bf16, 2.1 M fp32)
    (dict(V=4_200_000, dt=BF16, C=1, wsb=1 << 62), 7),
    (dict(V=2_100_000, C=1, wsb=1 << 62), 7),
    # a 256-row tile of W past 2^31 bytes (H = 4.2 M bf16)
    (dict(H=4_200_000, dt=BF16, C=1, wsb=1 << 62), 7),
    # a 256-row tile of the fp32 dW past 2^31 bytes (H = 2.1 M; its bf16 W tile still fits)
    (dict(H=2_100_000, dt=BF16, C=1, wsb=1 << 62), 7),
    # the transposed token chunk (bf16 only): chunk of 4.2 M tokens
    (dict(BT=4_200_000, H=8, dt=BF16, C=4_200_000, wsb=1 << 62), 7),
]


@pytest.mark.parametrize("kw,status", FWD_BWD_CASES)
def test_host_argument_checks(lib, kw, status):
    # fake, never-dereferenced addresses: every case is rejected on the host
    assert _call(lib, **kw) == status


FWD_DEFAULTS = dict(X=16, W=16, t=16, BT=8, H=128, V=256, ign=-100, C=0, dt=F32, loss=16, rl=None, ws=256,
                    wsb=1 << 20, err=16, stream=None)


def _call_fwd(lib, **kw):
    a = dict(FWD_DEFAULTS)
    a.update(kw)
    vp = ctypes.c_void_p
    return lib.flce_fwd(vp(a["X"]), vp(a["W"]), vp(a["t"]), a["BT"], a["H"], a["V"], a["ign"], a["C"], a["dt"],
                        vp(a["loss"]), vp(a["rl"]), vp(a["ws"]), a["wsb"], vp(a["err"]), vp(a["stream"]))


FWD_CASES = [
    (dict(dt=5), 2),
    (dict(H=0), 1),
    (dict(V=0), 1),
    (dict(BT=-1), 1),
    (dict(W=None), 1),
    (dict(X=None), 1),
    (dict(t=None), 1),
    (dict(loss=None), 1),
    (dict(ws=None), 1),
    (dict(err=None), 1),
    (dict(H=130), 7),
    (dict(H=132, dt=BF16), 7),
    (dict(X=24), 8),
    (dict(W=8), 8),
    (dict(ws=128), 8),
    (dict(t=20), 8),
    (dict(rl=18), 8),
    (dict(H=4_200_000, dt=BF16, C=1, wsb=1 << 62), 7),
    (dict(wsb=16), 3),
]


@pytest.mark.parametrize("kw,status", FWD_CASES)
def test_forward_host_argument_checks(lib, kw, status):
    assert _call_fwd(lib, **kw) == status


def test_forward_workspace_has_no_chunk_buffer(lib):
    # statistics only: 8 bytes per token and 128-wide vocabulary block, plus O(BT)
    for BT, H, V in ((8192, 4096, 128256), (16384, 3584, 152064), (8192, 3072, 256000)):
        ws = lib.flce_fwd_workspace_bytes(BT, H, V, 0, BF16)
        nvh = 2 * ((V + 255) // 256)
        assert ws <= BT * nvh * 8 + 3 * BT * 4 + 4096, (BT, H, V, ws)
        assert ws < lib.flce_workspace_bytes(BT, H, V, 0, BF16) / 4
    assert lib.flce_fwd_workspace_bytes(8, 0, 256, 0, F32) == 0
    assert lib.flce_fwd_workspace_bytes(8, 128, 256, 0, 9) == 0


CE_DEFAULTS = dict(lg=16, t=16, BT=4, V=10, ign=-100, loss=16, rl=None, ws=256, wsb=4096, err=16, stream=None)
CE_CASES = [
    (dict(BT=-1), 1),
    (dict(V=0), 1),
    (dict(V=1 << 31), 1),  # V >= 2^31
    (dict(lg=None), 1),
    (dict(loss=None), 1),
    (dict(lg=18), 8),
    (dict(wsb=1), 3),
]


@pytest.mark.parametrize("kw,status", CE_CASES)
def test_ce_host_argument_checks(lib, kw, status):
    a = dict(CE_DEFAULTS)
    a.update(kw)
    vp = ctypes.c_void_p
    assert lib.ce_fwd_bwd_inplace(vp(a["lg"]), vp(a["t"]), a["BT"], a["V"], a["ign"], vp(a["loss"]), vp(a["rl"]),
                                  vp(a["ws"]), a["wsb"], vp(a["err"]), vp(a["stream"])) == status


NOALLOC_MAX_ROWS = 1 << 21
NOALLOC_DEFAULTS = dict(lg=16, t=16, BT=4, V=10, ign=-100, loss=16, rl=None, err=16, stream=None)
NOALLOC_CASES = [
    (dict(BT=NOALLOC_MAX_ROWS + 1), 9),  # more rows than the static scratch holds
    (dict(BT=-1), 1),
    (dict(V=0), 1),
    (dict(lg=None), 1),
    (dict(loss=None), 1),
    (dict(err=None), 1),
    (dict(lg=18), 8),
    (dict(rl=18), 8),
    (dict(t=20), 8),
]


def test_noalloc_row_limit(lib):
    assert lib.ce_noalloc_max_rows() == NOALLOC_MAX_ROWS


@pytest.mark.parametrize("kw,status", NOALLOC_CASES)
def test_ce_noalloc_host_argument_checks(lib, kw, status):
    a = dict(NOALLOC_DEFAULTS)
    a.update(kw)
    vp = ctypes.c_void_p
    assert lib.ce_fwd_bwd_inplace_noalloc(vp(a["lg"]), vp(a["t"]), a["BT"], a["V"], a["ign"], vp(a["loss"]),
                                          vp(a["rl"]), vp(a["err"]), vp(a["stream"])) == status


def test_no_cpu_fallback_in_product_code():
    """The product package never imports the oracle and has no CPU path."""
    import pathlib

    pkg = pathlib.Path(__file__).resolve().parent.parent / "linear_cross_entropy_05_amd"
    for p in list(pkg.glob("*.py")) + list(pkg.glob("csrc/*")):
        text = p.read_text(errors="ignore")
        assert "oracle" not in text.lower().replace("oracle-free", ""), p
        assert "synth_inputs" not in text, p


ORPO_DEFAULTS = dict(X=16, W=16, t=16, ns=4, T=8, H=128, V=256, ign=-100, beta=0.1, C=0, dt=F32, loss=16, sl=None,
                     dX=16, dW=16, ws=256, wsb=1 << 24, err=16, stream=None)


def _call_orpo(lib, **kw):
    a = dict(ORPO_DEFAULTS)
    a.update(kw)
    vp = ctypes.c_void_p
    return lib.flce_orpo(vp(a["X"]), vp(a["W"]), vp(a["t"]), a["ns"], a["T"], a["H"], a["V"], a["ign"],
                         ctypes.c_float(a["beta"]), a["C"], a["dt"], vp(a["loss"]), vp(a["sl"]), vp(a["dX"]),
                         vp(a["dW"]), vp(a["ws"]), a["wsb"], vp(a["err"]), vp(a["stream"]))


ORPO_CASES = [
    (dict(dt=3), 2),
    (dict(ns=3), 1),
    (dict(ns=0), 1),
    (dict(T=0), 1),
    (dict(H=0), 1),
    (dict(X=None), 1),
    (dict(dX=None), 1),
    (dict(H=130), 7),
    (dict(X=24), 8),
    (dict(sl=18), 8),
    (dict(dX=24), 8),
    (dict(dW=20), 8),
    (dict(ws=128), 8),
    (dict(wsb=16), 3),
]


@pytest.mark.parametrize("kw,status", ORPO_CASES)
def test_orpo_host_argument_checks(lib, kw, status):
    assert _call_orpo(lib, **kw) == status


def test_orpo_workspace(lib):
    # one pass (a 4096-token chunk holds 2 pairs of 1024-token sequences): one
    # chunk's workspace, the gathered rows and their dX rows (4096 x 4096 bf16
    # each), targets, token arrays, per-sequence and per-pair sums
    ws = lib.flce_orpo_workspace_bytes(8, 1024, 4096, 128256, 0, BF16)
    # flce_fwd_bwd's workspace less its token-compaction arrays (positions,
    # gathered targets, scales and X rows), which the ORPO chunks do not use
    compaction = 4096 * (4 + 8 + 4) + 4096 * 4096 * 2
    one = lib.flce_workspace_bytes(4096, 4096, 128256, 4096, BF16) - compaction
    rows = 2 * 4096 * 4096 * 2
    assert one + rows < ws <= one + rows + 4096 * (8 + 4 + 4) + 8 * 24 + 4 * 8 + 8 * 256
    # two passes (a 4096-token sequence pair does not fit a 4096-token chunk):
    # the larger of the two passes' workspaces plus per-token and per-sequence arrays
    ws2 = lib.flce_orpo_workspace_bytes(2, 4096, 4096, 128256, 0, BF16)
    fb = lib.flce_workspace_bytes(8192, 4096, 128256, 0, BF16) - (8192 * 4 + 4096 * (8 + 4) + 4096 * 4096 * 2)
    assert fb < ws2 <= fb + 8192 * 8 + 2 * 24 + 4096
    assert lib.flce_orpo_workspace_bytes(3, 1024, 4096, 128256, 0, BF16) == 0
    assert lib.flce_orpo_workspace_bytes(8, 0, 4096, 128256, 0, BF16) == 0
