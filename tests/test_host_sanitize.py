"""The library's host-only unit (argument checks, chunk rule, workspace
layouts: linear_cross_entropy_05_amd/csrc/host_checks.cpp) built with the
address and undefined-behaviour sanitizers by the host compiler, then run on
the same rejection cases the C-ABI tests use (test_abi.py) and on a sweep of
shapes whose layouts must keep their invariants.  CPU only."""
import os
import shutil
import subprocess

import pytest

import test_abi as abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "linear_cross_entropy_05_amd", "csrc", "host_checks.cpp")
DRIVER = os.path.join(ROOT, "tests", "host", "asan_driver.cpp")
OUT = os.path.join(ROOT, "_build", "asan_driver")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


@pytest.fixture(scope="module")
def driver():
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no g++")
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-Wall", "-Wextra", *SAN, SRC, DRIVER, "-o", OUT]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return OUT


def _run(driver, lines):
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=1:detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([driver], input="\n".join(lines) + "\n", capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, f"sanitizer report:\n{r.stderr[-4000:]}"
    assert "runtime error" not in r.stderr, r.stderr[-4000:]
    out = r.stdout.split()
    assert len(out) == len(lines), r.stdout
    return out


def _p(v):
    return 0 if v is None else int(v)


def test_entry_point_checks_under_sanitizers(driver):
    lines, want = [], []
    for kw, status in abi.FWD_BWD_CASES + [({}, 0)]:
        a = dict(abi.FWD_BWD_DEFAULTS, **kw)
        lines.append("fwd_bwd " + " ".join(str(_p(a[k])) for k in
                     ("X", "W", "t", "s", "BT", "H", "V", "C", "dt", "loss", "rl", "dX", "dW", "ws", "wsb", "err")))
        want.append(status)
    for kw, status in abi.FWD_CASES + [({}, 0)]:
        a = dict(abi.FWD_DEFAULTS, **kw)
        lines.append("fwd " + " ".join(str(_p(a[k])) for k in
                     ("X", "W", "t", "BT", "H", "V", "C", "dt", "loss", "rl", "ws", "wsb", "err")))
        want.append(status)
    for kw, status in abi.ORPO_CASES + [({}, 0)]:
        a = dict(abi.ORPO_DEFAULTS, **kw)
        lines.append("orpo " + " ".join(str(_p(a[k])) for k in
                     ("X", "W", "t", "ns", "T", "H", "V", "C", "dt", "loss", "sl", "dX", "dW", "ws", "wsb", "err")))
        want.append(status)
    for kw, status in abi.CE_CASES + [({}, 0)]:
        a = dict(abi.CE_DEFAULTS, **kw)
        lines.append("ce " + " ".join(str(_p(a[k])) for k in ("lg", "t", "BT", "V", "loss", "rl", "ws", "wsb", "err")))
        want.append(status)
    for kw, status in abi.NOALLOC_CASES + [({}, 0)]:
        a = dict(abi.NOALLOC_DEFAULTS, **kw)
        lines.append("ce_noalloc " + " ".join(str(_p(a[k])) for k in ("lg", "t", "BT", "V", "loss", "rl", "err"))
                     + f" {abi.NOALLOC_MAX_ROWS}")
        want.append(status)
    got = [int(x) for x in _run(driver, lines)]
    assert got == want


def test_layouts_under_sanitizers(driver):
    lines = []
    for dt in (0, 1):
        for BT in (0, 1, 7, 8, 255, 256, 257, 1000, 4096, 5000, 8192, 16384, 1 << 20):
            for H in (4 * (1 + dt), 128, 2048, 3072, 3584, 4096):
                for V in (1, 2, 255, 256, 257, 32000, 50257, 128256, 152064, 256000, 2_000_000):
                    for C in (0, 1, 3, 1024, 4096):
                        lines.append(f"layout {BT} {H} {V} {C} {dt}")
    got = _run(driver, lines)
    bad = [(ln, g) for ln, g in zip(lines, got) if g != "ok"]
    assert not bad, bad[:10]


def test_size_queries_reject_huge_sizes_under_sanitizers(driver):
    big = (1 << 62) + 17
    lines = [f"query {big} 4096 128256 0 1", f"query 8192 {big} 128256 0 1", f"query 8192 4096 {big} 0 1",
             f"query {1 << 31} 4096 128256 0 1", "query -1 4096 128256 0 1", f"query {(1 << 31) - 1} 8 8 0 1"]
    got = _run(driver, lines)
    # (the logits-only workspace takes no hidden size: a huge H leaves it valid)
    assert got[:5] == ["0,0,0,0,0", f"0,0,0,0,{256 + 8192 * 4}", "0,0,0,0,0", "0,0,0,0,0", "0,0,0,0,0"], got
    # the largest accepted token count still gives a layout (and no overflow)
    assert all(int(v) > 0 for v in got[5].split(",")[:3]), got[5]


def test_xcd_ranges_under_sanitizers(driver):
    # every launch size up to 20,000 tiles plus the Llama head's and the
    # largest one the checks allow: the per-XCD ranges partition the tiles;
    # and the two-kind layout of the dX + dW launch is a bijection per kind
    assert _run(driver, ["tiles 20000"]) == ["ok"]
