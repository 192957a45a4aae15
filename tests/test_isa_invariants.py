"""Invariants of the generated gfx950 code that the kernels' inline assembly
relies on and the compiler does not check.  CPU only: hipcc cross-compiles the
device code to assembly here, with the library's own flags.

* m0: every direct-to-LDS copy sets m0 (its LDS destination) inside its own asm
  statement, right before the copy; nothing else in the kernels may write or
  read m0, because hipcc does not preserve a clobbered m0 for its own code.
* dW fold loads: the old-dW loads that the dW product issues from inline asm
  inside its K loop must not have their destination registers read or written
  before the workgroup barrier whose wait covers them (the compiler takes an
  asm load's output as written when the statement ends).
* No packed fp32 arithmetic in device code (the library is built without it).
"""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from linear_cross_entropy_05_amd import build  # noqa: E402

SOURCES = ["kernels_flce.hip", "kernels_ce.hip", "kernels_orpo.hip"]
DW_BF16 = "_ZN4flce7k_dx_dwIDF16bEEvNS_7BwdArgsIT_EE"  # the dX and dW products, one kernel


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    try:
        hipcc = build.hipcc()
    except RuntimeError:
        pytest.skip("no hipcc")
    out = tmp_path_factory.mktemp("isa")
    texts = {}
    for src in SOURCES:
        dst = os.path.join(out, src + ".s")
        cmd = [hipcc, *build.HIPCC_FLAGS, "--offload-device-only", "-S", "-o", dst, os.path.join(build.CSRC, src)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        texts[src] = open(dst).read()
    return texts


def _code(text):
    """(instruction text without comments, raw line) pairs."""
    return [(l.split(";")[0].strip(), l) for l in text.splitlines()]


def _regs(tok):
    m = re.match(r"[va]\[(\d+):(\d+)\]$", tok)
    if m:
        return {(tok[0], i) for i in range(int(m.group(1)), int(m.group(2)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def test_m0_written_only_by_the_copies(asm):
    writes = 0
    for src, text in asm.items():
        code = [c for c, _ in _code(text) if c]
        for i, ins in enumerate(code):
            if ins.startswith("s_mov_b32 m0,"):
                writes += 1
                nxt = code[i + 1]
                assert nxt.startswith("buffer_load_dword") and nxt.endswith(" lds"), (src, ins, nxt)
            else:
                assert not re.search(r"\bm0\b", ins), (src, ins)
    assert writes > 0  # the copies are there


def test_fold_loads_untouched_until_their_barrier(asm):
    lines = asm["kernels_flce.hip"].splitlines()
    start = next(i for i, l in enumerate(lines) if l.startswith(DW_BF16 + ":"))
    end = next(i for i in range(start, len(lines)) if lines[i].startswith(".Lfunc_end"))
    raw = lines[start:end]
    code = [l.split(";")[0].strip() for l in raw]
    checked = 0
    for i, ins in enumerate(code):
        asm_load = (re.match(r"buffer_load_dword(x4)?\b", ins) and not ins.endswith(" lds")
                    and "ASMSTART" in raw[i - 1])
        if not asm_load:
            continue
        checked += 1
        dst = _regs(ins.split()[1].rstrip(","))
        assert dst, ins
        for later in code[i + 1:]:
            if later.startswith("s_barrier"):
                break
            if not later:
                continue
            ops = [t.rstrip(",") for t in later.split()[1:]]
            touched = set().union(*(_regs(t) for t in ops)) if ops else set()
            if later.startswith("buffer_load_dword") and not later.endswith(" lds") and not (_regs(ops[0]) & dst):
                continue  # another fold load of the same group
            assert not (touched & dst), f"{ins} -> {later}"
        else:
            raise AssertionError(f"no barrier after {ins}")
    assert checked == 128  # 16 groups of 4 (one block per stage) + 8 groups of 8 (two per stage)


def test_no_packed_fp32_arithmetic(asm):
    for src, text in asm.items():
        for ins, _ in _code(text):
            assert not re.match(r"v_pk_(fma|mul|add)_f32\b", ins), (src, ins)
