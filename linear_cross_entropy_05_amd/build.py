"""Build the gfx950 shared library ``libflce.so`` in-tree with hipcc.

    python -m linear_cross_entropy_05_amd.build [--verbose]

Each HIP source is compiled to an object in ``_build/`` (in parallel), the
host-only C++ unit by the host compiler, then all are linked into
``linear_cross_entropy_05_amd/libflce.so``.  The library links
the HIP runtime by soname (libamdhip64.so.7), so inside a process that has
imported torch it binds to the same runtime torch uses.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libflce.so")
SOURCES = ["api.hip", "kernels_flce.hip", "kernels_ce.hip", "kernels_orpo.hip", "profile.hip"]
# host-only C++ (argument checks, layouts): built by the host compiler
HOST_SOURCES = ["host_checks.cpp"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=fast",
    "-munsafe-fp-atomics",
    # no packed fp32 arithmetic (v_pk_*_f32) anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (need ROCm with gfx950 support)")


def _compile(src: str, verbose: bool, extra: list[str]) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(
        line for line in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in line
    )
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)
    return obj


def host_cxx() -> str:
    for cand in (os.environ.get("CXX"), shutil.which("g++"), shutil.which("c++")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("no host C++ compiler (g++) found")


def _compile_host(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [host_cxx(), *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host compile failed on {src}:\n{r.stdout}{r.stderr}")
    return obj


def build(verbose: bool = False, extra: list[str] | None = None, out: str = LIB) -> str:
    """Compile every HIP source for gfx950 and the host-only unit, and link
    libflce.so; return its path."""
    os.makedirs(BUILD, exist_ok=True)
    extra = extra or []
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES) + len(HOST_SOURCES)) as ex:
        hip = [ex.submit(_compile, s, verbose, extra) for s in SOURCES]
        host = [ex.submit(_compile_host, s, verbose) for s in HOST_SOURCES]
        objs = [f.result() for f in hip + host]
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true", help="print per-kernel register/LDS usage")
    a = ap.parse_args(argv)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if a.resource_usage else []
    print(build(verbose=a.verbose or a.resource_usage, extra=extra))
    return 0


if __name__ == "__main__":
    sys.exit(main())
