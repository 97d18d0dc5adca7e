"""Build libspectra.so (HIP, gfx950) in-tree with hipcc.

    python -m dequant_gemv_spectra_amd.build [--jobs N] [--verbose]

Every source is compiled with packed-FP32 instructions disabled; the packer
is compiled without floating-point contraction so that each binary64 step
rounds on its own.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libspectra.so")
ARCH = "gfx950"

SOURCES = {
    "abi.hip": [],
    "pack.hip": ["-ffp-contract=off"],
    # the GEMV's 14 leading scalar arguments land in scalar registers at launch
    "gemv.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=14"],
    "mfma.hip": [],
    "step.hip": [],
    "image.cpp": [],  # host-only code
    "embed.hip": [],
    # k_kv_combine's scalar arguments preloaded into scalar registers as well
    "kv.hip": ["-ffp-contract=off", "-mllvm", "-amdgpu-kernarg-preload-count=14"],
}

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libspectra)")


def _compile(src: str, extra: list, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def build(jobs: int = 4, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max(1, jobs)) as ex:
        objs = list(ex.map(lambda kv: _compile(kv[0], kv[1], verbose), SOURCES.items()))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose))


if __name__ == "__main__":
    main()
