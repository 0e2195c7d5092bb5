"""Build libfa.so (HIP kernels for gfx950 + the C ABI) in place, next to this file.

    python -m exact_tiled_attention_forward_amd.build        # or build() from Python

Each source compiles to its own object under _build/ (in parallel), then hipcc links the
shared library.  Every HIP source is compiled with packed-fp32 instructions disabled.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")
ARCH = "gfx950"

SOURCES = ["fa_fwd.hip", "fa_bwd.hip", "fa_fp8.hip", "fa_api.cpp"]
# The race-check build: the same sources with -DFA_RACE_CHECK=1 (perturbed schedule,
# identical results; see csrc/fa_device.h).  Only the race-check tests load it.
RACECHECK_LIB = os.path.join(PKG, "libfa_racecheck.so")


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError(f"hipcc not found (looked for {cand})")
    return cand


def common_flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        "-Wno-unused-function",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE,
        "-I", CSRC,
    ]


def _compile(job) -> str:
    src, variant = job
    outdir = os.path.join(BUILD, variant) if variant else BUILD
    os.makedirs(outdir, exist_ok=True)
    obj = os.path.join(outdir, os.path.splitext(src)[0] + ".o")
    extra = ["-DFA_RACE_CHECK=1"] if variant == "racecheck" else []
    cmd = [hipcc(), *common_flags(), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in r.stderr.splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    return obj


def _link(objs, lib: str, verbose: bool):
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")


def build(verbose: bool = False) -> str:
    """Build libfa.so and the race-check build libfa_racecheck.so; returns the former."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(src, "") for src in SOURCES] + [(src, "racecheck") for src in SOURCES]
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = list(ex.map(_compile, jobs))
    _link(objs[:len(SOURCES)], LIB, verbose)
    _link(objs[len(SOURCES):], RACECHECK_LIB, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
