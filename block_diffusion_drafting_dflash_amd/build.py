"""Build libdflash.so and libdflash_harness.so in-tree for gfx950 with hipcc.

Usage: python -m block_diffusion_drafting_dflash_amd.build [-j N]
Every call recompiles (no staleness check); objects go to _build/.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
ARCH = "gfx950"

LIB_SOURCES = ["dflash_api.hip", "gemm.hip", "gemm_tiled.hip", "epilogue.hip",
               "attention.hip", "head.hip"]
HARNESS_SOURCES = ["harness.hip"]

LIB = os.path.join(PKG, "libdflash.so")
HARNESS_LIB = os.path.join(PKG, "libdflash_harness.so")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc",
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm 7.x expected under /opt/rocm)")


def common_flags():
    # DFLASH_HIPCC_FLAGS adds compiler flags (e.g. -D tuning overrides)
    extra = os.environ.get("DFLASH_HIPCC_FLAGS", "").split()
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", *extra,
            # hipcc -O3 forms packed fp32 ops by itself; keep them off
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            "-Wall", "-Wno-unused-function"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n"
                           f"{r.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o",
           tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, out)


def build(jobs: int = 8, verbose: bool = False) -> None:
    os.makedirs(BUILD, exist_ok=True)
    srcs = LIB_SOURCES + HARNESS_SOURCES
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, 16))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in LIB_SOURCES], LIB)
    _link([objs[s] for s in HARNESS_SOURCES], HARNESS_LIB)
    if verbose:
        print(f"built {LIB} and {HARNESS_LIB}")


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=8)
    build(ap.parse_args().j, verbose=True)
