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


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer (device code is
# built as usual): each -fsanitize applies to the host compilation only.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host",
                 "-fsanitize=undefined", "-Xarch_host",
                 "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def asan_runtime() -> str:
    """The shared AddressSanitizer runtime of the ROCm clang (to preload
    into an uninstrumented interpreter that loads a sanitized library)."""
    import glob
    c = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/"
                         "libclang_rt.asan-x86_64.so"))
    if not c:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found under "
                           "/opt/rocm/llvm")
    return c[-1]


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *common_flags(), *extra, "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n"
                           f"{r.stderr}")
    return obj


def _link(objs, out, extra=()):
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra,
           *objs, "-o", tmp]
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


def build_sanitized(out_dir: str, jobs: int = 8) -> str:
    """libdflash.so with host ASan + UBSan into out_dir (for the ABI
    validation tests on a machine without a GPU); returns its path."""
    os.makedirs(out_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, 16))) as ex:
        objs = list(ex.map(lambda f: _compile(f, out_dir, SANITIZE_HOST),
                           LIB_SOURCES))
    out = os.path.join(out_dir, "libdflash.so")
    _link(objs, out, SANITIZE_HOST)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=8)
    build(ap.parse_args().j, verbose=True)
