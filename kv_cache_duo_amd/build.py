"""Build libduo.so (gfx950 HIP kernels + C ABI) in-tree with hipcc.

Usage: python -m kv_cache_duo_amd.build   (or call build()).
Objects go to _build/ at the repository root; the shared library is written
next to this file, where the Python binding loads it.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libduo.so")
CEILING = os.path.join(HERE, "ceiling")  # measured HBM / MFMA ceilings (standalone)

SOURCES = ["duo_api.cpp", "append.hip", "decode.hip", "prefill.hip", "prefill_fp8.hip"]

ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 VALU instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # one lane issues the decode's pair-claim atomic; the atomic optimizer
    # would add a wave scan and wait for the result at once
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    if not os.path.exists(path):
        found = shutil.which("hipcc")
        if found is None:
            raise RuntimeError("hipcc not found; set ROCM_PATH")
        path = found
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libduo.so; return its path."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    cmd = [hipcc(), *COMMON, "-x", "hip", os.path.join(CSRC, "ceiling.hip"), "-o", CEILING + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for ceiling.hip:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(CEILING + ".tmp", CEILING)
    if verbose:
        print(f"built {LIB} and {CEILING}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
