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


# What a built library was made from: written beside libduo.so by build(),
# checked by the binding before it loads the library.
RECORD_NAME = "libduo.build.json"
BUILD_RECORD = os.path.join(HERE, RECORD_NAME)


def source_digest() -> str:
    """sha256 over the library's sources, its headers and the compile flags."""
    import hashlib
    h = hashlib.sha256()
    h.update(" ".join(f for f in COMMON if not f.startswith("-I")).encode())  # paths differ between machines
    names = sorted(SOURCES + [f for f in os.listdir(CSRC) if f.endswith(".h")])
    for name in names:
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    with open(os.path.join(INCLUDE, "duo.h"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()


def write_record(path: str) -> None:
    import json
    with open(path + ".tmp", "w") as f:
        json.dump({"sources_sha256": source_digest(), "arch": ARCH}, f)
    os.replace(path + ".tmp", path)


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
    write_record(BUILD_RECORD)
    cmd = [hipcc(), *COMMON, "-x", "hip", os.path.join(CSRC, "ceiling.hip"), "-o", CEILING + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for ceiling.hip:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(CEILING + ".tmp", CEILING)
    if verbose:
        print(f"built {LIB} and {CEILING}")
    return LIB


def sanitizer_runtime() -> str:
    """The compiler's AddressSanitizer runtime (it carries the
    UndefinedBehaviorSanitizer handlers too), to preload into a process that
    loads a sanitized host library."""
    import glob
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    found = sorted(glob.glob(os.path.join(rocm, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    if not found:
        raise RuntimeError("clang AddressSanitizer runtime not found under ROCM_PATH")
    return found[-1]


def build_host_sanitized(out_dir: str) -> str:
    """libduo.so with its host code (duo_api.cpp: validation, layout, page
    bookkeeping) built with AddressSanitizer and UndefinedBehaviorSanitizer.
    Device code is not instrumented (each -fsanitize= applies to the host
    pass only); the kernels' objects come from the last build().  Load it
    with sanitizer_runtime() preloaded.  Returns the library's path."""
    os.makedirs(out_dir, exist_ok=True)
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "duo_api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in COMMON if f != "-O3"]
    api = os.path.join(out_dir, "duo_api_san.o")
    cmd = [hipcc(), *flags, "-O1", "-g", *san, "-x", "hip", "-c", os.path.join(CSRC, "duo_api.cpp"), "-o", api]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for the sanitized host build:\n{' '.join(cmd)}\n{r.stderr}")
    lib = os.path.join(out_dir, "libduo.so")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *san, api, *objs, "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed for the sanitized host build:\n{' '.join(cmd)}\n{r.stderr}")
    write_record(os.path.join(out_dir, RECORD_NAME))
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
