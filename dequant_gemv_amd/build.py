"""Build the HIP library ``libdqg.so`` in-tree for gfx950 with hipcc.

Run ``python -m dequant_gemv_amd.build`` (or ``__graft_entry__.build()``).  It always
recompiles.  Objects go to ``_build/`` at the repository root; the shared library lands
next to this file, where the binding loads it from.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdqg.so")
SOURCES = ["dqg_kernels.hip", "dqg_experts.hip", "dqg_fused.hip", "dqg_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + common_flags()
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-o", tmp] + objs + [f"--offload-arch={ARCH}", "-fPIC"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the C ABI layer (argument
# checks, workspace layout, plan selection).  Only the host pass of dqg_api.cpp is
# instrumented (every -fsanitize= goes through -Xarch_host); the kernel objects of the normal
# build are linked in unchanged.  The result is loaded with the ASan runtime preloaded, on
# the CPU only: it is a checking build, never the library the product loads.
SAN_LIB = os.path.join(BUILD, "san", "libdqg.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
             "-fno-omit-frame-pointer", "-Xarch_host", "-shared-libsan"]


def asan_runtime() -> str:
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the clang ASan runtime was not found next to hipcc")
    return path


def build_sanitized(verbose: bool = True) -> str:
    san = os.path.dirname(SAN_LIB)
    os.makedirs(san, exist_ok=True)
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES
            if s != "dqg_api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        build(verbose)
    api_obj = os.path.join(san, "dqg_api.o")
    cmd = ([hipcc(), "-x", "hip", "-c", os.path.join(CSRC, "dqg_api.cpp"), "-o", api_obj]
           + common_flags() + ["-g"] + SAN_FLAGS)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    cmd = ([hipcc(), "-shared", "-o", SAN_LIB] + objs + [api_obj, f"--offload-arch={ARCH}",
                                                          "-fPIC"] + SAN_FLAGS)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {SAN_LIB}", file=sys.stderr)
    return SAN_LIB


if __name__ == "__main__":
    build_sanitized() if "--sanitize" in sys.argv[1:] else build()
