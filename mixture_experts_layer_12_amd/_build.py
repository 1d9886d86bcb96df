"""Build the HIP library libcolibri_moe.so for gfx950, in-tree.

Each source under csrc/ is compiled to an object with hipcc (in parallel), then
the objects are linked into one shared library next to this file.  The two
measurement kernels of csrc/ceilings.hip (used by the benchmark only) go into
a library of their own, libcolibri_ceilings.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libcolibri_moe.so")
CEIL_LIB = os.path.join(PKG, "libcolibri_ceilings.so")
CEIL_SOURCES = ["ceilings.hip"]

SOURCES = ["abi.cpp", "validate.cpp", "route.hip", "dispatch.hip", "ffn.hip", "ffn_gemm.hip", "ffn_decode.hip", "combine.hip",
           "quantize.hip", "ffn_decode_q4.hip"]
ARCH = os.environ.get("COLIBRI_OFFLOAD_ARCH", "gfx950")

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return h


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *HIP_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; drop that line
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err)
    return obj


def _link(objs, lib: str):
    tmp = lib + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES) + len(CEIL_SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES + CEIL_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], CEIL_LIB)
    if verbose:
        print(f"built {LIB} and {CEIL_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
