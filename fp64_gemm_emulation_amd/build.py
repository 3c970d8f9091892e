"""Build the HIP libraries for gfx950 in-tree.

Each ``csrc/*.hip`` file is compiled to an object with hipcc in parallel, then the
objects are linked into ``fp64_gemm_emulation_amd/liboz2.so`` (the library).  The
measurement aids ``calib/*.hip`` become ``libozcalib.so``, loaded by bench.py and by the
GPU test that drives the GEMM epilogue with chosen operand planes; the product path never
loads it.  Packed FP32 instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
OBJ_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "liboz2.so")
CALIB_DIR = os.path.join(PKG_DIR, "calib")
CALIB_LIB = os.path.join(PKG_DIR, "libozcalib.so")
INCLUDE = os.path.join(ROOT, "include")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every HIP source and link liboz2.so; returns the library path."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)), 16)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    tmp = CALIB_LIB + ".tmp"
    calib_srcs = sorted(os.path.join(CALIB_DIR, f) for f in os.listdir(CALIB_DIR) if f.endswith(".hip"))
    cmd = [HIPCC, *COMMON_FLAGS, "-shared", "-o", tmp, *calib_srcs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {calib_srcs}:\n{res.stderr}")
    os.replace(tmp, CALIB_LIB)
    if verbose:
        print(f"built {LIB_PATH} and {CALIB_LIB}", file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
