"""Host code of the library under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library's C ABI entry points validate their arguments on the host before any HIP
call, and the per-output reconstruction arithmetic (oz2_crt_round.hpp) is ordinary C++
that also compiles for the host.  Both are built here with the sanitizers on the host
code only (each -fsanitize after -Xarch_host; the library's objects also carry their
gfx950 device code, which is registered at load time but never launched) and run without a
GPU:
  * tests/host_abi_driver.cpp calls every product entry point with invalid arguments and
    empty shapes, the workspace arithmetic up to the largest accepted sizes, and the
    table / string / state queries, checking each documented return value;
  * tests/crt_harness.cpp runs the reconstruction on the exact-integer cases of
    test_crt_arith.py (ties, binade edges, the largest |X|, subnormal results), whose
    outputs must also equal the exact values.
Any sanitizer report makes the program exit nonzero.
"""
import os
import random
import struct
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from tests import test_crt_arith as crt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp64_gemm_emulation_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _hipcc(args, objs=(), device=False):
    """hipcc of the sources in args (as HIP), linking the objects objs; host code only, or
    with the gfx950 device code as in the library build (the sanitizers apply to the host
    code either way)."""
    target = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] if device \
        else ["--offload-host-only"]
    res = subprocess.run([HIPCC, *target, "-std=c++17", "-O1", "-g", *HOST_SAN,
                          f"-I{INCLUDE}", f"-I{CSRC}", "-x", "hip", *args,
                          *(["-x", "none", *objs] if objs else [])], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]


@pytest.fixture(scope="module")
def build_dir(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    return tmp_path_factory.mktemp("san")


@pytest.fixture(scope="module")
def abi_driver(build_dir):
    # the library's kernels are registered at load time, so its objects carry device code
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = [str(build_dir / (f[:-4] + ".o")) for f in srcs]
    with ThreadPoolExecutor(min(len(srcs), os.cpu_count() or 4)) as ex:
        list(ex.map(lambda so: _hipcc(["-fPIC", "-c", os.path.join(CSRC, so[0]), "-o", so[1]], device=True),
                    zip(srcs, objs)))
    exe = str(build_dir / "host_abi_driver")
    _hipcc([os.path.join(ROOT, "tests", "host_abi_driver.cpp"), "-o", exe], objs, device=True)
    return exe


@pytest.fixture(scope="module")
def crt_harness(build_dir):
    exe = str(build_dir / "crt_harness")
    _hipcc([os.path.join(ROOT, "tests", "crt_harness.cpp"), "-o", exe])
    return exe


def test_abi_validation_clean_under_sanitizers(abi_driver):
    res = subprocess.run([abi_driver], capture_output=True, text=True, env=ENV, timeout=120)
    assert res.returncode == 0 and res.stdout.strip().endswith("ok"), (res.stdout + res.stderr)[-3000:]
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr[-3000:]


@pytest.mark.parametrize("s", [2, 8, 14, 18, 20])
def test_crt_arithmetic_clean_under_sanitizers(crt_harness, s):
    rng = random.Random(3000 + s)
    ms = crt.moduli(s)
    cases = [(x, crt.scale_for(x, rng)) for x in crt.cases_for(s, rng)] + crt.subnormal_cases(s, rng)
    lines = [f"{s} {sc} " + " ".join(str(x % m) for m in ms) for x, sc in cases]
    res = subprocess.run([crt_harness], input="\n".join(lines) + "\n", capture_output=True, text=True, env=ENV,
                         timeout=300)
    assert res.returncode == 0, res.stderr[-3000:]
    assert "runtime error" not in res.stderr, res.stderr[-3000:]
    got = res.stdout.split("\n")[: len(cases)]
    for (x, sc), line in zip(cases, got):
        words = " ".join(f"{(x >> (32 * k)) & 0xFFFFFFFF:08x}" for k in range(5))
        bits = struct.unpack("<Q", struct.pack("<d", crt.rn_scaled(x, sc)))[0]
        assert line == f"{words} {bits:016x}", (x, sc, line)
