"""C-ABI checks that need no GPU: the library loads, exports every entry point the
header declares, validates arguments on the host before anything is launched, and
its compile-time constants agree with the oracle's independent derivation."""
import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "oz2.h")


@pytest.fixture(scope="module")
def lib():
    from fp64_gemm_emulation_amd import build as b
    if not os.path.exists(b.LIB_PATH):
        b.build()
    from fp64_gemm_emulation_amd import binding
    return binding


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(ozaki2_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_entry_points():
    names = declared_functions()
    for expected in ["ozaki2_dgemm", "ozaki2_dgemm_debug", "ozaki2_workspace_size", "ozaki2_set_workspace",
                     "ozaki2_timing_begin", "ozaki2_timing_end", "ozaki2_get_flags", "ozaki2_moduli",
                     "ozaki2_tau", "ozaki2_status_string", "ozaki2_release"]:
        assert expected in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_moduli_and_tau_match_oracle(lib):
    for s in range(oracle.MIN_S, oracle.MAX_S + 1):
        rc, mods = lib.ozaki2_moduli(s)
        assert rc == lib.OZ2_OK
        assert mods == oracle.moduli(s)
        assert lib.ozaki2_tau(s) == oracle.tau(s)
    assert lib.ozaki2_moduli(1)[0] == lib.OZ2_ERR_ARG
    assert lib.ozaki2_moduli(21)[0] == lib.OZ2_ERR_ARG
    assert lib.ozaki2_tau(21) == -1


def test_argument_validation_before_launch(lib):
    """Invalid arguments return an error before any HIP call (so this runs without a GPU)."""
    A, B, C = 0x10000, 0x20000000, 0x40000000  # never dereferenced
    call = lib.ozaki2_dgemm
    ok = dict(p=8, q=8, r=8, A=A, lda=8, B=B, ldb=8, C=C, ldc=8, s=8, mode=0, stream=None)

    def run(**kw):
        a = dict(ok)
        a.update(kw)
        return call(a["p"], a["q"], a["r"], a["A"], a["lda"], a["B"], a["ldb"], a["C"], a["ldc"],
                    a["s"], a["mode"], a["stream"])

    assert run(s=1) == lib.OZ2_ERR_ARG
    assert run(s=21) == lib.OZ2_ERR_ARG
    assert run(mode=2) == lib.OZ2_ERR_ARG
    assert run(p=-1) == lib.OZ2_ERR_ARG
    assert run(lda=7) == lib.OZ2_ERR_ARG
    assert run(ldb=7) == lib.OZ2_ERR_ARG
    assert run(ldc=7) == lib.OZ2_ERR_ARG
    assert run(C=None) == lib.OZ2_ERR_ARG
    assert run(A=None) == lib.OZ2_ERR_ARG
    assert run(q=524288, ldb=524288) == lib.OZ2_ERR_UNSUPPORTED   # beyond OZ2_MAX_Q
    assert run(C=A + 8) == lib.OZ2_ERR_ARG          # C overlaps A
    assert run(p=0) == lib.OZ2_OK                     # empty: no work, nothing launched
    assert run(r=0) == lib.OZ2_OK
    assert lib.ozaki2_dgemm_debug(8, 8, 8, A, 8, B, 8, C, 8, 1, 0, None, None) == lib.OZ2_ERR_ARG


def test_noalloc_checks_before_launch(lib):
    """ozaki2_dgemm_noalloc validates like ozaki2_dgemm and rejects a product whose workspace
    exceeds its fixed scratch, all before any HIP call (so this runs without a GPU)."""
    A, B, C = 0x10000, 0x20000000, 0x40000000  # never dereferenced
    call = lib.ozaki2_dgemm_noalloc
    assert call(8, 8, 8, A, 8, B, 8, C, 8, 1, 0, None) == lib.OZ2_ERR_ARG
    assert call(8, 8, 8, A, 8, B, 8, C, 8, 8, 2, None) == lib.OZ2_ERR_ARG
    assert call(8, 8, 8, A, 8, B, 8, None, 8, 8, 0, None) == lib.OZ2_ERR_ARG
    assert call(0, 8, 8, A, 8, B, 8, C, 8, 8, 0, None) == lib.OZ2_OK
    big = (4096, 4096, 4096, 14)
    assert lib.ozaki2_workspace_size(*big, 0) > lib.OZ2_NOALLOC_SCRATCH_BYTES
    n, _, _, s = big
    assert call(n, n, n, A, n, B, n, C, n, s, 0, None) == lib.OZ2_ERR_WORKSPACE
    assert "ozaki2_dgemm_noalloc" in lib.ozaki2_status_string(lib.OZ2_ERR_WORKSPACE)
    # square products at the largest s the scratch holds (documented in the header)
    for n, s_max in ((2048, 20), (3072, 9), (4096, 5)):
        assert lib.ozaki2_workspace_size(n, n, n, s_max, 1) <= lib.OZ2_NOALLOC_SCRATCH_BYTES
        if s_max < 20:
            assert lib.ozaki2_workspace_size(n, n, n, s_max + 1, 0) > lib.OZ2_NOALLOC_SCRATCH_BYTES
    # the raw P_t dump is exact int32 only without K-blocking
    dump = lib.OZ2Dump(P=0x60000000)
    q = lib.OZ2_MAX_Q_P_DUMP + 1
    assert lib.ozaki2_dgemm_debug(8, q, 8, A, 8, B, q, C, 8, 8, 0, None, dump) == lib.OZ2_ERR_UNSUPPORTED


def test_ex_argument_validation_before_launch(lib):
    """ozaki2_dgemm_ex: operation codes and the leading dimensions of transposed operands."""
    A, B, C = 0x10000, 0x20000000, 0x40000000  # never dereferenced
    N, T = lib.OZ2_OP_N, lib.OZ2_OP_T
    ok = dict(ta=N, tb=N, p=8, q=6, r=4, alpha=1.0, A=A, lda=8, B=B, ldb=6, beta=0.0, C=C, ldc=8, s=8, mode=0)

    def run(**kw):
        a = dict(ok)
        a.update(kw)
        return lib.ozaki2_dgemm_ex(a["ta"], a["tb"], a["p"], a["q"], a["r"], a["alpha"], a["A"], a["lda"], a["B"],
                                   a["ldb"], a["beta"], a["C"], a["ldc"], a["s"], a["mode"], None)

    assert run(ta=2) == lib.OZ2_ERR_ARG
    assert run(tb=-1) == lib.OZ2_ERR_ARG
    assert run(lda=7) == lib.OZ2_ERR_ARG                 # A is p x q: lda >= p
    assert run(ta=T, lda=5) == lib.OZ2_ERR_ARG           # A is q x p: lda >= q
    assert run(ldb=5) == lib.OZ2_ERR_ARG                 # B is q x r: ldb >= q
    assert run(tb=T, ldb=3) == lib.OZ2_ERR_ARG           # B is r x q: ldb >= r
    assert run(C=A + 8) == lib.OZ2_ERR_ARG               # C overlaps A
    assert run(ta=T, C=A + 8 * 6 * 7) == lib.OZ2_ERR_ARG  # last element of the q x p A
    assert run(p=0) == lib.OZ2_OK
    assert run(s=21) == lib.OZ2_ERR_ARG


def test_workspace_size(lib):
    ws = lib.ozaki2_workspace_size
    assert ws(0, 8, 8, 8, 0) == 0
    assert ws(8, 8, 8, 1, 0) == 0
    assert ws(8, 524288, 8, 8, 0) == 0
    assert ws(8, 131072, 8, 8, 0) > 0                  # K-blocked inner dimensions
    small = ws(100, 100, 100, 8, 0)
    assert small > 0 and small % 256 == 0
    assert ws(100, 100, 100, 14, 0) > small
    # int8 operand planes and residue planes dominate: s (p_pad q_pad + r_pad q_pad + r_pad p_pad)
    n = 8192
    assert ws(n, n, n, 14, 0) >= 14 * 3 * n * n
    assert lib.ozaki2_set_workspace(0x101, 1024) == lib.OZ2_ERR_ARG   # misaligned
    assert lib.ozaki2_set_workspace(None, 0) == lib.OZ2_OK


def test_status_strings(lib):
    for code in range(5):
        assert isinstance(lib.ozaki2_status_string(code), str)
    assert "unknown" in lib.ozaki2_status_string(99)


def test_calibration_library_exports_entry_point(lib):
    """bench.py's MFMA-ceiling aid is a separate library: built beside liboz2.so, with its
    entry point exported and its argument checks answering without a launch."""
    from fp64_gemm_emulation_amd import build as b
    assert os.path.exists(b.CALIB_LIB)
    calib = ctypes.CDLL(b.CALIB_LIB)
    fn = calib.oz2calib_mfma_i8
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    assert fn(None, 1, 1, None, None) == 1
    assert fn(ctypes.c_void_p(16), 0, 1, ctypes.c_void_p(16), None) == 1


def test_tensor_wrappers_reject_bad_operands_before_the_library(lib):
    """The torch conveniences check shapes, dtypes and devices on the host and raise
    before any library call (nothing here touches a GPU)."""
    import torch
    a = torch.zeros(4, 3, dtype=torch.float64)
    b = torch.zeros(3, 5, dtype=torch.float64)
    with pytest.raises(ValueError, match="inner dimensions"):
        lib.dgemm(a, torch.zeros(4, 5, dtype=torch.float64))
    with pytest.raises(ValueError, match="wrong shape"):
        lib.dgemm(a, b, out=torch.zeros(5, 4, dtype=torch.float64))
    with pytest.raises(ValueError):          # host tensors are not device memory
        lib.dgemm(a, b)
    with pytest.raises(ValueError, match="beta != 0 needs C"):
        lib.dgemm_ex(a, b, beta=1.0)
    with pytest.raises(ValueError, match="wrong shape"):
        lib.dgemm_ex(a, b, C=torch.zeros(4, 4, dtype=torch.float64))


def test_stage_times_need_a_timed_call(lib):
    """ozaki2_get_stage_ms answers on the host when there is nothing to report."""
    import ctypes as ct
    assert lib._LIB.ozaki2_get_stage_ms(None) == lib.OZ2_ERR_ARG
    rc, _ = lib.ozaki2_get_stage_ms()
    assert rc == lib.OZ2_ERR_ARG          # no call has been timed in this process
