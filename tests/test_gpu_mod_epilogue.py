"""The GEMM epilogue's output reduction R_t = P_t mod m_t ("Profiling Ozaki II: The Cost
Behind Fast INT8 GEMMs", Part I section 1, blue stage) at large |P|, on every modulus and
every output element, against exact integer arithmetic.

Random residues keep |P| near sqrt(q) 10^4, far below the range the reduction must cover.
The residue-plane GEMM of the calibration library (calib/gemm_tile_probe.hip) uses the
library's own epilogue helpers (the modulus constants, the per-value reduction and the
packing of four residues per word) on caller-supplied int8 operand planes, so it can be
driven with chosen operands: with A_t[i, k] = a_i over the first half of the inner
dimension and a2_i over the second, and B_t[k, j] = b_j / b2_j likewise, every output is
P_ij = (K / 2)(a_i b_j + a2_i b2_j) exactly, the a's and b's run over all of [-128, 127],
and at K = 16384 |P| reaches 2^28 with both signs.  The expected residues are computed
with int64 integer arithmetic, independently of the kernels.
"""
import ctypes
import os

import pytest

import oracle
from tests.gpu_helpers import log

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
N = 16384
S = 20


@pytest.fixture(scope="module")
def calib():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    path = os.path.join(ROOT, "fp64_gemm_emulation_amd", "libozcalib.so")
    if not os.path.exists(path):
        pytest.fail("libozcalib.so is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    lib.oz2calib_gemm_tiles.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_void_p]
    lib.oz2calib_gemm_tiles.restype = ctypes.c_int
    return lib


def _values(mult, add):
    """n values covering every int8 value, in a scattered order."""
    import torch
    idx = torch.arange(N, dtype=torch.int64, device="cuda")
    return ((idx * mult + add) % 256 - 128).to(torch.int8)


def _plane(first, second):
    """One n x n operand plane in the library's tile layout ([256-row block][64-byte stage]
    [256 rows][64 bytes], chunks swizzled within a row): row i holds first[i] over the
    first half of the inner dimension and second[i] over the second half (constant within
    a row's stage segment, so the chunk swizzle does not matter)."""
    import torch
    stages = N // 64
    p = torch.empty((N // 256, stages, 256, 64), dtype=torch.int8, device="cuda")
    p[:, : stages // 2] = first.view(N // 256, 1, 256, 1)
    p[:, stages // 2:] = second.view(N // 256, 1, 256, 1)
    return p.view(-1)


@pytest.mark.parametrize("tile", [256, 128])
def test_mod_reduction_at_large_products_every_modulus(calib, tile):
    import torch
    a, a2 = _values(37, 11), _values(101, 5)
    b, b2 = _values(53, 7), _values(29, 200)
    pa, pb = _plane(a, a2), _plane(b, b2)
    at = pa.repeat(S)
    bt = pb.repeat(S)
    res = torch.empty(S * N * N, dtype=torch.uint8, device="cuda")
    res.fill_(0xEE)
    log(f"[mod epilogue] tile={tile} n=q={N} s={S}")
    rc = calib.oz2calib_gemm_tiles(at.data_ptr(), bt.data_ptr(), N, S, tile, res.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    mods = oracle.moduli(S)
    half = N // 2
    a64, a264, b64, b264 = (v.to(torch.int64) for v in (a, a2, b, b2))
    pmax = 0
    chunk = 1024
    for j0 in range(0, N, chunk):
        # P[i, j] for columns j0 .. j0 + chunk - 1, exact in int64
        p = half * (a64[:, None] * b64[None, j0:j0 + chunk] + a264[:, None] * b264[None, j0:j0 + chunk])
        pmax = max(pmax, int(p.abs().max()))
        for t, m in enumerate(mods):
            want = torch.remainder(p, m).to(torch.uint8).t()           # [chunk (j), N (i)]
            got = res[t * N * N:(t + 1) * N * N].view(N, N)[j0:j0 + chunk]  # column-major plane
            if not torch.equal(got, want):
                bad = (got != want).nonzero()[0].tolist()
                jj, ii = j0 + bad[0], bad[1]
                raise AssertionError(f"tile {tile}, modulus {m}: R[{ii},{jj}] = {int(got[bad[0], ii])}, "
                                     f"want {int(want[bad[0], ii])} (P = {int(p[ii, bad[0]])})")
    assert pmax >= 1 << 27
    log(f"[mod epilogue] ok: every element of {S} planes, |P| up to {pmax}")
