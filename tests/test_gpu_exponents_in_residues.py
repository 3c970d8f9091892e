"""Fast-mode scaling exponents computed inside the residue launch ("Profiling Ozaki II: The
Cost Behind Fast INT8 GEMMs", Part I section 2).

For small untransposed fast-mode products with inner dimensions up to 16 blocks of 256,
the residue launch combines each line's statistics partials itself instead of reading d
and b from a separate exponent launch.  A call that requests the A' dump takes the other
path (separate exponent launch, dumping residue kernels), so the two paths can be run on
the same inputs: d, b, every R_t plane, X and C must be identical, and d, b must equal
the oracle's exponents.  The inputs carry the cases the combination has to get right:
all-zero lines, lines whose leading or trailing blocks are zero, lines far below and
above 1 in magnitude, and block counts 1, 3, 16 (the largest on this path) and 17 (the
smallest off it), and the full-size 2048^3 product.
"""
import numpy as np
import pytest

import oracle
from fp64_gemm_emulation_amd.workloads import generate
from tests.gpu_helpers import assert_equal, log, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def oz():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    from fp64_gemm_emulation_amd import binding
    return binding


def _operands(p, q, r, seed):
    A = generate(p, q, 0.5, seed)
    B = generate(q, r, 0.5, seed + 1)
    A[min(5, p - 1), :] = 0.0                        # all-zero row
    B[:, min(3, r - 1)] = 0.0                        # all-zero column
    if q > 256:
        A[min(7, p - 1), :256] = 0.0                 # leading block zero
        B[256:, min(6, r - 1)] = 0.0                 # only the first block nonzero
    A[min(9, p - 1), :] *= 2.0 ** -600               # far below 1
    B[:, min(4, r - 1)] *= 2.0 ** 500                # far above 1
    A[min(11, p - 1), q // 2] = 3.0 ** 40            # one dominant element
    return A, B


@pytest.mark.parametrize("s,shape", [(s, shape) for s in (8, 14, 20)
                                     for shape in ((300, 517, 129), (257, 4096, 255), (64, 4097, 70), (40, 200, 33),
                                                   (1, 1, 1))]
                         + [(14, (2048, 2048, 2048)), (14, (1024, 4096, 1024))])
def test_exponents_in_residue_launch_match_the_exponent_launch(oz, shape, s):
    """The last two shapes have at least one row-statistics workgroup per compute unit, so
    the merged statistics launch also takes its rows-first order."""
    import torch
    p, q, r = shape
    A, B = _operands(p, q, r, 700 + q)
    Ad, Bd = to_device(A), to_device(B)
    log(f"[exp in residues] p,q,r={p},{q},{r} s={s}")
    inres = oz.dgemm_debug(Ad, Bd, s, "fast", want=("d", "b", "R", "X"))
    separate = oz.dgemm_debug(Ad, Bd, s, "fast", want=("d", "b", "Ap", "R", "X"))
    for k in ("d", "b", "R", "X"):
        assert torch.equal(inres[k], separate[k]), f"{k} differs between the two exponent paths"
    assert torch.equal(inres["C"].view(torch.int64), separate["C"].view(torch.int64)), "C differs"
    d_ref, _, _ = oracle.fast_exponents(A, s)
    b_ref, _, _ = oracle.fast_exponents(np.ascontiguousarray(B.T), s)
    assert_equal(inres["d"].cpu().numpy(), d_ref.astype(np.int32), "d")
    assert_equal(inres["b"].cpu().numpy(), b_ref.astype(np.int32), "b")
    log("[exp in residues] ok")


@pytest.mark.parametrize("s", [8, 14])
def test_exponents_in_residue_launch_with_padded_leading_dimensions(oz, s):
    """The same comparison with leading dimensions larger than the matrices (the residue
    launch's clamped element addresses run over each line's own stride)."""
    import torch
    p, q, r = 200, 700, 150
    A, B = _operands(p, q, r, 901)
    Abig = torch.full((q, p + 56), float("nan"), dtype=torch.float64, device="cuda").t()   # ld p + 56
    Abig[:p, :] = to_device(A)
    Bbig = torch.full((r, q + 100), float("nan"), dtype=torch.float64, device="cuda").t()  # ld q + 100
    Bbig[:q, :] = to_device(B)
    Ad, Bd = Abig[:p, :], Bbig[:q, :]
    log(f"[exp in residues] padded p,q,r={p},{q},{r} s={s}")
    inres = oz.dgemm_debug(Ad, Bd, s, "fast", want=("d", "b", "R", "X"))
    rc, flags = oz.ozaki2_get_flags()
    assert rc == oz.OZ2_OK and flags == 0  # the NaN padding is never read
    separate = oz.dgemm_debug(Ad, Bd, s, "fast", want=("d", "b", "Ap", "R", "X"))
    for k in ("d", "b", "R", "X"):
        assert torch.equal(inres[k], separate[k]), f"{k} differs between the two exponent paths"
    assert torch.equal(inres["C"].view(torch.int64), separate["C"].view(torch.int64)), "C differs"
    d_ref, _, _ = oracle.fast_exponents(A, s)
    assert_equal(inres["d"].cpu().numpy(), d_ref.astype(np.int32), "d")
    log("[exp in residues] ok")


@pytest.mark.parametrize("case", range(12))
def test_exponents_in_residue_launch_random_shapes(oz, case):
    """Seeded random shapes (p, r up to 700, q up to 6000, so both sides of the 16-block
    limit) and input spreads, both exponent paths compared as above."""
    import torch
    rng = np.random.default_rng(4100 + case)
    p, q, r = (int(rng.integers(1, 701)), int(rng.integers(1, 6001)), int(rng.integers(1, 701)))
    s = int(rng.choice([2, 6, 11, 14, 17, 20]))
    phi = float(rng.choice([0.0, 0.5, 1.0, 2.0]))
    A = generate(p, q, phi, 5000 + case)
    B = generate(q, r, phi, 6000 + case)
    Ad, Bd = to_device(A), to_device(B)
    log(f"[exp in residues] random case {case}: p,q,r={p},{q},{r} s={s} phi={phi}")
    inres = oz.dgemm_debug(Ad, Bd, s, "fast", want=("d", "b", "R", "X"))
    separate = oz.dgemm_debug(Ad, Bd, s, "fast", want=("d", "b", "Ap", "R", "X"))
    for k in ("d", "b", "R", "X"):
        assert torch.equal(inres[k], separate[k]), f"{k} differs between the two exponent paths"
    assert torch.equal(inres["C"].view(torch.int64), separate["C"].view(torch.int64)), "C differs"
    d_ref, _, _ = oracle.fast_exponents(A, s)
    b_ref, _, _ = oracle.fast_exponents(np.ascontiguousarray(B.T), s)
    assert_equal(inres["d"].cpu().numpy(), d_ref.astype(np.int32), "d")
    assert_equal(inres["b"].cpu().numpy(), b_ref.astype(np.int32), "b")
    log("[exp in residues] ok")
