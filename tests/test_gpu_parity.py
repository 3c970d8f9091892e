"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer intermediates (d, b, A', B', A_t, B_t, P_t, R_t, X and, for accu, e, f, Abar,
Bbar, rho, gamma) must be bit-exact; the FP64 result C must satisfy
|C_gpu - C_oracle|_ij <= 4 * 2^-53 * (|A||B|)_ij.  Small and ragged shapes are compared
in full; the full-size workloads are compared on sampled rows and columns.
"""
import numpy as np
import pytest

import oracle
from fp64_gemm_emulation_amd.workloads import WORKLOADS, generate
from tests.gpu_helpers import (compare_full, compare_sampled, log, sample_indices, to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def oz():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    from fp64_gemm_emulation_amd import binding
    return binding


def _full_case(oz, A, B, s, mode, label):
    log(f"[full] {label}: p,q,r={A.shape[0]},{A.shape[1]},{B.shape[1]} s={s} mode={mode}")
    out = oz.dgemm_debug(to_device(A), to_device(B), s, mode)
    ref = oracle.ozaki2(A, B, s, mode)
    ndiff = compare_full(out, ref, A, B, s, mode)
    log(f"[full] {label}: ok ({ndiff} C entries differ from the correctly rounded value)")
    return out, ref


def test_workload_n256_fast_s8_full(oz):
    w = WORKLOADS["n256_fast_s8"]
    A, B = w.inputs()
    _full_case(oz, A, B, w.s, w.mode, w.name)


@pytest.mark.parametrize("mode", ["fast", "accu"])
@pytest.mark.parametrize("shape", [(300, 517, 129), (1, 1, 1), (257, 256, 255), (513, 1000, 70), (5, 2049, 3),
                                   (70, 9000, 45)])
def test_ragged_shapes(oz, mode, shape):
    p, q, r = shape
    A = generate(p, q, 1.0, 11 + p)
    B = generate(q, r, 1.0, 12 + r)
    _full_case(oz, A, B, 14, mode, f"ragged{shape}")


@pytest.mark.parametrize("mode", ["fast", "accu"])
@pytest.mark.parametrize("s", list(range(2, 21)))
def test_every_modulus_count(oz, mode, s):
    A = generate(70, 300, 1.0, 100 + s)
    B = generate(300, 45, 1.0, 200 + s)
    _full_case(oz, A, B, s, mode, f"s{s}")


@pytest.mark.parametrize("case", range(16))
def test_random_small_shapes(oz, case):
    """Seeded random shapes (each dimension 1..399), moduli counts, modes and exponent
    spreads, every intermediate compared."""
    rng = np.random.default_rng(9000 + case)
    p, q, r = (int(x) for x in rng.integers(1, 400, size=3))
    s = int(rng.integers(2, 21))
    mode = ("fast", "accu")[case % 2]
    phi = float(rng.choice([0.5, 1.0, 2.0]))
    A = generate(p, q, phi, 9100 + case)
    B = generate(q, r, phi, 9200 + case)
    _full_case(oz, A, B, s, mode, f"random {case} phi={phi}")


@pytest.mark.parametrize("mode", ["fast", "accu"])
def test_edge_values(oz, mode):
    A = generate(64, 300, 4.0, 5)          # very wide exponent spread
    B = generate(300, 40, 4.0, 6)
    A[3, :] = 0.0                           # zero row
    B[:, 7] = 0.0                           # zero column
    A[5, 10] = 5e-324                       # subnormals
    A[6, :20] = -3e-310
    B[11, 2] = 1e300                        # huge
    B[12, 3] = -1e-300
    A[9, :] = 1.0                           # flat row
    _full_case(oz, A, B, 14, mode, "edges")


@pytest.mark.parametrize("mode", ["fast", "accu"])
def test_lines_whose_products_all_vanish(oz, mode):
    """A nonzero row of A supported only on zero rows of B (accu: bound peak rho = 0) and a
    nonzero column of B supported only on zero columns of A (gamma = 0): the exponents of
    such lines (scaled as lines of peak 1 in accu), their truncations and residues, and
    their exactly zero outputs, bit-exact against the oracle."""
    A = generate(70, 300, 1.0, 41)
    B = generate(300, 45, 1.0, 42)
    A[:, 40:48] = 0.0
    B[:, 9] = 0.0
    B[40:48, 9] = generate(8, 1, 3.0, 43)[:, 0] * 1e150     # column 9 of B meets only zero columns of A
    B[200:203, :] = 0.0
    A[17, :] = 0.0
    A[17, 200:203] = [-3e-250, 1e-249, 7e-251]              # row 17 of A meets only zero rows of B
    out, ref = _full_case(oz, A, B, 14, mode, "vanishing lines")
    if mode == "accu":
        assert int(ref["rho"][17]) == 0 and int(ref["gamma"][9]) == 0
    c = out["C"].cpu().numpy()
    assert not c[17, :].any() and not c[:, 9].any()


@pytest.mark.parametrize("mode", ["fast", "accu"])
def test_subnormal_results_rounded_once(oz, mode):
    """Entries of C below 2^-1022, s = 20: rows of A scaled by 2^-1000 against columns of B
    scaled by 2^-60 (normal inputs, subnormal products), a row of subnormal entries of A,
    and rows built so that (AB)_ij = 2^-1074 (Y + 1/2 -+ 2^-56) exactly, where rounding X to
    53 bits and then scaling lands on the tie and rounds to the wrong neighbour.  Every entry
    must be the correctly rounded RN(X 2^-(d_i + b_j)), one rounding at the subnormal unit."""
    A = generate(60, 300, 1.0, 81)
    B = generate(300, 40, 1.0, 82)
    A[:20, :] = np.ldexp(A[:20, :], -1000)
    B[:, :15] = np.ldexp(B[:, :15], -60)
    A[25, :] = np.ldexp(A[25, :], -1060)            # subnormal inputs
    B[:, 30:34] = 0.0
    B[0:2, 30:34] = 2.0 ** -75
    for k, (y, sgn) in enumerate([(5, -1), (4, 1), (1, -1), (2, 1), (1001, -1), (1000, 1)]):
        for neg in (False, True):
            i = 40 + 2 * k + neg
            A[i, :] = 0.0
            A[i, 0] = (2 * y + 1) * 2.0 ** -1000
            A[i, 1] = sgn * 2.0 ** -1055
            if neg:
                A[i, :2] = -A[i, :2]
    out, ref = _full_case(oz, A, B, 20, mode, "subnormal C")
    c = ref["C"]
    tiny = (c != 0) & (np.abs(c) < 2.0 ** -1022)
    assert tiny.sum() > 500, "the case must produce subnormal results"
    d, b = ref["d"], ref["b"]
    twice = sum(1 for i, j in zip(*np.nonzero(tiny))
                if np.ldexp(float(int(ref["X"][i, j])), -int(d[i] + b[j])) != c[i, j])
    assert twice >= 48, "the built rows must reach results that two roundings get wrong"
    assert np.array_equal(out["C"].cpu().numpy()[40:52, 30] / 2.0 ** -1074,
                          [5, -5, 5, -5, 1, -1, 3, -3, 1001, -1001, 1001, -1001])


def _block_spread(rows, q, seed):
    """rows x q with every 256-long block of a line at its own scale: exponent gaps to the
    line maximum of 0, 3, 7, 9 and about 1000, an all-zero block, a block of subnormals,
    and the line maximum sometimes in the short last block."""
    rng = np.random.default_rng(seed)
    X = generate(rows, q, 0.5, seed)
    nblk = (q + 255) // 256
    shifts = [0, -3, -7, -9, -1000, None, -1060]
    for i in range(rows):
        order = rng.permutation(len(shifts))[:nblk]
        for b in range(nblk):
            sh = shifts[order[b]]
            sl = slice(256 * b, min(256 * (b + 1), q))
            if sh is None:
                X[i, sl] = 0.0
            else:
                X[i, sl] = np.ldexp(X[i, sl], sh)
    return X


@pytest.mark.parametrize("s", [14, 18])
@pytest.mark.parametrize("mode", ["fast", "accu"])
def test_lines_near_the_scaled_bound(oz, mode, s):
    """Lines whose mass sits in one element are scaled up to |A'| near the bound 2^(tau/2),
    beside dense lines several bits below it, through the production residue kernels (no
    A' / B' dump).  d, b, A_t, B_t, R_t, X (and accu's e, f, rho, gamma, Abar, Bbar)
    bit-exact and C within tolerance, in full."""
    p, q, r = 200, 700, 150
    A = generate(p, q, 0.5, 71 + s)
    B = generate(q, r, 0.5, 72 + s)
    for i in (0, 37, 150, 199):
        A[i, (5 * i) % q] = 1e6
    A[198, :] = 0.0  # a single nonzero element: the scaled line reaches the bound itself
    A[198, 3] = 7e5
    for j in (3, 90, 149):
        B[(7 * j) % q, j] = -3e5
    # no A' / B' dump: the production residue kernels run, and their A_t, B_t are compared
    label = f"near-bound s{s} {mode}"
    log(f"[full] {label}: p,q,r={p},{q},{r}")
    want = ("d", "b", "At", "Bt", "R", "X") + (("e", "f", "rho", "gamma", "Abar", "Bbar") if mode == "accu" else ())
    out = oz.dgemm_debug(to_device(A), to_device(B), s, mode, want=want)
    ref = oracle.ozaki2(A, B, s, mode)
    compare_full(out, ref, A, B, s, mode)
    # the dominant lines reach |A'| >= 2^53, where the second digit word of the residue
    # kernels carries nonzero digits
    top_a = out["d"].cpu().numpy().astype(np.int64) + np.frexp(np.abs(A).max(axis=1))[1]
    assert top_a.max() >= 54, int(top_a.max())
    log(f"[full] {label}: ok")


@pytest.mark.parametrize("mode", ["fast", "accu"])
def test_block_exponent_spread(oz, mode):
    """Blocks of one line far apart in scale: the block exponents, the accu bound inputs
    formed from them, and every later stage, bit-exact against the oracle."""
    A = _block_spread(70, 1100, 61)
    B = _block_spread(33, 1100, 62).T.copy()
    _full_case(oz, A, B, 14, mode, "block spread")


@pytest.mark.parametrize("mode", ["fast", "accu"])
def test_small_integers_exact(oz, mode):
    rng = np.random.default_rng(3)
    A = rng.integers(-1000, 1001, size=(90, 200)).astype(np.float64)
    B = rng.integers(-1000, 1001, size=(200, 77)).astype(np.float64)
    out, ref = _full_case(oz, A, B, 14, mode, "integers")
    exact = (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float64)
    assert np.array_equal(out["C"].cpu().numpy(), exact)


def test_inner_dimension_zero_gives_zero(oz):
    import torch
    A = torch.empty((5, 0), dtype=torch.float64, device="cuda")
    B = torch.empty((0, 4), dtype=torch.float64, device="cuda")
    C = oz.empty_colmajor(5, 4)
    C.fill_(7.0)
    rc = oz.ozaki2_dgemm(5, 0, 4, 0, 5, 0, 1, C.data_ptr(), 5, 8, 0, torch.cuda.current_stream().cuda_stream)
    assert rc == oz.OZ2_OK
    torch.cuda.synchronize()
    assert not C.cpu().numpy().any()


@pytest.mark.parametrize("mode", ["fast", "accu"])
def test_nonfinite_flagged(oz, mode):
    """A non-finite input sets the flag of that call and only that call: untransposed operands
    (one residue launch for both), a transposed A and a NaN in B (one launch each)."""
    import torch
    A = generate(40, 64, 0.5, 1)
    B = generate(64, 30, 0.5, 2)
    A[3, 4] = np.inf
    oz.dgemm(to_device(A), to_device(B), 8, mode)
    rc, flags = oz.ozaki2_get_flags()
    assert rc == oz.OZ2_OK and flags & 1
    oz.dgemm(to_device(generate(40, 64, 0.5, 1)), to_device(B), 8, mode)
    rc, flags = oz.ozaki2_get_flags()
    assert rc == oz.OZ2_OK and flags == 0
    oz.dgemm_ex(to_device(A.T.copy()), to_device(B), transa=True, s=8, mode=mode)
    rc, flags = oz.ozaki2_get_flags()
    assert rc == oz.OZ2_OK and flags & 1
    B2 = B.copy()
    B2[10, 7] = np.nan
    oz.dgemm(to_device(generate(40, 64, 0.5, 1)), to_device(B2), 8, mode)
    rc, flags = oz.ozaki2_get_flags()
    assert rc == oz.OZ2_OK and flags & 1
    oz.dgemm_ex(to_device(generate(40, 64, 0.5, 1).T.copy()), to_device(B), transa=True, s=8, mode=mode)
    rc, flags = oz.ozaki2_get_flags()
    assert rc == oz.OZ2_OK and flags == 0
    torch.cuda.synchronize()


def test_deterministic_and_leading_dimensions(oz):
    import torch
    A = generate(200, 333, 1.0, 7)
    B = generate(333, 150, 1.0, 8)
    Ad, Bd = to_device(A), to_device(B)
    c1 = oz.dgemm(Ad, Bd, 14, "accu")
    c2 = oz.dgemm(Ad, Bd, 14, "accu")
    assert torch.equal(c1, c2)
    # padded leading dimensions give the same result
    Abig = torch.zeros((333, 256), dtype=torch.float64, device="cuda").t()   # ld 256 > 200
    Abig[:200, :] = Ad
    Ap = Abig[:200, :]
    Bbig = torch.zeros((150, 400), dtype=torch.float64, device="cuda").t()   # ld 400 > 333
    Bbig[:333, :] = Bd
    Bp = Bbig[:333, :]
    Cbig = torch.zeros((150, 300), dtype=torch.float64, device="cuda").t()
    Cp = Cbig[:200, :]
    oz.dgemm(Ap, Bp, 14, "accu", out=Cp)
    torch.cuda.synchronize()
    assert torch.equal(Cp, c1)
    assert not Cbig[200:, :].any()


def test_runs_on_the_callers_stream(oz):
    """A call on a side stream (default priority), with stage timing on, gives the same C
    as one on the default stream, and its timing events are recorded on that stream."""
    import torch
    A = generate(300, 700, 0.5, 17)
    B = generate(700, 260, 0.5, 18)
    Ad, Bd = to_device(A), to_device(B)
    c_default = oz.dgemm(Ad, Bd, 14, "fast")
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        assert oz.ozaki2_timing_begin(2) == oz.OZ2_OK
        c_side = oz.empty_colmajor(300, 260)
        for _ in range(2):
            oz.dgemm(Ad, Bd, 14, "fast", out=c_side, stream=side)
    side.synchronize()
    rc, last_ms = oz.ozaki2_get_stage_ms()
    assert rc == oz.OZ2_OK and all(t > 0.0 for t in last_ms)
    rc, stage_ms, ncalls = oz.ozaki2_timing_end()
    assert rc == oz.OZ2_OK and ncalls == 2 and all(t > 0.0 for t in stage_ms)
    assert all(a <= b + 1e-3 for a, b in zip(last_ms, stage_ms))   # one call's stages within the two-call sums
    assert torch.equal(c_side, c_default)


def test_graph_capture_replays(oz):
    """One call captured into a graph (caller workspace, so nothing is allocated inside the
    capture) and replayed four times, with eager calls and synchronizations in between;
    every replay must give the eager result."""
    import torch
    p, q, r, s = 300, 517, 200, 14
    A = generate(p, q, 0.5, 71)
    B = generate(q, r, 0.5, 72)
    Ad, Bd = to_device(A), to_device(B)
    need = oz.ozaki2_workspace_size(p, q, r, s, oz.OZ2_FAST)
    ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    base = (ws.data_ptr() + 255) // 256 * 256
    assert oz.ozaki2_set_workspace(base, need) == oz.OZ2_OK
    try:
        side = torch.cuda.Stream()
        C = oz.empty_colmajor(p, r)
        with torch.cuda.stream(side):
            oz.dgemm(Ad, Bd, s, "fast", out=C, stream=side)
        side.synchronize()
        want = C.clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            oz.dgemm(Ad, Bd, s, "fast", out=C, stream=side)
        for k in range(4):
            C.fill_(float("nan"))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(C, want), f"replay {k}"
            other = oz.dgemm(Ad, Bd, s, "fast")           # eager work between replays
            torch.cuda.synchronize()
            assert torch.equal(other, want)
        del graph
        torch.cuda.synchronize()
    finally:
        assert oz.ozaki2_set_workspace(None, 0) == oz.OZ2_OK


def test_caller_workspace_and_timing(oz):
    import torch
    A = generate(128, 256, 0.5, 1)
    B = generate(256, 96, 0.5, 2)
    Ad, Bd = to_device(A), to_device(B)
    ref = oz.dgemm(Ad, Bd, 8, "fast")
    need = oz.ozaki2_workspace_size(128, 256, 96, 8, 0)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    assert oz.ozaki2_set_workspace(ws.data_ptr(), need) == oz.OZ2_OK
    try:
        assert oz.ozaki2_timing_begin(4) == oz.OZ2_OK
        c = oz.dgemm(Ad, Bd, 8, "fast")
        c = oz.dgemm(Ad, Bd, 8, "fast")
        rc, ms, n = oz.ozaki2_timing_end()
        assert rc == oz.OZ2_OK and n == 2 and all(v >= 0 for v in ms)
        assert torch.equal(c, ref)
        with pytest.raises(oz.Oz2Error):
            oz.dgemm(Ad, Bd, 14, "fast")          # needs more than the caller gave
        torch.cuda.synchronize()
    finally:
        assert oz.ozaki2_set_workspace(None, 0) == oz.OZ2_OK


# ---------------------------------------------------------------------------
# Full-size workloads, sampled comparison
# ---------------------------------------------------------------------------
def _sampled_case(oz, name, nsamp=12):
    import torch
    w = WORKLOADS[name]
    log(f"[sampled] {name}: generating inputs n={w.n}")
    A, B = w.inputs()
    # no raw P_t dump: the GEMM then runs exactly as in ozaki2_dgemm (the large-grid
    # 16x16x64 kernel), and its R_t, X and C are compared
    want = ("d", "b", "Ap", "Bp", "At", "Bt", "R", "X") + (("rho", "gamma", "Abar", "Bbar") if w.mode == "accu" else ())
    log(f"[sampled] {name}: GPU run s={w.s} mode={w.mode}")
    out = oz.dgemm_debug(to_device(A), to_device(B), w.s, w.mode, want=want)
    torch.cuda.synchronize()
    rows = sample_indices(w.n, nsamp, 1)
    cols = sample_indices(w.n, nsamp, 2)
    log(f"[sampled] {name}: oracle on {len(rows)} rows x {len(cols)} cols")
    ref = oracle.ozaki2_sample(A, B, w.s, w.mode, rows, cols)
    ndiff = compare_sampled(out, ref, A, B, w.s, w.mode, rows, cols)
    if w.mode == "fast" and w.n <= 8192:
        log(f"[sampled] {name}: full d and b vectors")
        d_ref, _, _ = oracle.fast_exponents(A, w.s)
        b_ref, _, _ = oracle.fast_exponents(B.T, w.s)
        assert np.array_equal(out["d"].cpu().numpy(), d_ref.astype(np.int32))
        assert np.array_equal(out["b"].cpu().numpy(), b_ref.astype(np.int32))
    log(f"[sampled] {name}: ok ({ndiff} sampled C entries differ from the correctly rounded value)")
    del out
    torch.cuda.empty_cache()


def test_workload_n2048_fast_s14(oz):
    _sampled_case(oz, "n2048_fast_s14", nsamp=24)


def test_workload_n8192_fast_s14(oz):
    _sampled_case(oz, "n8192_fast_s14")


def test_workload_n8192_accu_s14(oz):
    _sampled_case(oz, "n8192_accu_s14")


def test_workload_n16384_fast_s18(oz):
    _sampled_case(oz, "n16384_fast_s18", nsamp=8)


def test_workload_n16384_accu_s18(oz):
    _sampled_case(oz, "n16384_accu_s18", nsamp=8)


@pytest.mark.parametrize("mode", ["fast", "accu"])
def test_edge_values_on_the_production_path(oz, mode):
    """The edge values of test_edge_values in a product large enough for the production
    path: 3072 x 3000 x 3072 (A and B above 128 MiB, so the statistics and residue passes
    read them non-temporally; 2016 tiles on the 8-wave GEMM), no A' / B' dump (the
    production residue kernels run).  The special rows and columns and a sample of the
    others are compared with the oracle, d and b in full."""
    import torch
    p, q, r, s = 3072, 3000, 3072, 14
    A = generate(p, q, 4.0, 15)
    B = generate(q, r, 4.0, 16)
    A[3, :] = 0.0                           # zero row
    B[:, 7] = 0.0                           # zero column
    A[5, 10] = 5e-324                       # subnormals
    A[6, :20] = -3e-310
    A[2900, :] = 5e-320
    B[11, 2] = 1e300                        # huge
    B[12, 3] = -1e-300
    A[9, :] = 1.0                           # flat row
    A[1800, 77] = 1e200                     # one dominant element
    want = ("d", "b", "At", "Bt", "R", "X") + (("rho", "gamma", "Abar", "Bbar") if mode == "accu" else ())
    log(f"[edges, production path] mode={mode} p,q,r={p},{q},{r} s={s}")
    out = oz.dgemm_debug(to_device(A), to_device(B), s, mode, want=want)
    torch.cuda.synchronize()
    rows = np.array(sorted(set(sample_indices(p, 8, 13).tolist()) | {3, 5, 6, 9, 1800, 2900, 3071}))
    cols = np.array(sorted(set(sample_indices(r, 8, 14).tolist()) | {2, 3, 7, 3071}))
    ref = oracle.ozaki2_sample(A, B, s, mode, rows, cols)
    compare_sampled(out, ref, A, B, s, mode, rows, cols)
    if mode == "fast":
        d_ref, _, _ = oracle.fast_exponents(A, s)
        b_ref, _, _ = oracle.fast_exponents(np.asarray(B).T, s)
        assert np.array_equal(out["d"].cpu().numpy(), d_ref.astype(np.int32)), "d"
        assert np.array_equal(out["b"].cpu().numpy(), b_ref.astype(np.int32)), "b"
    log("[edges, production path] ok")


@pytest.mark.parametrize("raw_p", [False, True])
@pytest.mark.parametrize("mode", ["fast", "accu"])
def test_large_tiles_on_ragged_shape(oz, mode, raw_p):
    """1800 x 300 x 1790 with s = 20: enough 256 x 256 tiles (8 x 8 x 20) for the large-grid
    GEMM, whose ragged last tile row and column are sampled.  Without the raw P_t dump the
    production 16x16x64 kernel runs; with it, the kernel form that also writes P_t."""
    import torch
    p, q, r, s = 1800, 300, 1790, 20
    A = generate(p, q, 1.0, 91)
    B = generate(q, r, 1.0, 92)
    want = ("d", "b", "Ap", "Bp", "At", "Bt", "R", "X") + (("P",) if raw_p else ()) + \
        (("rho", "gamma", "Abar", "Bbar") if mode == "accu" else ())
    log(f"[large tiles] mode={mode} raw_p={raw_p} p,q,r={p},{q},{r} s={s}")
    out = oz.dgemm_debug(to_device(A), to_device(B), s, mode, want=want)
    torch.cuda.synchronize()
    rows = np.array(sorted(set(sample_indices(p, 10, 3).tolist()) | {1535, 1536, 1790, 1799}))
    cols = np.array(sorted(set(sample_indices(r, 10, 4).tolist()) | {1535, 1536, 1780, 1789}))
    ref = oracle.ozaki2_sample(A, B, s, mode, rows, cols)
    compare_sampled(out, ref, A, B, s, mode, rows, cols)
    log("[large tiles] ok")
