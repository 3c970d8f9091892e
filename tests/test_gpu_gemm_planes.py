"""Element-complete parity of the production GEMM (gemm_w8_kernel: 8 waves of
v_mfma_i32_16x16x64_i8, 256 x 256 tiles), which runs whenever a launch has at least 512
tiles of 256 x 256 over all its planes.  Every element of the compared R_t planes must
equal the oracle's R_t = (A_t B_t) mod m_t ("Ozaki II supplement", section 1.1: with
2 c_max < M the CRT of these residues is X = A'B' exactly), so a slip confined to one
lane, register or tile position cannot hide between samples.

The oracle's step functions (exponents, scaled truncation, centered residues, exact
products, output residues) run in that order on the whole operands; the elementwise ones
are called on row ranges in threads (NumPy releases the GIL), which changes nothing
about what they compute.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
from fp64_gemm_emulation_amd.workloads import WORKLOADS, generate
from tests.gpu_helpers import assert_chat_close, assert_equal, compare_sampled, log, sample_indices, to_device

pytestmark = pytest.mark.gpu

_THREADS = 8


@pytest.fixture(scope="module")
def oz():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    from fp64_gemm_emulation_amd import binding
    return binding


def _ranges(n, parts):
    edges = np.linspace(0, n, min(parts, max(n, 1)) + 1).astype(int)
    return [(int(a), int(b)) for a, b in zip(edges[:-1], edges[1:]) if b > a]


def _by_rows(fn, nrows):
    """fn(lo, hi) over row ranges in threads, results stacked along axis 0."""
    with ThreadPoolExecutor(_THREADS) as ex:
        parts = list(ex.map(lambda rg: fn(*rg), _ranges(nrows, 4 * _THREADS)))
    return np.concatenate(parts, axis=0)


def oracle_exponents(A, B, s, mode):
    """(d, b, extras) from the oracle: fast per line (row ranges in threads), accu whole."""
    if mode == "accu":
        out = oracle.accu_exponents(A, B, s)
        return out["d"], out["b"], out
    Bt = np.asarray(B).T
    d = _by_rows(lambda lo, hi: oracle.fast_exponents(A[lo:hi], s)[0], A.shape[0])
    b = _by_rows(lambda lo, hi: oracle.fast_exponents(Bt[lo:hi], s)[0], Bt.shape[0])
    return d, b, {}


def oracle_planes(A, B, s, d, b, planes):
    """Yield (t, R_t) for the requested modulus indices, R_t p x r, from the oracle's steps:
    A' = trunc(2^d A), B' = trunc(B 2^b), centered residues, exact product, mod m_t."""
    Bt = np.asarray(B).T
    ap = _by_rows(lambda lo, hi: oracle.scale_truncate(A[lo:hi], d[lo:hi]), A.shape[0])
    bpt = _by_rows(lambda lo, hi: oracle.scale_truncate(Bt[lo:hi], b[lo:hi]), Bt.shape[0])
    mods = oracle.moduli(s)
    for t in planes:
        m = mods[t]
        at = _by_rows(lambda lo, hi: oracle.centered_residue(ap[lo:hi], m), ap.shape[0])
        btt = _by_rows(lambda lo, hi: oracle.centered_residue(bpt[lo:hi], m), bpt.shape[0])
        yield t, oracle.output_residue(oracle.residue_product(at, btt.T), m), at, btt


def big_tiles(p, r, s):
    return ((p + 255) // 256) * ((r + 255) // 256) * s


def _compare_planes(out, A, B, s, d, b, planes, label, operands=False):
    for t, R, at, btt in oracle_planes(A, B, s, d, b, planes):
        assert_equal(out["R"][t].cpu().numpy().T, R.astype(np.uint8), f"{label} R_t t={t}")
        if operands:
            assert_equal(out["At"][t].cpu().numpy(), at.astype(np.int8), f"{label} A_t t={t}")
            assert_equal(out["Bt"][t].cpu().numpy(), btt.astype(np.int8), f"{label} B_t t={t}")
        log(f"[planes] {label}: plane t={t} (m={oracle.moduli(s)[t]}) equal in full")


@pytest.mark.parametrize("mode", ["fast", "accu"])
def test_production_gemm_every_plane_in_full(oz, mode):
    """p = r = 2048, q = 700, s = 14: 896 tiles, the 8-wave kernel.  Every R_t, A_t and B_t
    element, d and b (and e, f, rho, gamma in accu) in full; X and C on samples."""
    import torch
    p, q, r, s = 2048, 700, 2048, 14
    assert big_tiles(p, r, s) >= 512
    A = generate(p, q, 1.0, 501)
    B = generate(q, r, 1.0, 502)
    # no A' / B' dump, so the production residue kernels write the compared A_t, B_t
    want = ("d", "b", "At", "Bt", "R", "X") + (("e", "f", "rho", "gamma", "Abar", "Bbar")
                                               if mode == "accu" else ())
    log(f"[planes] production GEMM {mode}: p,q,r={p},{q},{r} s={s}")
    out = oz.dgemm_debug(to_device(A), to_device(B), s, mode, want=want)
    torch.cuda.synchronize()
    d, b, ex = oracle_exponents(A, B, s, mode)
    assert_equal(out["d"].cpu().numpy(), d.astype(np.int32), "d")
    assert_equal(out["b"].cpu().numpy(), b.astype(np.int32), "b")
    if mode == "accu":
        assert_equal(out["rho"].cpu().numpy(), ex["rho"].astype(np.int32), "rho")
        assert_equal(out["gamma"].cpu().numpy(), ex["gamma"].astype(np.int32), "gamma")
    _compare_planes(out, A, B, s, d, b, range(s), f"2048x700x2048 {mode}", operands=True)
    rows = sample_indices(p, 12, 5)
    cols = sample_indices(r, 12, 6)
    compare_sampled(out, oracle.ozaki2_sample(A, B, s, mode, rows, cols), A, B, s, mode, rows, cols)
    log(f"[planes] production GEMM {mode}: ok")


@pytest.mark.parametrize("p,q,r,s", [(2048, 300, 2048, 9), (2048, 300, 1536, 11)])
def test_partial_last_round_every_plane_in_full(oz, p, q, r, s):
    """Grids of the 8-wave kernel whose last round on a 256-CU device is partly empty:
    576 tiles (s = 9, odd) and 528 tiles of a non-square product (s = 11).  Every R_t in
    full, so tiles of the first and the last round, and of every plane, are all checked."""
    import torch
    assert big_tiles(p, r, s) >= 512 and 0 < big_tiles(p, r, s) % 256 <= 128
    A = generate(p, q, 1.0, 511)
    B = generate(q, r, 1.0, 512)
    log(f"[planes] partial last round: p,q,r={p},{q},{r} s={s}")
    out = oz.dgemm_debug(to_device(A), to_device(B), s, "fast", want=("d", "b", "R"))
    torch.cuda.synchronize()
    d, b, _ = oracle_exponents(A, B, s, "fast")
    assert_equal(out["d"].cpu().numpy(), d.astype(np.int32), "d")
    assert_equal(out["b"].cpu().numpy(), b.astype(np.int32), "b")
    _compare_planes(out, A, B, s, d, b, range(s), f"{p}x{q}x{r} s{s}")


def test_headline_workload_planes_in_full(oz):
    """n = 8192 fast, s = 14: the m = 256 plane and an odd plane (m = 199) in full."""
    import torch
    w = WORKLOADS["n8192_fast_s14"]
    A, B = w.inputs()
    log(f"[planes] {w.name}: GPU run")
    out = oz.dgemm_debug(to_device(A), to_device(B), w.s, w.mode, want=("d", "b", "R"))
    torch.cuda.synchronize()
    log(f"[planes] {w.name}: oracle exponents")
    d, b, _ = oracle_exponents(A, B, w.s, w.mode)
    assert_equal(out["d"].cpu().numpy(), d.astype(np.int32), "d")
    assert_equal(out["b"].cpu().numpy(), b.astype(np.int32), "b")
    _compare_planes(out, A, B, w.s, d, b, [0, w.s - 1], w.name)
    del out
    torch.cuda.empty_cache()


def test_largest_workload_planes_in_full(oz):
    """n = 16384 fast, s = 18 (256 stages of the inner dimension per tile, the longest
    K loop of the five workloads): d and b, the m = 256 plane and the last odd plane
    (m = 181) in full."""
    import torch
    w = WORKLOADS["n16384_fast_s18"]
    A, B = w.inputs()
    log(f"[planes] {w.name}: GPU run")
    out = oz.dgemm_debug(to_device(A), to_device(B), w.s, w.mode, want=("d", "b", "R"))
    torch.cuda.synchronize()
    log(f"[planes] {w.name}: oracle exponents")
    d, b, _ = oracle_exponents(A, B, w.s, w.mode)
    assert_equal(out["d"].cpu().numpy(), d.astype(np.int32), "d")
    assert_equal(out["b"].cpu().numpy(), b.astype(np.int32), "b")
    _compare_planes(out, A, B, w.s, d, b, [0, w.s - 1], w.name)
    del out
    torch.cuda.empty_cache()


def test_accu_workload_scalings_in_full(oz):
    """n = 8192 accu, s = 14 (bound GEMM on the 8-wave kernel with its row / column maximum
    epilogue): e, f, rho, gamma, d and b in full, and one residue plane (m = 233) in full."""
    import torch
    w = WORKLOADS["n8192_accu_s14"]
    A, B = w.inputs()
    log(f"[planes] {w.name}: GPU run")
    assert big_tiles(w.n, w.n, 1) >= 512
    out = oz.dgemm_debug(to_device(A), to_device(B), w.s, w.mode,
                         want=("d", "b", "e", "f", "rho", "gamma", "R"))
    torch.cuda.synchronize()
    log(f"[planes] {w.name}: oracle bound product")
    d, b, ex = oracle_exponents(A, B, w.s, w.mode)
    assert all(v is not None for v in ex["e"]) and all(v is not None for v in ex["f"])
    assert_equal(out["e"].cpu().numpy(), np.array(ex["e"], dtype=np.int32), "e")
    assert_equal(out["f"].cpu().numpy(), np.array(ex["f"], dtype=np.int32), "f")
    assert_equal(out["rho"].cpu().numpy(), ex["rho"].astype(np.int32), "rho")
    assert_equal(out["gamma"].cpu().numpy(), ex["gamma"].astype(np.int32), "gamma")
    assert_equal(out["d"].cpu().numpy(), d.astype(np.int32), "d")
    assert_equal(out["b"].cpu().numpy(), b.astype(np.int32), "b")
    _compare_planes(out, A, B, w.s, d, b, [7], w.name)
    del out
    torch.cuda.empty_cache()


def test_k_blocked_production_gemm_every_plane(oz):
    """q = 2^17 + 256 (two K-blocks: the second runs the 8-wave kernel's accumulate
    epilogue, R_t <- (P_block + R_t) mod m_t), p = r = 1281 (ragged last tile row and
    column), s = 15: 540 tiles.  Every element of every R_t plane; X and C on samples."""
    import torch
    p, q, r, s = 1281, (1 << 17) + 256, 1281, 15
    assert big_tiles(p, r, s) >= 512
    A = generate(p, q, 0.5, 601)
    B = generate(q, r, 0.5, 602)
    log(f"[planes] K-blocked: p,q,r={p},{q},{r} s={s}")
    out = oz.dgemm_debug(to_device(A), to_device(B), s, "fast", want=("d", "b", "At", "Bt", "R", "X"))
    torch.cuda.synchronize()
    d, b, _ = oracle_exponents(A, B, s, "fast")
    assert_equal(out["d"].cpu().numpy(), d.astype(np.int32), "d")
    assert_equal(out["b"].cpu().numpy(), b.astype(np.int32), "b")
    _compare_planes(out, A, B, s, d, b, range(s), "K-blocked")
    rows = np.array(sorted(set(sample_indices(p, 5, 7).tolist()) | {255, 256, 1279, 1280}))
    cols = np.array(sorted(set(sample_indices(r, 5, 8).tolist()) | {255, 256, 1279, 1280}))
    compare_sampled(out, oracle.ozaki2_sample(A, B, s, "fast", rows, cols), A, B, s, "fast", rows, cols)
    log("[planes] K-blocked: ok")
    del out
    torch.cuda.empty_cache()


# Row values of A and column values of B for the INT32-extreme case below: each row of A
# (column of B) is one constant, so every A'_t (B'_t) entry of a line is one residue and
# P_t[i, j] = q rho(A'_i) rho(B'_j) exactly.  Chosen (by a search over the oracle's residues
# of such lines) so that most planes reach |P_t| >= 2^30 and the largest 2^30.97 at
# q = 131071, the longest inner dimension one launch covers.
_EXTREME_X = [0.8122686777911212, 0.3467247145518215, 0.09158796504591349, -0.4837182962908233,
              -0.8651221338159478, 0.4372684343765658, -0.9013546892409319, 0.6037519305692991]
_EXTREME_Y = [-0.15756668806272445, -0.7597194561131462, -0.022761176011345974, 0.47856384225672954,
              0.49893093563626234, -0.12307763329453159, -0.22521746631645212, -0.20208214895857712]


@pytest.mark.parametrize("mode,q", [("fast", (1 << 17) - 1), ("fast", (1 << 17) + 1000), ("accu", (1 << 17) - 1)])
def test_production_gemm_at_int32_extremes(oz, mode, q):
    """The production GEMM (p = r = 2048, s = 20: 1280 tiles of 256 x 256) with products
    |P_t| up to 2^30.97, every modulus: A[i, :] = x[i mod 8], B[:, j] = y[j mod 8], so every
    output of the GPU equals one of the oracle's 8 x 8 outputs of the 8 x q x 8 product with
    the same lines, and every element of every R_t plane, d, b and C is compared with it.
    q = 2^17 - 1 is one launch; q = 2^17 + 1000 runs two K-blocks, the second through the
    accumulate epilogue.  In accu mode the bound product's row and column maxima over all
    2048 columns and rows equal those over the 8 distinct ones, so the 8 x q x 8 oracle
    gives the same exponents as the whole product."""
    import torch
    p = r = 2048
    s = 20
    assert big_tiles(p, r, s) >= 512
    xs = np.array(_EXTREME_X)
    ys = np.array(_EXTREME_Y)
    log(f"[extremes] {mode}: oracle on the 8 x {q} x 8 product")
    ref = oracle.ozaki2(np.repeat(xs[:, None], q, axis=1), np.repeat(ys[None, :], q, axis=0), s, mode)
    if q < (1 << 17):
        pmax = max(int(np.abs(pt).max()) for pt in ref["P"])
        assert pmax >= 2 ** 30.9, pmax
    dev = torch.device("cuda")
    rows = torch.arange(p, device=dev) % 8
    cols = torch.arange(r, device=dev) % 8
    A = torch.tensor(xs, device=dev)[rows][:, None].expand(p, q)
    B = torch.tensor(ys, device=dev)[cols][None, :].expand(q, r)
    Ad = oz.colmajor(A)
    Bd = oz.colmajor(B)
    del A, B
    log(f"[extremes] {mode}: p,q,r={p},{q},{r} s={s}")
    out = oz.dgemm_debug(Ad, Bd, s, mode, want=("d", "b", "R"))
    torch.cuda.synchronize()
    del Ad, Bd
    assert torch.equal(out["d"], torch.tensor(ref["d"].astype(np.int32), device=dev)[rows]), "d"
    assert torch.equal(out["b"], torch.tensor(ref["b"].astype(np.int32), device=dev)[cols]), "b"
    for t, m in enumerate(ref["moduli"]):
        small = torch.tensor(np.asarray(ref["R"][t], dtype=np.uint8), device=dev)   # [i mod 8, j mod 8]
        want = small.t()[cols][:, rows]                                                # [j, i]
        got = out["R"][t]
        if not torch.equal(got, want):
            jj, ii = (got != want).nonzero()[0].tolist()
            raise AssertionError(f"R[{t}] (m = {m}) at ({ii}, {jj}): {int(got[jj, ii])} != {int(want[jj, ii])}")
    c_ref = np.asarray(ref["C"], dtype=np.float64)[np.arange(p)[:, None] % 8, np.arange(r)[None, :] % 8]
    tol = 4.0 * 2.0 ** -53 * q * np.abs(xs[np.arange(p) % 8][:, None] * ys[np.arange(r) % 8][None, :])
    assert_chat_close(out["C"].cpu().numpy(), c_ref, tol, "C")
    log("[extremes] ok: every element of every plane")
    del out
    torch.cuda.empty_cache()
