"""GPU parity of the general entry point ozaki2_dgemm_ex and of K-blocked inner dimensions.

* transposed operands: ozaki2_dgemm_ex on A^T / B^T as stored must give exactly the
  result of ozaki2_dgemm on explicit copies of op(A), op(B) (same scalings, residues and
  CRT), and that result must match the oracle on op(A), op(B);
* alpha / beta: C <- alpha C_hat + beta C as oracle.alpha_beta_update defines it;
* q beyond 2^17: the GEMM runs over K-blocks of 2^17 and accumulates their residues mod
  m_t; d, b, R_t and X must stay bit-exact against the oracle.
"""
import numpy as np
import pytest

import oracle
from fp64_gemm_emulation_amd.workloads import generate
from tests.gpu_helpers import (assert_chat_close, assert_correctly_rounded, assert_equal, chat_tolerance, log, to_device,
                               x_limbs_to_int)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def oz():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    from fp64_gemm_emulation_amd import binding
    return binding


def _padded(a_np, extra):
    """Column-major device copy of a_np with leading dimension rows + extra."""
    import torch
    rows, cols = a_np.shape
    buf = torch.full((cols, rows + extra), float("nan"), dtype=torch.float64, device="cuda")
    buf[:, :rows] = torch.from_numpy(np.ascontiguousarray(a_np.T)).cuda()
    return buf.t()[:rows, :]


@pytest.mark.parametrize("mode", ["fast", "accu"])
@pytest.mark.parametrize("ta,tb", [(False, False), (True, False), (False, True), (True, True)])
def test_transposed_operands(oz, mode, ta, tb):
    p, q, r, s = 300, 517, 129, 14
    opA = generate(p, q, 1.0, 41)
    opB = generate(q, r, 1.0, 42)
    log(f"[ex] transa={ta} transb={tb} mode={mode} p,q,r={p},{q},{r}")
    A_stored = _padded(opA.T if ta else opA, 3)
    B_stored = _padded(opB.T if tb else opB, 5)
    c_ex = oz.dgemm_ex(A_stored, B_stored, transa=ta, transb=tb, s=s, mode=mode).cpu().numpy()
    c_plain = oz.dgemm(to_device(opA), to_device(opB), s, mode).cpu().numpy()
    assert_equal(c_ex, c_plain, "ozaki2_dgemm_ex vs ozaki2_dgemm on op(A), op(B)")
    ref = oracle.ozaki2(opA, opB, s, mode)
    assert_chat_close(c_ex, ref["C"], chat_tolerance(opA, opB, np.arange(p), np.arange(r)), "C")
    assert_correctly_rounded(c_ex, ref["C"], "C")
    log(f"[ex] ok ({int(np.sum(c_ex != ref['C']))} entries differ from the correctly rounded value)")


@pytest.mark.parametrize("mode,ta,tb", [("fast", True, False), ("fast", False, True), ("fast", True, True),
                                        ("accu", True, True)])
def test_transposed_operands_on_the_production_path(oz, mode, ta, tb):
    """3072 x 3000 x 2560, s = 14: A and B above 128 MiB (non-temporal reads in the
    statistics and residue passes, whose row and column kernels swap roles for transposed
    operands) and 1680 tiles on the 8-wave GEMM.  ozaki2_dgemm_ex must equal ozaki2_dgemm
    on explicit copies of op(A), op(B) bit for bit, and sampled entries must match the
    oracle."""
    import torch
    from tests.gpu_helpers import sample_indices
    p, q, r, s = 3072, 3000, 2560, 14
    opA = generate(p, q, 1.0, 43)
    opB = generate(q, r, 1.0, 44)
    log(f"[ex large] transa={ta} transb={tb} mode={mode} p,q,r={p},{q},{r}")
    A_stored = to_device(np.ascontiguousarray(opA.T) if ta else opA)
    B_stored = to_device(np.ascontiguousarray(opB.T) if tb else opB)
    c_ex = oz.dgemm_ex(A_stored, B_stored, transa=ta, transb=tb, s=s, mode=mode)
    del A_stored, B_stored
    c_plain = oz.dgemm(to_device(opA), to_device(opB), s, mode)
    torch.cuda.synchronize()
    assert torch.equal(c_ex, c_plain), "ozaki2_dgemm_ex vs ozaki2_dgemm on op(A), op(B)"
    rows = sample_indices(p, 10, 21)
    cols = sample_indices(r, 10, 22)
    ref = oracle.ozaki2_sample(opA, opB, s, mode, rows, cols)
    c = c_ex.cpu().numpy()[np.ix_(rows, cols)]
    assert_chat_close(c, ref["C"], chat_tolerance(opA, opB, rows, cols), "C")
    assert_correctly_rounded(c, ref["C"], "C")
    log("[ex large] ok")


@pytest.mark.parametrize("mode", ["fast", "accu"])
@pytest.mark.parametrize("alpha,beta", [(-0.75, 1.5), (2.0, 0.0), (1.0, -1.0), (0.0, 0.5)])
def test_alpha_beta(oz, mode, alpha, beta):
    import torch
    p, q, r, s = 130, 260, 70, 14
    A = generate(p, q, 0.5, 51)
    B = generate(q, r, 0.5, 52)
    C0 = generate(p, r, 0.5, 53) if beta != 0.0 else np.full((p, r), np.nan)
    log(f"[ex] alpha={alpha} beta={beta} mode={mode}")
    Cd = to_device(C0)
    got = oz.dgemm_ex(to_device(A), to_device(B), alpha=alpha, beta=beta, C=Cd, s=s, mode=mode).cpu().numpy()
    ref = oracle.ozaki2(A, B, s, mode)
    want = oracle.alpha_beta_update(ref["C"], alpha, beta, C0)
    tol = abs(alpha) * chat_tolerance(A, B, np.arange(p), np.arange(r)) + 2.0 ** -52 * np.abs(want)
    assert_chat_close(got, want, tol, "alpha C_hat + beta C")
    assert torch.isfinite(torch.from_numpy(got)).all()
    log(f"[ex] ok ({int(np.sum(got != want))} entries differ from the oracle's update)")


def test_empty_inner_dimension_scales_c(oz):
    p, r = 33, 17
    C0 = generate(p, r, 0.5, 61)
    Cd = to_device(C0)
    import torch
    A = torch.empty((p, 0), dtype=torch.float64, device="cuda")
    B = torch.empty((0, r), dtype=torch.float64, device="cuda")
    got = oz.dgemm_ex(A, B, alpha=3.0, beta=-2.0, C=Cd, s=8).cpu().numpy()
    assert_equal(got, oracle.alpha_beta_update(np.zeros((p, r)), 3.0, -2.0, C0), "q = 0")


@pytest.mark.parametrize("mode", ["fast", "accu"])
def test_k_blocked_inner_dimension(oz, mode):
    """q = 131372: two K-blocks (131072 + 300 inner-dimension elements)."""
    p, q, r, s = 40, 131372, 24, 8
    A = generate(p, q, 0.5, 71)
    B = generate(q, r, 0.5, 72)
    log(f"[kblock] mode={mode} p,q,r={p},{q},{r} s={s}")
    out = oz.dgemm_debug(to_device(A), to_device(B), s, mode, want=("d", "b", "R", "X"))
    ref = oracle.ozaki2(A, B, s, mode)
    assert_equal(out["d"].cpu().numpy(), ref["d"].astype(np.int32), "d")
    assert_equal(out["b"].cpu().numpy(), ref["b"].astype(np.int32), "b")
    rt = out["R"].cpu().numpy()
    for t in range(s):
        assert_equal(rt[t], ref["R"][t].T.astype(np.uint8), f"R_t t={t}")
    xg = out["X"].cpu().numpy()
    for j in range(r):
        for i in range(p):
            assert x_limbs_to_int(xg[j, i]) == int(ref["X"][i, j]), f"X[{i},{j}]"
    assert_chat_close(out["C"].cpu().numpy(), ref["C"], chat_tolerance(A, B, np.arange(p), np.arange(r)), "C")
    log("[kblock] ok")


def test_k_blocked_on_large_grid(oz):
    """q = 131372 (two K-blocks) with p = r = 1536, s = 15: 540 tiles of 256 x 256, so the first
    K-block runs in the large-grid 16x16x64 kernel and the second accumulates its residues in
    the K-block epilogue; sampled entries of R_t, X and C against the oracle."""
    import torch
    p, q, r, s = 1536, 131372, 1536, 15
    A = generate(p, q, 0.5, 73)
    B = generate(q, r, 0.5, 74)
    log(f"[kblock large] p,q,r={p},{q},{r} s={s}")
    out = oz.dgemm_debug(to_device(A), to_device(B), s, "fast", want=("d", "b", "R", "X"))
    torch.cuda.synchronize()
    rows = np.array([0, 255, 256, 777, 1279, 1535])
    cols = np.array([1, 254, 511, 512, 1024, 1534])
    ref = oracle.ozaki2_sample(A, B, s, "fast", rows, cols)
    assert_equal(out["d"][rows].cpu().numpy(), ref["d"].astype(np.int32), "d")
    assert_equal(out["b"][cols].cpu().numpy(), ref["b"].astype(np.int32), "b")
    rows_t = torch.as_tensor(rows, device="cuda")
    cols_t = torch.as_tensor(cols, device="cuda")
    rt = out["R"][:, cols_t][:, :, rows_t].cpu().numpy()
    for t in range(s):
        assert_equal(rt[t], ref["R"][t].T.astype(np.uint8), f"R_t t={t}")
    xg = out["X"][cols_t][:, rows_t].cpu().numpy()
    for jj in range(len(cols)):
        for ii in range(len(rows)):
            assert x_limbs_to_int(xg[jj, ii]) == int(ref["X"][ii, jj]), f"X[{rows[ii]},{cols[jj]}]"
    c = out["C"][rows_t][:, cols_t].cpu().numpy()
    assert_chat_close(c, ref["C"], chat_tolerance(A, B, rows, cols), "C")
    log("[kblock large] ok")


def test_p_dump_refused_when_k_blocked(oz):
    import torch
    p, q, r = 8, oz.OZ2_MAX_Q_P_DUMP + 1, 8
    A = torch.zeros((p, q), dtype=torch.float64, device="cuda").t().contiguous().t()
    B = torch.zeros((q, r), dtype=torch.float64, device="cuda").t().contiguous().t()
    with pytest.raises(oz.Oz2Error) as info:
        oz.dgemm_debug(A, B, 8, "fast", want=("P",))
    assert info.value.status == oz.OZ2_ERR_UNSUPPORTED


@pytest.mark.parametrize("mode", ["fast", "accu"])
def test_max_inner_dimension_max_s(oz, mode):
    """q = OZ2_MAX_Q = 2^19 - 1 (four K-blocks) with s = 20."""
    p, q, r, s = 8, oz.OZ2_MAX_Q, 8, 20
    A = generate(p, q, 1.0, 81)
    B = generate(q, r, 1.0, 82)
    log(f"[max q] mode={mode} p,q,r={p},{q},{r} s={s}")
    out = oz.dgemm_debug(to_device(A), to_device(B), s, mode, want=("d", "b", "X"))
    ref = oracle.ozaki2(A, B, s, mode)
    assert_equal(out["d"].cpu().numpy(), ref["d"].astype(np.int32), "d")
    assert_equal(out["b"].cpu().numpy(), ref["b"].astype(np.int32), "b")
    xg = out["X"].cpu().numpy()
    for j in range(r):
        for i in range(p):
            assert x_limbs_to_int(xg[j, i]) == int(ref["X"][i, j]), f"X[{i},{j}]"
    assert_chat_close(out["C"].cpu().numpy(), ref["C"], chat_tolerance(A, B, np.arange(p), np.arange(r)), "C")
    log("[max q] ok")


def test_accu_bound_product_at_its_int32_limit(oz):
    """Every entry 2 - 2^-52 quantizes to 64, so the bound product is q 64^2 = 2147479552 at
    q = OZ2_MAX_Q, the largest INT32 value the accu bound GEMM can meet."""
    p, q, r, s = 4, oz.OZ2_MAX_Q, 4, 8
    v = 2.0 - 2.0 ** -52
    A = np.full((p, q), v, order="F")
    B = np.full((q, r), -v, order="F")
    out = oz.dgemm_debug(to_device(A), to_device(B), s, "accu", want=("rho", "gamma", "d", "b"))
    assert (out["rho"].cpu().numpy() == q * 64 * 64).all()
    assert (out["gamma"].cpu().numpy() == q * 64 * 64).all()
    ref = oracle.ozaki2(A, B, s, "accu")
    assert_equal(out["d"].cpu().numpy(), ref["d"].astype(np.int32), "d")
    assert_equal(out["b"].cpu().numpy(), ref["b"].astype(np.int32), "b")
    assert_chat_close(out["C"].cpu().numpy(), ref["C"], chat_tolerance(A, B, np.arange(p), np.arange(r)), "C")


@pytest.mark.parametrize("mode", ["fast", "accu"])
@pytest.mark.parametrize("shape", [(1 << 23, 5, 3), (3, 5, 1 << 23)])
def test_max_rows_or_columns(oz, shape, mode):
    """p or r at the largest accepted size, 2^23 (the launch grids at their widest)."""
    p, q, r = shape
    s = 2
    A = generate(p, q, 0.5, 83)
    B = generate(q, r, 0.5, 84)
    log(f"[max dim] p,q,r={p},{q},{r} s={s} mode={mode}")
    out = oz.dgemm_debug(to_device(A), to_device(B), s, mode, want=("d", "b"))
    rows = np.array(sorted({0, 1, p // 2, p - 2, p - 1}))
    cols = np.array(sorted({0, 1, r // 2, r - 2, r - 1}))
    ref = oracle.ozaki2_sample(A, B, s, mode, rows, cols)
    import torch
    assert_equal(out["d"][torch.as_tensor(rows, device="cuda")].cpu().numpy(), ref["d"].astype(np.int32), "d")
    assert_equal(out["b"][torch.as_tensor(cols, device="cuda")].cpu().numpy(), ref["b"].astype(np.int32), "b")
    c = out["C"][torch.as_tensor(rows, device="cuda")][:, torch.as_tensor(cols, device="cuda")].cpu().numpy()
    assert_chat_close(c, ref["C"], chat_tolerance(A, B, rows, cols), "C")
    log("[max dim] ok")
