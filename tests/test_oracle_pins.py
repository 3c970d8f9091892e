"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks one oracle step against something other than the oracle
itself: numbers printed on the pages (tests/golden), a textbook definition
evaluated by brute force with Python integers, a closed form, or an exact
rational (Fraction) bound.  A plausible mistake in any step (a dropped term, a
wrong sign, interval or index, a transposed operand, rounding instead of
truncation, an off-by-one exponent) fails at least one of them; see
test_oracle_mutations.py for planted mistakes.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from fp64_gemm_emulation_amd.workloads import generate

ALL_S = list(range(oracle.MIN_S, oracle.MAX_S + 1))


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "pages_constants.json")) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# Moduli, M, range budget
# --------------------------------------------------------------------------
def test_moduli_s8_matches_workload_list(golden_dir):
    with open(os.path.join(golden_dir, "workload_moduli_s8.txt")) as f:
        line = [ln for ln in f if ln.strip() and not ln.startswith("#")][0]
    expected = [int(v) for v in line.split(",")]
    assert oracle.moduli(8) == expected


@pytest.mark.parametrize("s", ALL_S)
def test_moduli_pairwise_coprime_greedy(s):
    mods = oracle.moduli(s)
    assert len(mods) == s and all(2 <= m <= 256 for m in mods)
    assert mods == sorted(mods, reverse=True)
    for a in range(s):
        for b in range(a + 1, s):
            assert math.gcd(mods[a], mods[b]) == 1
    # greedy: every skipped integer shares a factor with a larger chosen modulus
    chosen = set(mods)
    for m in range(mods[-1] + 1, 257):
        if m not in chosen:
            assert any(math.gcd(m, c) > 1 for c in mods if c > m)


def test_range_bits_16_moduli(golden_dir):
    g = _golden(golden_dir)["range_bits_16_moduli"]
    bits = math.log2(oracle.modulus_product(16))
    assert abs(bits - g["value"]) <= g["tolerance"]


@pytest.mark.parametrize("s", ALL_S)
def test_tau_is_reconstruction_budget(s):
    M = oracle.modulus_product(s)
    t = oracle.tau(s)
    # |X| <= 2^tau must give 2|X| < M (condition 2 c_max < M), and tau is the largest such
    assert 2 * (1 << t) < M
    assert 2 * (1 << (t + 1)) >= M - 2


def test_int32_accumulation_condition(golden_dir):
    g = _golden(golden_dir)
    limit = g["int32_safe_q_limit"]["value"]
    pb = g["int8_product_bound"]["value"]
    for s in ALL_S:
        for m in oracle.moduli(s):
            assert (m // 2) ** 2 <= pb
    assert (limit - 1) * pb < 2 ** 31 <= limit * pb


def test_eq18_equal_budget_on_flat_rows():
    """All-ones rows: fast d equals Eq. 18's k = floor(1/2 log2((M/2-1)/q)).

    Ozaki II supplement section 2: with |a'| <= 2^k for every entry of a
    length-q dot product, (|A'||B'|)_ij <= q 2^(2k); Eq. 18 gives the equal
    per-input budget.  For a row of q = 2^j ones the norm bound and the
    max bound coincide, so the fast exponent must be exactly that k.
    """
    for s in (2, 8, 14, 18, 20):
        M = oracle.modulus_product(s)
        for j in range(0, 13):
            q = 1 << j
            k = math.floor(0.5 * math.log2((M // 2 - 1) / q))
            # exact floor: largest k with q 4^k <= M/2 - 1
            while q * 4 ** (k + 1) <= M // 2 - 1:
                k += 1
            while q * 4 ** k > M // 2 - 1:
                k -= 1
            d, _, _ = oracle.fast_exponents(np.ones((1, q)), s)
            assert int(d[0]) == k, (s, q)


# --------------------------------------------------------------------------
# Centered residues
# --------------------------------------------------------------------------
def _interesting_integers(rng, count):
    vals = [0, 1, -1, 127, -127, 128, -128, 129, 255, -255, 256, -256, 257,
            2 ** 31, -(2 ** 31), 2 ** 53, 2 ** 63, -(2 ** 63), 2 ** 70 + 2 ** 20, 3 * 2 ** 90]
    for _ in range(count):
        mu = int(rng.integers(0, 2 ** 53))
        k = int(rng.integers(0, 64))
        v = mu << k if rng.random() < 0.5 else mu >> int(rng.integers(0, 53))
        vals.append(-v if rng.random() < 0.5 else v)
    # every value must be exactly representable in float64
    return [v for v in vals if int(float(v)) == v]


def test_centered_residue_definition():
    rng = np.random.default_rng(7)
    ints = _interesting_integers(rng, 400)
    x = np.array([float(v) for v in ints])
    for m in oracle.moduli(20):
        r = oracle.centered_residue(x, m)
        lo, hi = -(m // 2), -(-m // 2) - 1
        for v, rv in zip(ints, r):
            rv = int(rv)
            assert lo <= rv <= hi
            assert (v - rv) % m == 0


def test_centered_residue_m256_boundary(golden_dir):
    g = _golden(golden_dir)["int8_m256_interval"]
    r = oracle.centered_residue(np.array([128.0, -128.0, 127.0, 255.0, 256.0]), 256)
    assert int(r[0]) == g["residue_of_128"]
    assert list(map(int, r)) == [-128, -128, 127, -1, 0]
    full = oracle.centered_residue(np.arange(-600, 600, dtype=np.float64), 256)
    assert full.min() == g["value"][0] and full.max() == g["value"][1]


def test_residue_matches_pages_split_route(golden_dir):
    """Profiling Ozaki II section 10.1: |a| = u0 + 2^32 u1 and
    |a| mod m = [(u0 mod m) + beta (u1 mod m)] mod m, beta = 2^32 mod m,
    with the bracket at most 65280; valid for |a| < 2^63."""
    bracket_max = _golden(golden_dir)["split_bracket_max"]["value"]
    rng = np.random.default_rng(11)
    ints = [v for v in _interesting_integers(rng, 300) if abs(v) < 2 ** 63]
    x = np.array([float(v) for v in ints])
    for m in oracle.moduli(20):
        beta = (2 ** 32) % m
        r = oracle.centered_residue(x, m)
        for v, rv in zip(ints, r):
            a = abs(v)
            u0, u1 = a & 0xFFFFFFFF, a >> 32
            bracket = (u0 % m) + beta * (u1 % m)
            assert bracket <= bracket_max
            mag = bracket % m
            signed = (-mag) % m if v < 0 else mag
            centered = signed - m if signed > -(-m // 2) - 1 else signed
            assert int(rv) == centered


# --------------------------------------------------------------------------
# Products and output residues
# --------------------------------------------------------------------------
def test_residue_product_bruteforce():
    rng = np.random.default_rng(3)
    for shape in [(1, 1, 1), (3, 5, 2), (7, 64, 4)]:
        p, q, r = shape
        at = rng.integers(-128, 128, size=(p, q))
        bt = rng.integers(-128, 128, size=(q, r))
        at[0, 0] = -128
        bt[0, 0] = -128
        got = oracle.residue_product(at, bt)
        for i in range(p):
            for j in range(r):
                assert int(got[i, j]) == sum(int(at[i, l]) * int(bt[l, j]) for l in range(q))


def test_output_residue_nonnegative():
    vals = np.array([-(2 ** 31) + 1, -300, -1, 0, 1, 300, 2 ** 31 - 1], dtype=np.int64)
    for m in oracle.moduli(20):
        r = oracle.output_residue(vals, m)
        for v, rv in zip(vals, r):
            assert 0 <= int(rv) < m and (int(v) - int(rv)) % m == 0


# --------------------------------------------------------------------------
# CRT
# --------------------------------------------------------------------------
@pytest.mark.parametrize("s", [2, 8, 14, 18, 20])
def test_crt_unique_representative(s):
    rng = np.random.default_rng(s)
    mods = oracle.moduli(s)
    M = math.prod(mods)
    res = [rng.integers(0, m, size=50) for m in mods]
    res[0][0] = 0
    x = oracle.crt(res, s)
    for k in range(50):
        v = int(x[k])
        assert -M // 2 <= v < M // 2
        for t, m in enumerate(mods):
            assert v % m == int(res[t][k])


@pytest.mark.parametrize("mode", ["fast", "accu"])
@pytest.mark.parametrize("s", [2, 8, 14, 18, 20])
@pytest.mark.parametrize("phi", [0.5, 1.0, 4.0])
def test_crt_recovers_exact_integer_product(mode, s, phi):
    """X == A'B' against arbitrary-precision Python-int brute force."""
    rng = np.random.default_rng(100 * s + int(phi * 10))
    p, q, r = int(rng.integers(1, 7)), int(rng.integers(1, 9)), int(rng.integers(1, 7))
    A = generate(p, q, phi, 1000 + s)
    B = generate(q, r, phi, 2000 + s)
    out = oracle.ozaki2(A, B, s, mode)
    ap = [[int(v) for v in row] for row in out["Ap"]]
    bp = [[int(v) for v in row] for row in out["Bp"]]
    for i in range(p):
        for j in range(r):
            exact = sum(ap[i][l] * bp[l][j] for l in range(q))
            assert int(out["X"][i, j]) == exact
            assert abs(exact) <= 2 ** oracle.tau(s)
            assert sum(abs(ap[i][l] * bp[l][j]) for l in range(q)) <= 2 ** oracle.tau(s)


# --------------------------------------------------------------------------
# Scaling: fast
# --------------------------------------------------------------------------
def _rows_zoo(rng):
    yield generate(6, 700, 0.5, 5)
    yield generate(4, 513, 4.0, 6)
    a = generate(3, 300, 1.0, 7)
    a[0, :] = 0.0
    a[1, 5:] = 0.0
    a[2, 17] = 1e-300
    yield a
    yield np.array([[5e-324, -1e-310, 0.0, 3e-320]])
    yield np.array([[1e300, -1e-300, 1.0]])


@pytest.mark.parametrize("s", [2, 8, 14, 18, 20])
def test_fast_exponent_sound_and_near_maximal(s):
    t = oracle.tau(s)
    rng = np.random.default_rng(s)
    for rows in _rows_zoo(rng):
        d, e, S = oracle.fast_exponents(rows, s)
        for i in range(rows.shape[0]):
            norm2 = sum((Fraction(float(v)) ** 2 for v in rows[i]), Fraction(0))
            if norm2 == 0:
                assert d[i] == 0
                continue
            # the integer bound really bounds the squared norm
            assert norm2 <= Fraction(S[i]) * Fraction(2) ** (2 * (e[i] - oracle.F_BITS))
            scaled = norm2 * Fraction(4) ** int(d[i])
            assert scaled <= 2 ** t                                  # sound
            assert scaled * 4 * (1 + Fraction(1, 256)) > 2 ** t      # near-maximal


# --------------------------------------------------------------------------
# Scaling: accu
# --------------------------------------------------------------------------
@pytest.mark.parametrize("s", [2, 8, 14, 18, 20])
def test_accu_bound_inputs_round_upward(s):
    rows = generate(5, 200, 2.0, 9)
    rows[4, :] = 0.0
    e, abar = oracle.accu_bound_inputs(rows)
    assert e[4] is None and not abar[4].any()
    for i in range(4):
        mx = max(abs(float(v)) for v in rows[i])
        assert 2.0 ** (e[i] - 1) <= mx < 2.0 ** e[i]
        for l in range(rows.shape[1]):
            exact = Fraction(abs(float(rows[i, l]))) * Fraction(2) ** (oracle.Q_BITS - e[i])
            q_il = int(abar[i, l])
            assert 0 <= q_il <= 2 ** oracle.Q_BITS
            assert q_il - 1 < exact <= q_il


def test_eq18_equal_budget_on_flat_lines_accu():
    """All-ones 1 x q A and q x 1 B: accu d and b both equal Eq. 18's k.

    Ozaki II supplement section 2, Eq. 18: with |a'| <= 2^k and |b'| <= 2^k the
    product is bounded by q 2^(2k), and the equal budget is the largest k with
    q 4^k <= M/2 - 1.  For lines of ones the bound product is the exact product,
    so the accu exponents must be exactly that k (the fast mode's counterpart is
    test_eq18_equal_budget_on_flat_rows).
    """
    for s in (2, 8, 14, 18, 20):
        M = oracle.modulus_product(s)
        for j in range(0, 13):
            q = 1 << j
            k = 0
            while q * 4 ** (k + 1) <= M // 2 - 1:
                k += 1
            assert q * 4 ** k <= M // 2 - 1 < q * 4 ** (k + 1)
            out = oracle.accu_exponents(np.ones((1, q)), np.ones((q, 1)), s)
            assert int(out["d"][0]) == k and int(out["b"][0]) == k, (s, q)


def _pow2_at_least(v):
    """Smallest power of two >= v (v >= 1), by doubling."""
    p = 1
    while p < v:
        p *= 2
    return p


@pytest.mark.parametrize("s", [2, 8, 14, 18, 20])
def test_accu_exponent_maximal_against_bruteforce(s):
    """Bound product and its maxima by Python-int loops; d and b are the largest
    integers whose squared scale times the bound peak (rounded up to a power of two,
    so the equal split stays an integer exponent) fits the budget 2^tau:
      4^(d + e - Q) P2(rho) <= 2^tau < 4^(d + 1 + e - Q) P2(rho).
    The upward-quantized inputs are rebuilt here from exact Fractions."""
    t = oracle.tau(s)
    Q = oracle.Q_BITS
    A = generate(6, 37, 2.0, 300 + s)
    B = generate(37, 5, 2.0, 400 + s)
    A[4, :] = 0.0                        # zero row: d = 0
    out = oracle.accu_exponents(A, B, s)

    def quantize(line):
        mx = max(abs(Fraction(float(v))) for v in line)
        if mx == 0:
            return None, [0] * len(line)
        e = 0
        while Fraction(2) ** e <= mx:
            e += 1
        while Fraction(2) ** (e - 1) > mx:
            e -= 1
        qs = []
        for v in line:
            x = abs(Fraction(float(v))) * Fraction(2) ** (Q - e)
            qs.append(-((-x.numerator) // x.denominator))   # exact ceiling
        return e, qs

    rows = [quantize(A[i, :]) for i in range(A.shape[0])]
    cols = [quantize(B[:, j]) for j in range(B.shape[1])]
    y = [[sum(a * b for a, b in zip(rq, cq)) for (_, cq) in cols] for (_, rq) in rows]
    for lines, peaks, exps in ((rows, [max(r) for r in y], out["d"]),
                               (cols, [max(y[i][j] for i in range(len(rows))) for j in range(len(cols))], out["b"])):
        for (e, _), peak, d in zip(lines, peaks, exps):
            d = int(d)
            if e is None:
                assert d == 0
                continue
            assert peak >= 1
            p2 = _pow2_at_least(peak)
            assert Fraction(4) ** (d + e - Q) * p2 <= 2 ** t
            assert Fraction(4) ** (d + 1 + e - Q) * p2 > 2 ** t


@pytest.mark.parametrize("s", [8, 14, 20])
def test_accu_nonzero_line_with_zero_bound_peak(s):
    """A nonzero row of A whose products with every column of B vanish (its support
    meets only zero rows of B) has rho = 0, and likewise a column of B against zero
    columns of A has gamma = 0.  Reading taken: such a line is scaled as if its peak
    were 1, d = floor(tau / 2) + Q - e, which keeps |A'| <= 2^(floor(tau/2) + Q) like any
    line with a nonzero peak; its outputs are exactly 0 whatever its exponent."""
    t = oracle.tau(s)
    A = generate(4, 6, 1.0, 7)
    B = generate(6, 3, 1.0, 8)
    A[:, 2] = 0.0                        # column 2 of A is zero ...
    B[:, 1] = 0.0
    B[2, 1] = 1e200                      # ... so column 1 of B (support {2}) has gamma = 0
    B[4, :] = 0.0                        # row 4 of B is zero ...
    A[1, :] = 0.0
    A[1, 4] = -3e-250                    # ... so row 1 of A (support {4}) has rho = 0
    out = oracle.accu_exponents(A, B, s)
    assert int(out["rho"][1]) == 0 and int(out["gamma"][1]) == 0
    assert int(out["d"][1]) == t // 2 + oracle.Q_BITS - out["e"][1]
    assert int(out["b"][1]) == t // 2 + oracle.Q_BITS - out["f"][1]
    full = oracle.ozaki2(A, B, s, "accu")
    assert np.abs(full["Ap"][1]).max() <= 2.0 ** (t // 2 + oracle.Q_BITS)
    assert np.abs(full["Bp"][:, 1]).max() <= 2.0 ** (t // 2 + oracle.Q_BITS)
    assert not full["C"][1, :].any() and not full["C"][:, 1].any()
    assert all(int(v) == 0 for v in full["X"][1, :]) and all(int(v) == 0 for v in full["X"][:, 1])


@pytest.mark.parametrize("s", [2, 8, 14, 18, 20])
def test_accu_bound_product_and_scaling_sound(s):
    A = generate(5, 40, 1.5, 21 + s)
    B = generate(40, 4, 1.5, 31 + s)
    A[2, :] = 0.0
    out = oracle.accu_exponents(A, B, s)
    ab, bb = out["Abar"], out["Bbar"]
    for i in range(5):
        for j in range(4):
            assert int(out["Y"][i, j]) == sum(int(ab[i, l]) * int(bb[j, l]) for l in range(40))
    assert list(out["rho"]) == [max(int(v) for v in out["Y"][i]) for i in range(5)]
    assert list(out["gamma"]) == [max(int(out["Y"][i, j]) for i in range(5)) for j in range(4)]
    t = oracle.tau(s)
    d, b = out["d"], out["b"]
    for i in range(5):
        for j in range(4):
            bound = sum((abs(Fraction(float(A[i, l]))) * abs(Fraction(float(B[l, j])))
                         for l in range(40)), Fraction(0))
            assert bound * Fraction(2) ** int(d[i] + b[j]) <= 2 ** t


# --------------------------------------------------------------------------
# C_hat
# --------------------------------------------------------------------------
@pytest.mark.parametrize("mode", ["fast", "accu"])
@pytest.mark.parametrize("s", [8, 14, 18])
def test_small_integer_inputs_give_exact_product(mode, s):
    rng = np.random.default_rng(s)
    A = rng.integers(-1000, 1001, size=(17, 33)).astype(np.float64)
    B = rng.integers(-1000, 1001, size=(33, 9)).astype(np.float64)
    out = oracle.ozaki2(A, B, s, mode)
    assert (out["d"] >= 0).all() and (out["b"] >= 0).all()
    exact = A.astype(np.int64) @ B.astype(np.int64)
    assert np.array_equal(out["C"], exact.astype(np.float64))


@pytest.mark.parametrize("s", [8, 14, 18])
def test_identity_right_factor_closed_form(s):
    A = generate(9, 12, 1.0, 77)
    out = oracle.ozaki2(A, np.eye(12), s, "fast")
    t = oracle.tau(s)
    # column j of I: e = 1, S = 2^(2F-2), so b_j = floor((tau - 2F + 2)/2) + F - 1
    assert all(int(v) == (t - 2 * oracle.F_BITS + 2) // 2 + oracle.F_BITS - 1 for v in out["b"])
    for i in range(9):
        di = int(out["d"][i])
        for j in range(12):
            want = math.ldexp(float(math.trunc(math.ldexp(float(A[i, j]), di))), -di)
            assert out["C"][i, j] == want


@pytest.mark.parametrize("mode", ["fast", "accu"])
@pytest.mark.parametrize("s", [2, 8, 14, 18])
def test_error_within_truncation_bound(mode, s):
    """|C_hat - AB| <= sum_l (2^-d_i |b_lj| + 2^-b_j |a_il| + 2^-(d_i+b_j)) + ulp/2."""
    A = generate(6, 25, 1.0, 40 + s)
    B = generate(25, 5, 1.0, 50 + s)
    out = oracle.ozaki2(A, B, s, mode)
    exact = oracle.exact_product(A, B)
    for i in range(6):
        for j in range(5):
            di, bj = int(out["d"][i]), int(out["b"][j])
            bound = sum((Fraction(2) ** -di * abs(Fraction(float(B[l, j])))
                         + Fraction(2) ** -bj * abs(Fraction(float(A[i, l])))
                         + Fraction(2) ** -(di + bj)) for l in range(25))
            c = out["C"][i, j]
            half_ulp = Fraction(math.ulp(c)) / 2 if c != 0 else Fraction(0)
            assert abs(Fraction(float(c)) - exact[i, j]) <= bound + half_ulp


@pytest.mark.parametrize("mode", ["fast", "accu"])
def test_zero_lines_and_empty_shapes(mode):
    A = generate(5, 7, 0.5, 1)
    B = generate(7, 4, 0.5, 2)
    A[1, :] = 0
    B[:, 2] = 0
    out = oracle.ozaki2(A, B, 14, mode)
    assert out["d"][1] == 0 and out["b"][2] == 0
    assert not out["C"][1, :].any() and not out["C"][:, 2].any()
    for p, q, r in [(0, 3, 2), (3, 0, 2), (3, 2, 0)]:
        o = oracle.ozaki2(np.ones((p, q)), np.ones((q, r)), 8, mode)
        assert o["C"].shape == (p, r) and not o["C"].any()


def test_nonfinite_inputs_rejected():
    A = np.ones((2, 2))
    A[0, 1] = np.inf
    with pytest.raises(ValueError):
        oracle.ozaki2(A, np.ones((2, 2)), 8, "fast")


@pytest.mark.parametrize("mode", ["fast", "accu"])
def test_sampled_entries_equal_full_run(mode):
    A = generate(40, 300, 1.0, 8)
    B = generate(300, 35, 1.0, 9)
    full = oracle.ozaki2(A, B, 14, mode)
    rows, cols = [0, 7, 39], [1, 34]
    smp = oracle.ozaki2_sample(A, B, 14, mode, rows, cols)
    assert np.array_equal(smp["d"], full["d"][rows])
    assert np.array_equal(smp["b"], full["b"][cols])
    assert np.array_equal(smp["C"], full["C"][np.ix_(rows, cols)])
    assert all(int(a) == int(b) for a, b in zip(smp["X"].ravel(), full["X"][np.ix_(rows, cols)].ravel()))


def test_alpha_beta_update_pins():
    """The general entry point's update C <- alpha C_hat + beta C, pinned to facts outside
    the oracle: numpy's correctly rounded multiply, exact small-integer arithmetic, and a
    fused multiply-add case whose single rounding differs from two roundings."""
    rng = np.random.default_rng(11)
    c_hat = rng.standard_normal((5, 7))
    c = rng.standard_normal((5, 7))
    assert np.array_equal(oracle.alpha_beta_update(c_hat, 1.0, 0.0), c_hat)
    assert np.array_equal(oracle.alpha_beta_update(c_hat, 0.3, 0.0, c), 0.3 * c_hat)
    # beta == 0 never reads C
    assert np.array_equal(oracle.alpha_beta_update(c_hat, 2.0, 0.0, np.full_like(c, np.nan)), 2.0 * c_hat)
    ch = rng.integers(-1000, 1000, (4, 4)).astype(np.float64)
    ci = rng.integers(-1000, 1000, (4, 4)).astype(np.float64)
    assert np.array_equal(oracle.alpha_beta_update(ch, 3.0, -2.0, ci), 3.0 * ch - 2.0 * ci)
    a = 1.0 + 2.0 ** -30
    two_roundings = a * a - 1.0          # RN(a a) drops the 2^-60 term
    assert two_roundings == 2.0 ** -29
    got = oracle.alpha_beta_update(np.array([[a]]), a, 1.0, np.array([[-1.0]]))
    assert got[0, 0] == 2.0 ** -29 + 2.0 ** -60
