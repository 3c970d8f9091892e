"""Plain CPU oracle of Ozaki Scheme II: FP64 C = A B from s INT8 modular GEMMs + CRT.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path.

Sources (web pages; cited by title and section):
  [P] "Profiling Ozaki II: The Cost Behind Fast INT8 GEMMs" (kevinhyj.github.io)
  [S] "Ozaki II supplement: INT8 range conditions and paper performance results"
      (edgep.me)

Pipeline ([P] Part I section 1, stage table; [S] section 1.1):
  1. bounds -> power-of-two diagonal scalings D = diag(2^d), E = diag(2^b)
  2. A' = trunc(D A), B' = trunc(B E)                      (toward zero)
  3. A_t = rho_{m_t}(A'), B_t = rho_{m_t}(B')              (centered residues)
  4. P_t = A_t B_t                                         (exact integer GEMM)
  5. R_t = P_t mod m_t                                     (nonnegative)
  6. X = CRT_M(R_1..R_s) in [-M/2, M/2)
  7. C_hat = D^-1 X E^-1

Everything here is exact: integers are NumPy int64 where they provably fit and
Python ints otherwise; the only library primitive is a float64 matrix product
for P_t, which is exact because every term is an integer of magnitude <= 2^14
and every partial sum stays below q * 2^14 < 2^53 (below 2^31 for q < 2^17,
[S] section 1.3; the oracle takes any q).

Readings taken where the pages leave a step open (each also listed in the
design notes of the repository):
  * moduli: the first s of the pairwise-coprime integers taken greedily in
    descending order from 256 ([S] section 1.2 says <= 256, pairwise coprime,
    larger is better; the list itself is not printed).
  * reconstruction budget: tau = floor(log2(M/2 - 1)); scalings guarantee
    |(A'B')_ij| <= 2^tau <= M/2 - 1, which is the condition 2 c_max < M of
    [S] section 1.1.
  * fast bound ([P] section 2 Cauchy-Schwarz, section 5.1 max-abs and
    sum-of-squares, upward rounding): the sum of squares is taken exactly on
    integers, each |a| quantized upward to F_BITS fractional bits relative to
    the max-abs exponent of its CHUNK-long block, blocks combined with an
    upward-rounded shift.  The budget 2^tau is split equally between the row
    of A and the column of B (as in Eq. 18 of [S] section 2) and d is the
    largest integer that keeps the scaled squared-norm bound <= 2^tau.
  * accu bound ([P] section 2 and section 5.1 "accu"): |A| and |B| quantized
    upward to integers in [0, 2^Q_BITS] relative to each row's / column's
    max-abs exponent, one exact integer product Y, row maxima rho_i and column
    maxima gamma_j, equal split through Y_ij <= sqrt(rho_i gamma_j).
  * X -> FP64: one correctly rounded (nearest-even) conversion of the exact
    value X * 2^(-d_i - b_j).

Pins (tests/test_oracle_pins.py): moduli, M and tau against the pages' range
figures; residues against their definition by brute force and against the
split-integer route of [P] section 10.1; products and X = A'B' against Python
integer brute force; scalings against exact rational soundness bounds, and the
exponents of both modes against Eq. 18 of [S] section 2 on flat lines (where the
equal budget is the exact exponent) and against maximality under the equal
split (accu: bound product and maxima by Python-int brute force); C_hat against
exact products and closed forms.  The exponent rule away from flat lines is this
oracle's reading (the pages give no formula), so its agreement with another
implementation's choice there is not pinned; its value on flat lines, its
soundness and its maximality are.
"""
from __future__ import annotations

import math
from fractions import Fraction

import time

import numpy as np

__all__ = [
    "F_BITS", "CHUNK", "Q_BITS", "MIN_S", "MAX_S",
    "moduli", "modulus_product", "tau",
    "split", "exponent_of", "fast_stats", "fast_exponents",
    "accu_bound_inputs", "accu_exponents",
    "scale_truncate", "centered_residue", "residue_product",
    "output_residue", "crt", "inverse_scale",
    "ozaki2", "ozaki2_sample", "clog2",
]

F_BITS = 20   # fractional bits of the upward-quantized |a| in the fast bound
CHUNK = 256   # block length along the inner dimension for the fast bound
Q_BITS = 6    # accu bound inputs are integers in [0, 2^Q_BITS] (fit in int8)
MIN_S, MAX_S = 2, 20
_NEG = -(1 << 40)  # "no nonzero element" exponent sentinel


# ---------------------------------------------------------------------------
# Moduli, M and the reconstruction budget ([S] sections 1.1, 1.2, 1.4)
# ---------------------------------------------------------------------------
def moduli(s: int) -> list[int]:
    """First s pairwise-coprime integers taken greedily downward from 256.

    [S] section 1.2: m <= 256 keeps centered residues inside INT8 and moduli
    must be pairwise coprime; larger moduli give more range bits per GEMM.
    """
    if not (MIN_S <= s <= MAX_S):
        raise ValueError(f"s must be in [{MIN_S}, {MAX_S}], got {s}")
    chosen: list[int] = []
    m = 256
    while len(chosen) < s:
        if all(math.gcd(m, c) == 1 for c in chosen):
            chosen.append(m)
        m -= 1
    return chosen


def modulus_product(s: int) -> int:
    """M = prod_t m_t ([P] Part I section 1)."""
    return math.prod(moduli(s))


def tau(s: int) -> int:
    """Largest integer with 2^tau <= M/2 - 1 (M is even: 256 is a modulus)."""
    half = modulus_product(s) // 2
    return (half - 1).bit_length() - 1


def clog2(x: int) -> int:
    """ceil(log2(x)) for an integer x >= 1, i.e. bitlen(x - 1)."""
    if x < 1:
        raise ValueError("clog2 needs x >= 1")
    return (int(x) - 1).bit_length()


# ---------------------------------------------------------------------------
# Exact decomposition of FP64 values
# ---------------------------------------------------------------------------
def _check_finite(x: np.ndarray, name: str) -> None:
    if not np.all(np.isfinite(x)):
        raise ValueError(f"{name} holds non-finite values; the method is defined for finite inputs")


def split(x: np.ndarray):
    """|x| = mu * 2**eta with integer 0 <= mu < 2**53 (exact, elementwise).

    Zero gives mu = 0.  Subnormals are handled: frexp normalizes them.
    """
    mant, ex = np.frexp(np.abs(np.asarray(x, dtype=np.float64)))
    mu = np.ldexp(mant, 53).astype(np.int64)   # exact: <= 53 significant bits
    eta = ex.astype(np.int64) - 53
    return mu, eta


def _bitlen53(mu: np.ndarray) -> np.ndarray:
    """Bit length of nonnegative integers < 2**53 (exact via float64)."""
    return np.frexp(mu.astype(np.float64))[1].astype(np.int64)


def exponent_of(x: np.ndarray) -> np.ndarray:
    """E(x) with 2^(E-1) <= |x| < 2^E for x != 0; _NEG for x == 0."""
    mu, eta = split(x)
    return np.where(mu > 0, eta + _bitlen53(mu), _NEG)


def _ceil_mul_pow2(mu: np.ndarray, k: np.ndarray) -> np.ndarray:
    """ceil(mu * 2**k) elementwise, exact, for int64 mu >= 0 and int64 k.

    Callers guarantee the result fits comfortably in int64 when k > 0.
    """
    mu = np.asarray(mu, dtype=np.int64)
    k = np.broadcast_to(np.asarray(k, dtype=np.int64), mu.shape)
    out = np.zeros(mu.shape, dtype=np.int64)
    left = (k >= 0) & (mu > 0)
    out[left] = mu[left] << k[left]
    right = (k < 0) & (mu > 0)
    sh = -k[right]
    small = sh <= 62
    vals = mu[right]
    shc = np.minimum(sh, 62)
    ceil_small = (vals + (np.int64(1) << shc) - 1) >> shc
    out[right] = np.where(small, ceil_small, 1)  # tiny positive -> 1
    return out


# ---------------------------------------------------------------------------
# fast bound: max-abs and upward sum of squares per row ([P] sections 2, 5.1)
# ---------------------------------------------------------------------------
def fast_stats(rows: np.ndarray):
    """Per row of ``rows`` (2-D): (e_i, S_i) with ||row_i||_2^2 <= 4^(e_i-F) S_i.

    e_i = E(max_l |a_il|); the row is cut into CHUNK-long blocks; in block c
    with exponent e_ic = E(block max), u_l = ceil(|a_il| 2^(F - e_ic)) is the
    upward quantization of |a_il| ([P] section 5.1: upward rounding so the
    bound is never underestimated); S_ic = sum u_l^2 exactly; then
    S_i = sum_c ceil(S_ic / 4^(e_i - e_ic)).  All-zero rows give (None, 0).
    """
    rows = np.asarray(rows, dtype=np.float64)
    p, q = rows.shape
    e_out: list = [None] * p
    s_out = [0] * p
    if p == 0 or q == 0:
        return e_out, s_out
    nch = -(-q // CHUNK)
    pad = nch * CHUNK - q
    blk = 1024  # rows per block, bounds memory
    for r0 in range(0, p, blk):
        a = np.pad(rows[r0:r0 + blk], ((0, 0), (0, pad)))
        nb = a.shape[0]
        mu, eta = split(a)
        mu = mu.reshape(nb, nch, CHUNK)
        eta = eta.reshape(nb, nch, CHUNK)
        ex = np.where(mu > 0, eta + _bitlen53(mu), _NEG)
        e_c = ex.max(axis=2)                                   # block max-abs exponent
        k = np.where(mu > 0, eta + F_BITS - e_c[:, :, None], 0)
        u = _ceil_mul_pow2(mu, k)                              # in [0, 2^F]
        s_c = (u * u).sum(axis=2)                              # <= CHUNK * 2^(2F)
        for i in range(nb):
            live = [c for c in range(nch) if s_c[i, c] > 0]
            if not live:
                continue
            e_i = max(int(e_c[i, c]) for c in live)
            total = 0
            for c in live:
                sh = 2 * (e_i - int(e_c[i, c]))
                total += -((-int(s_c[i, c])) >> sh)           # ceil(S_ic / 2^sh)
            e_out[r0 + i] = e_i
            s_out[r0 + i] = total
    return e_out, s_out


def fast_exponents(rows: np.ndarray, s: int):
    """Scaling exponents for the fast mode, one per row of ``rows``.

    d_i = floor((tau - clog2(S_i)) / 2) + F - e_i, the largest integer with
    4^(d_i + e_i - F) S_i <= 2^tau, so ||2^d_i row_i||_2 <= 2^(tau/2); with the
    Cauchy-Schwarz bound of [P] section 2 this gives |(A'B')_ij| <= 2^tau.
    All-zero rows get d_i = 0.  Returns (d, e, S).
    """
    t = tau(s)
    e, S = fast_stats(rows)
    d = np.zeros(len(e), dtype=np.int64)
    for i, (ei, si) in enumerate(zip(e, S)):
        if ei is None:
            continue
        d[i] = (t - clog2(si)) // 2 + F_BITS - ei
    return d, e, S


# ---------------------------------------------------------------------------
# accu bound: upward INT8 quantization + one integer GEMM ([P] sections 2, 5.1)
# ---------------------------------------------------------------------------
def accu_bound_inputs(rows: np.ndarray):
    """Abar_il = ceil(|a_il| 2^(Q - e_i)) in [0, 2^Q], e_i = E(max_l |a_il|).

    [P] section 2: absolute inputs scaled and rounded upward to INT8 so each
    reconstructed entry Abar_il 2^(e_i - Q) bounds |a_il|.  Zero rows give e
    = None and an all-zero Abar row.  Returns (e (list), Abar int64 array).
    """
    rows = np.asarray(rows, dtype=np.float64)
    p, q = rows.shape
    mu, eta = split(rows)
    ex = np.where(mu > 0, eta + _bitlen53(mu), _NEG)
    e_row = ex.max(axis=1) if q > 0 else np.full(p, _NEG, dtype=np.int64)
    k = np.where(mu > 0, eta + Q_BITS - e_row[:, None], 0)
    abar = _ceil_mul_pow2(mu, k)
    e_list = [None if int(v) == _NEG else int(v) for v in e_row]
    return e_list, abar


def _accu_d(e_list, peaks, s: int) -> np.ndarray:
    """d = floor((tau - clog2(max(peak, 1))) / 2) + Q - e; zero line -> 0.

    The largest integer with 4^(d + e - Q) 2^clog2(peak) <= 2^tau: the budget split
    equally through Y_ij <= sqrt(rho_i gamma_j).  A nonzero line whose peak is 0 (every
    one of its bound products vanishes, so its outputs are exactly 0) is scaled as a
    line of peak 1, which keeps its |A'| below 2^(floor(tau/2) + Q) like every other line.
    """
    t = tau(s)
    d = np.zeros(len(e_list), dtype=np.int64)
    for i, (ei, pk) in enumerate(zip(e_list, peaks)):
        if ei is None:
            continue
        d[i] = (t - clog2(max(int(pk), 1))) // 2 + Q_BITS - ei
    return d


def accu_exponents(A: np.ndarray, B: np.ndarray, s: int):
    """Row exponents d (for A) and column exponents b (for B) of the accu mode.

    Y = Abar Bbar exactly (integers <= q 2^(2Q) < 2^31); rho_i = max_j Y_ij and
    gamma_j = max_i Y_ij ([P] section 5.1: row/column maxima of the bound
    output give the final exponents).  Since |a_il| <= Abar_il 2^(e_i - Q) and
    Y_ij <= sqrt(rho_i gamma_j), the split d_i, b_j below keeps
    (|A'||B'|)_ij <= 2^tau.  Returns dict with d, b, e, f, Abar, Bbar, Y, rho, gamma.
    """
    e, abar = accu_bound_inputs(A)
    f, bbar_t = accu_bound_inputs(np.asarray(B).T)      # rows of B^T = columns of B
    y = (abar.astype(np.float64) @ bbar_t.T.astype(np.float64)).astype(np.int64)
    p, r = y.shape
    rho = y.max(axis=1) if r > 0 else np.zeros(p, dtype=np.int64)
    gamma = y.max(axis=0) if p > 0 else np.zeros(r, dtype=np.int64)
    d = _accu_d(e, rho, s)
    b = _accu_d(f, gamma, s)
    return dict(d=d, b=b, e=e, f=f, Abar=abar, Bbar=bbar_t, Y=y, rho=rho, gamma=gamma)


# ---------------------------------------------------------------------------
# Scale + truncate, residues, products, output residues
# ---------------------------------------------------------------------------
def scale_truncate(rows: np.ndarray, d: np.ndarray) -> np.ndarray:
    """trunc(2^d_i * a_il) per row i, exact ([P] Part I section 1: toward zero).

    The result is an integer with at most 53 significant bits, so it is
    returned exactly as float64.
    """
    rows = np.asarray(rows, dtype=np.float64)
    mu, eta = split(rows)
    sig = eta + np.asarray(d, dtype=np.int64)[:, None]
    up = np.ldexp(mu.astype(np.float64), np.clip(sig, 0, 4000).astype(np.int32))
    down = (mu >> np.clip(-sig, 0, 63)).astype(np.float64)
    mag = np.where(sig >= 0, up, down)
    return np.where(rows < 0, -mag, mag)


def centered_residue(xp: np.ndarray, m: int) -> np.ndarray:
    """rho_m(x'): the integer in [-floor(m/2), ceil(m/2) - 1] congruent to x'.

    [S] section 1.2.  ``xp`` holds exact integers as float64 (possibly far
    beyond 2^63): |x'| = mu 2^eta, so |x'| mod m = (mu mod m)(2^eta mod m) mod m
    when eta >= 0, and mu >> -eta is the integer itself when eta < 0.
    """
    mu, eta = split(xp)
    pos = eta >= 0
    emax = int(eta[pos].max()) if np.any(pos) else 0
    pow_tab = np.array([pow(2, k, m) for k in range(emax + 1)], dtype=np.int64)
    r_pos = ((mu % m) * pow_tab[np.clip(eta, 0, emax)]) % m
    r_neg = (mu >> np.clip(-eta, 0, 63)) % m
    r = np.where(pos, r_pos, r_neg)
    r = np.where(np.asarray(xp) < 0, (-r) % m, r)          # residue of the signed value
    h = m // 2
    return ((r + h) % m) - h


def residue_product(at: np.ndarray, bt: np.ndarray) -> np.ndarray:
    """P_t = A_t B_t as int64 (float64 GEMM is exact here, see module doc)."""
    return (np.asarray(at, dtype=np.float64) @ np.asarray(bt, dtype=np.float64)).astype(np.int64)


def output_residue(p_t: np.ndarray, m: int) -> np.ndarray:
    """R_t = P_t mod m_t, the nonnegative residue ([P] Part I section 1, blue stage)."""
    return np.mod(p_t, m)


# ---------------------------------------------------------------------------
# CRT and inverse scaling
# ---------------------------------------------------------------------------
def crt(residues, s: int) -> np.ndarray:
    """X: the unique integer in [-M/2, M/2) with X = R_t (mod m_t) for all t.

    Mixed-radix (Garner) digits in int64, then X as Python ints (object array).
    """
    mods = moduli(s)
    M = math.prod(mods)
    shape = np.asarray(residues[0]).shape
    digits = []
    for t, m in enumerate(mods):
        acc = np.zeros(shape, dtype=np.int64)
        w = 1  # m_1 ... m_{k} mod m
        for k in range(t):
            acc = (acc + digits[k] * w) % m
            w = (w * mods[k]) % m
        inv = pow(w, -1, m) if t > 0 else 1
        digits.append(((np.asarray(residues[t], dtype=np.int64) - acc) * inv) % m)
    x = np.zeros(shape, dtype=object)
    radix = 1
    for t, m in enumerate(mods):
        x = x + digits[t].astype(object) * radix
        radix *= m
    half = M // 2
    return np.where(x >= half, x - M, x)


def inverse_scale(x: np.ndarray, d: np.ndarray, b: np.ndarray) -> np.ndarray:
    """C_hat_ij = RN(X_ij * 2^(-d_i - b_j)), correctly rounded to nearest-even.

    Python int true division and int->float conversion are correctly rounded.
    """
    p, r = x.shape
    out = np.empty((p, r), dtype=np.float64)
    for i in range(p):
        for j in range(r):
            k = int(d[i]) + int(b[j])
            v = int(x[i, j])
            out[i, j] = v / (1 << k) if k >= 0 else float(v << (-k))
    return out


# ---------------------------------------------------------------------------
# Whole pipeline
# ---------------------------------------------------------------------------
def _exponents(A, B, s, mode):
    if mode == "fast":
        d, _, _ = fast_exponents(A, s)
        b, _, _ = fast_exponents(np.asarray(B).T, s)
        return dict(d=d, b=b)
    if mode == "accu":
        return accu_exponents(A, B, s)
    raise ValueError(f"mode must be 'fast' or 'accu', got {mode!r}")


def ozaki2(A: np.ndarray, B: np.ndarray, s: int, mode: str = "fast") -> dict:
    """Every intermediate of one Ozaki II product C_hat ~ A B (small sizes).

    Returns a dict with d, b, Ap (A'), Bp (B'), At, Bt, P, R (lists over t,
    At p x q, Bt q x r, P and R p x r), X (object array), C (float64), plus the
    accu-only bound quantities when mode == 'accu'.
    """
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[0]:
        raise ValueError("A must be p x q and B q x r")
    _check_finite(A, "A")
    _check_finite(B, "B")
    mods = moduli(s)
    out = _exponents(A, B, s, mode)
    d, b = out["d"], out["b"]
    ap = scale_truncate(A, d)
    bp = scale_truncate(B.T, b).T
    at, bt, pt, rt = [], [], [], []
    for m in mods:
        a_m = centered_residue(ap, m)
        b_m = centered_residue(bp, m)
        p_m = residue_product(a_m, b_m)
        at.append(a_m)
        bt.append(b_m)
        pt.append(p_m)
        rt.append(output_residue(p_m, m))
    x = crt(rt, s) if rt[0].size else np.zeros(rt[0].shape, dtype=object)
    c = inverse_scale(x, d, b)
    out.update(Ap=ap, Bp=bp, At=at, Bt=bt, P=pt, R=rt, X=x, C=c, moduli=mods)
    return out


def ozaki2_sample(A, B, s: int, mode: str, rows, cols, timings: dict | None = None) -> dict:
    """The same quantities restricted to output rows ``rows`` and columns ``cols``.

    Scaling exponents still see whole rows of A / columns of B (fast) or the
    whole bound product (accu), so the sampled entries equal those of a full
    run.  At, Ap are len(rows) x q; Bt, Bp are q x len(cols).  When ``timings``
    is a dict it receives the wall seconds of each stage (scaling, residues,
    gemm = products and output residues, crt = reconstruction and inverse
    scaling); the computation is the same either way.
    """
    clock = time.perf_counter
    t_start = clock()
    spent = {"scaling": 0.0, "residues": 0.0, "gemm": 0.0, "crt": 0.0}
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    mods = moduli(s)
    a_rows = A[rows]
    b_cols = B[:, cols]
    _check_finite(a_rows, "A rows")
    _check_finite(b_cols, "B columns")
    out: dict = {}
    if mode == "fast":
        d, _, _ = fast_exponents(a_rows, s)
        b, _, _ = fast_exponents(b_cols.T, s)
    elif mode == "accu":
        _check_finite(A, "A")
        _check_finite(B, "B")
        e, abar = accu_bound_inputs(A)
        f, bbar_t = accu_bound_inputs(B.T)
        ab = abar.astype(np.float64)
        bb = bbar_t.astype(np.float64)
        y_rows = (ab[rows] @ bb.T).astype(np.int64)          # len(rows) x r
        y_cols = (ab @ bb[cols].T).astype(np.int64)          # p x len(cols)
        rho = y_rows.max(axis=1) if y_rows.shape[1] else np.zeros(len(rows), np.int64)
        gamma = y_cols.max(axis=0) if y_cols.shape[0] else np.zeros(len(cols), np.int64)
        d = _accu_d([e[i] for i in rows], rho, s)
        b = _accu_d([f[j] for j in cols], gamma, s)
        out.update(rho=rho, gamma=gamma, Abar=abar[rows], Bbar=bbar_t[cols],
                   e=[e[i] for i in rows], f=[f[j] for j in cols])
    else:
        raise ValueError(f"mode must be 'fast' or 'accu', got {mode!r}")
    t0 = clock()
    spent["scaling"] = t0 - t_start
    ap = scale_truncate(a_rows, d)
    bp = scale_truncate(b_cols.T, b).T
    at, bt, pt, rt = [], [], [], []
    for m in mods:
        a_m = centered_residue(ap, m)
        b_m = centered_residue(bp, m)
        t2 = clock()
        p_m = residue_product(a_m, b_m)
        at.append(a_m)
        bt.append(b_m)
        pt.append(p_m)
        rt.append(output_residue(p_m, m))
        spent["gemm"] += clock() - t2
    t3 = clock()
    x = crt(rt, s) if rt[0].size else np.zeros(rt[0].shape, dtype=object)
    c = inverse_scale(x, d, b)
    spent["crt"] = clock() - t3
    # scaled truncation and residues: everything between the scalings and the CRT but the products
    spent["residues"] = (t3 - t0) - spent["gemm"]
    if timings is not None:
        timings.update(spent)
    out.update(d=d, b=b, Ap=ap, Bp=bp, At=at, Bt=bt, P=pt, R=rt, X=x, C=c, moduli=mods,
               rows=rows, cols=cols)
    return out


def alpha_beta_update(c_hat: np.ndarray, alpha: float, beta: float, c: np.ndarray | None = None) -> np.ndarray:
    """C <- alpha C_hat + beta C, the update of the library's general entry point.

    The pages define only C = A B; scaling the product and accumulating into C follow
    the usual GEMM convention, with this rounding: beta == 0 gives RN(alpha C_hat) and
    C is not read; otherwise RN(alpha C_hat + RN(beta C)), one rounding of the sum (a
    fused multiply-add).  Computed with exact rationals and one correctly rounded
    conversion per entry.
    """
    c_hat = np.asarray(c_hat, dtype=np.float64)
    out = np.empty_like(c_hat)
    fa = Fraction(alpha)
    for idx in np.ndindex(c_hat.shape):
        v = fa * Fraction(float(c_hat[idx]))
        if beta != 0.0:
            v += Fraction(float(np.float64(beta) * np.float64(c[idx])))
        out[idx] = float(v)
    return out


__all__.append("alpha_beta_update")


def exact_product(A: np.ndarray, B: np.ndarray):
    """(A B) as exact Fractions (object array) for tiny inputs; for error pins."""
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    p, q = A.shape
    r = B.shape[1]
    out = np.empty((p, r), dtype=object)
    for i in range(p):
        for j in range(r):
            out[i, j] = sum((Fraction(float(A[i, l])) * Fraction(float(B[l, j])) for l in range(q)),
                            Fraction(0))
    return out


__all__.append("exact_product")
