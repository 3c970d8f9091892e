"""The arithmetic identity behind the GEMM epilogue's output reduction R = P mod m
("Profiling Ozaki II: The Cost Behind Fast INT8 GEMMs", Part I section 1, blue stage),
checked with exact rational arithmetic.

The epilogue holds P' = P - h in INT32 (h = (m - 1) / 2 for odd m: the accumulators start
at -h), forms y = RN(P' RN(1/m) + 1.5 2^52 - e) in FP64 with e = h m^-1 (mod 256), reads
the low 24 bits L of y's low word as a signed number, and keeps the low byte of P' - m L.
The claim is that this byte is P mod m for every |P'| < 2^31: y - (1.5 2^52 - e) is
round(P'/m), because P' RN(1/m) lies within 2^-22 / m of P'/m and P'/m is never closer than
1 / (2m) to a half-integer, and m e = h (mod 256) shifts the centered remainder into
[0, m).  Here every step is evaluated exactly (the FMA's exact sum rounded once to the
integer grid of [2^52, 2^53), ties to even) at the ends of the INT32 range, around the
rounding boundaries and on random values, for every odd modulus the method uses.
"""
import random
from fractions import Fraction

import oracle

MAGIC = 3 * 2 ** 51  # 1.5 2^52


def _rn_int(x: Fraction) -> int:
    q, r = divmod(x.numerator, x.denominator)
    twice = 2 * r
    if twice > x.denominator or (twice == x.denominator and q % 2 == 1):
        q += 1
    return q


def _epilogue_byte(pp: int, m: int) -> int:
    h = (m - 1) // 2
    e = h * pow(m, -1, 256) % 256
    inv = Fraction(1.0 / m)                       # RN(1/m) in FP64
    y = _rn_int(pp * inv + (MAGIC - e))           # one FMA, one rounding; y in [2^52, 2^53)
    assert 2 ** 52 <= y < 2 ** 53
    low = (y - 2 ** 52) % 2 ** 32                 # the low word of y's bit pattern
    l24 = low % 2 ** 24
    l24 = l24 - 2 ** 24 if l24 >= 2 ** 23 else l24
    return (pp - m * l24) % 256                   # v_mad_i32_i24, low byte


def _cases(m: int, rng: random.Random):
    h = (m - 1) // 2
    lim = 2 ** 31 - 1
    vals = [lim, -lim, lim - h, -lim + h, 0, 1, -1, h, -h, h + 1, -h - 1]
    for k in [rng.randrange(-lim // m, lim // m) for _ in range(40)] + [lim // m, -(lim // m)]:
        for d in (-h - 1, -h, -1, 0, 1, h, h + 1):
            v = k * m + d
            if -lim <= v <= lim:
                vals.append(v)
    vals += [rng.randrange(-lim, lim + 1) for _ in range(200)]
    return vals


def test_epilogue_reduction_is_p_mod_m_for_every_odd_modulus():
    rng = random.Random(20260101)
    for m in oracle.moduli(20):
        if m % 2 == 0:
            continue  # m = 256: the low byte of P itself
        h = (m - 1) // 2
        for pp in _cases(m, rng):
            got = _epilogue_byte(pp, m)
            assert got == (pp + h) % m, f"m={m}, P'={pp}: {got} != {(pp + h) % m}"


def test_a_wrong_shift_breaks_the_identity():
    """The shift e is what moves the centered remainder into [0, m): without it the recipe
    gives the centered residue's low byte, which differs from P mod m for most values."""
    m = 253
    h = (m - 1) // 2
    inv = Fraction(1.0 / m)
    wrong = 0
    for pp in range(-1000, 1000):
        y = _rn_int(pp * inv + MAGIC)
        l24 = ((y - 2 ** 52) % 2 ** 32) % 2 ** 24
        l24 = l24 - 2 ** 24 if l24 >= 2 ** 23 else l24
        wrong += (pp - m * l24) % 256 != (pp + h) % m
    assert wrong > 1000
