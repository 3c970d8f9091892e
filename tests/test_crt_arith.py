"""The per-output reconstruction arithmetic of the HIP library, run on the host.

The CRT stage ("Profiling Ozaki II: The Cost Behind Fast INT8 GEMMs", Part I section 1, red
stage) must return, for residues R_t = X mod m_t, the exact integer X in [-M/2, M/2) and
RN(X) 2^scale (round to nearest, ties to even).  ``tests/crt_harness.cpp`` runs the
library's own device functions (``oz2_crt_round.hpp``: limb sums, the quotient estimate,
the carries and the rounding) on the CPU; here they are checked against Python's exact
integers, whose int -> float conversion is correctly rounded, on the values where such code
goes wrong: exact ties and their neighbours, powers of two, the largest |X| the scalings
allow (2^tau), and the magnitudes where the rounding switches between its cases.
"""
import math
import os
import random
import struct
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp64_gemm_emulation_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def moduli(s):
    """Pairwise coprime moduli taken greedily downward from 256."""
    out = []
    c = 256
    while len(out) < s:
        if all(math.gcd(c, m) == 1 for m in out):
            out.append(c)
        c -= 1
    return out


def tau(M):
    return (M // 2 - 1).bit_length() - 1


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    exe = str(tmp_path_factory.mktemp("crt") / "crt_harness")
    cmd = [HIPCC, "-x", "hip", "--offload-host-only", "-std=c++17", "-O2", f"-I{CSRC}",
           os.path.join(ROOT, "tests", "crt_harness.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return exe


def with_rounding_bits(v, lsb, rnd, sticky, rng):
    """v > 2^54 with its last significand bit, round bit and sticky bits (at v's own
    binade, 53-bit significand) set to the given values."""
    e = v.bit_length()
    low = e - 54                                               # bits below the round bit
    v = (v >> (low + 2)) << (low + 2)
    v |= (lsb << (low + 1)) | (rnd << low)
    if sticky:
        v |= rng.randint(1, (1 << low) - 1) if low > 0 else 0
    return v


def cases_for(s, rng):
    M = math.prod(moduli(s))
    T = tau(M)
    xs = {0, 1, -1, 2, -2, 2**T, -(2**T), 2**T - 1, -(2**T - 1)}
    for e in range(T + 1):
        for d in (-1, 0, 1):
            xs.update({2**e + d, -(2**e) + d})
    # magnitudes where the rounding switches level: |floor(X / 2^(32 j))| near 2^21
    for j in range(1, 6):
        for base in (2 ** (32 * j + 21), 2 ** (32 * j + 20)):
            for d in (-(2 ** (32 * j)) - 1, -(2 ** (32 * j)), -1, 0, 1, 2 ** (32 * j) - 1, 2 ** (32 * j)):
                for x in (base + d, -base + d):
                    if abs(x) <= 2**T:
                        xs.add(x)
    # exact ties (a 54-bit odd significand) and their neighbours, in every binade above 2^53
    for e in range(54, T + 1):
        for _ in range(6):
            m = rng.getrandbits(53) | (1 << 53) | 1          # 54 bits, odd: halfway
            x = m << (e - 54)
            if x > 2**T:
                continue
            for d in (-1, 0, 1):
                xs.update({x + d, -(x + d)})
        x = 2**e + 2 ** (e - 53)                              # tie just above a power of two
        if x <= 2**T:
            xs.update({x, -x, x + 1, x - 1})
    # every (last bit, round bit, sticky) combination at random magnitudes, and in a band
    # around every power of two (where a limb-level switch of the rounding can sit, for any
    # limb width): |X| within 2^(e - 12) of 2^e
    mags = [rng.randint(2**55, 2**T) for _ in range(60)] if T > 56 else []
    for e in range(56, T + 1):
        for v in (2**e - rng.randint(1, 2 ** (e - 12)), 2**e + rng.randint(0, 2 ** (e - 12))):
            if 2**55 < v <= 2**T:
                mags.append(v)
    for v in mags:
        for lsb in (0, 1):
            for rnd in (0, 1):
                for st in (0, 1):
                    x = with_rounding_bits(v, lsb, rnd, st, rng)
                    if abs(x) <= 2**T:
                        xs.update({x, -x})
    for _ in range(400):
        e = rng.randint(0, T)
        xs.add(rng.randint(-(2**e), 2**e))
    return sorted(xs)


def rn_scaled(x, sc):
    """RN(x 2^sc) rounded once: Python's int -> float conversion and int / int true division
    are correctly rounded (to nearest, ties to even), below the normal range too."""
    return float(x << sc) if sc >= 0 else x / (1 << -sc)


def subnormal_cases(s, rng):
    """(X, scale) pairs whose result X 2^scale lies below 2^-1022: X in every binade (with
    random low bits, exact ties at the result's unit 2^g, and their neighbours), and scales
    that put the result's unit at each bit position g from X's low end up past its top
    (down to results that round to 0 or to the smallest subnormal)."""
    M = math.prod(moduli(s))
    T = tau(M)
    out = []
    for e in range(1, T + 1):
        xs = [rng.randint(2 ** (e - 1), 2**e - 1)] if e > 1 else [1]
        for x in xs:
            n = x.bit_length()
            for g in sorted({1, 2, max(1, n - 53), max(1, n - 52), max(1, n - 20), n - 1 if n > 1 else 1, n, n + 1, n + 2}):
                sc = -1074 - g
                tie = ((x >> g) << g) | (1 << (g - 1))                 # exactly halfway at unit 2^g
                for v in (x, tie, tie - 1, tie + 1, tie + (1 << g)):
                    if 0 < v <= 2**T and abs(v) * 2.0 ** -g < 2.0**52:
                        out.extend([(v, sc), (-v, sc)])
    # around the normal boundary: results just below and at 2^-1022
    for g in (1, 3, 30):
        for v in ((1 << (52 + g)) - 1, (1 << (52 + g)) - (1 << (g - 1)), (1 << (52 + g)) - (1 << g) - (1 << (g - 1))):
            if v <= 2**T:
                out.extend([(v, -1074 - g), (-v, -1074 - g)])
    return out


def scale_for(x, rng):
    """A scale that keeps |RN(x)| 2^scale normal and finite."""
    if x == 0:
        return rng.randint(-100, 100)
    return rng.randint(-1000, 1000 - abs(x).bit_length())


@pytest.mark.parametrize("s", list(range(2, 21)))
def test_crt_arith_exact_words_and_rounding(harness, s):
    rng = random.Random(1000 + s)
    ms = moduli(s)
    xs = cases_for(s, rng)
    lines, want = [], []
    for x in xs:
        sc = scale_for(x, rng)
        lines.append(f"{s} {sc} " + " ".join(str(x % m) for m in ms))
        words = [(x >> (32 * k)) & 0xFFFFFFFF for k in range(5)]
        val = rn_scaled(x, sc)
        bits = struct.unpack("<Q", struct.pack("<d", val))[0]
        want.append(" ".join(f"{w:08x}" for w in words) + f" {bits:016x}")
    res = subprocess.run([harness], input="\n".join(lines) + "\n", capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    got = res.stdout.split("\n")[: len(want)]
    bad = [(x, g, w) for x, g, w in zip(xs, got, want) if g != w]
    assert not bad, f"s={s}: {len(bad)} of {len(xs)} differ, first: X={bad[0][0]} got {bad[0][1]} want {bad[0][2]}"


def test_crt_arith_cases_cover_ties_and_binades():
    """The case list holds exact ties, and every rounding-bit pattern with both signs in
    every binade from 2^56 to 2^tau, for the largest s."""
    rng = random.Random(7)
    xs = cases_for(20, rng)
    ties = [x for x in xs if abs(x).bit_length() > 54 and
            (abs(x) >> (abs(x).bit_length() - 54)) & 1 and
            abs(x) % (1 << (abs(x).bit_length() - 54)) == 0]
    assert len(ties) > 100
    T = tau(math.prod(moduli(20)))
    seen = set()
    for x in xs:
        e = abs(x).bit_length()
        if e > 56:
            low = e - 54
            seen.add((e, x < 0, (abs(x) >> (low + 1)) & 1, (abs(x) >> low) & 1, abs(x) % (1 << low) != 0))
    missing = [(e, neg, a, b, c) for e in range(58, T) for neg in (False, True)
               for a in (0, 1) for b in (0, 1) for c in (False, True) if (e, neg, a, b, c) not in seen]
    assert not missing, missing[:5]


@pytest.mark.parametrize("s", [2, 3, 8, 14, 18, 20])
def test_crt_arith_subnormal_results_rounded_once(harness, s):
    """Results below the normal range are RN(X 2^scale) itself, one rounding at the
    subnormal unit 2^-1074 (ties to even), not X rounded to 53 bits and then again."""
    rng = random.Random(2000 + s)
    ms = moduli(s)
    cases = subnormal_cases(s, rng)
    lines, want = [], []
    for x, sc in cases:
        lines.append(f"{s} {sc} " + " ".join(str(x % m) for m in ms))
        bits = struct.unpack("<Q", struct.pack("<d", rn_scaled(x, sc)))[0]
        want.append(f"{bits:016x}")
    res = subprocess.run([harness], input="\n".join(lines) + "\n", capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    got = [ln.split()[-1] for ln in res.stdout.split("\n")[: len(want)]]
    bad = [(c, g, w) for c, g, w in zip(cases, got, want) if g != w]
    assert not bad, f"s={s}: {len(bad)} of {len(cases)} differ, first: X, scale={bad[0][0]} got {bad[0][1]} want {bad[0][2]}"
    # where X can exceed 53 bits, the cases reach results that a 53-bit rounding followed by a
    # scaling gets wrong
    twice = sum(1 for x, sc in cases if math.ldexp(float(x), sc) != rn_scaled(x, sc))
    assert twice > 0 or tau(math.prod(ms)) < 54
