"""Seeded synthetic FP64 inputs for the Ozaki II GEMM emulation.

This module only draws random matrices; it holds none of the method's
arithmetic, so both the HIP path's tests/benchmark and the CPU oracle can take
their inputs from it without sharing any computation.

Entry distribution: ``(U(0,1) - 0.5) * exp(phi * N(0,1))``.  The profiling
study ("Profiling Ozaki II: The Cost Behind Fast INT8 GEMMs", Part II section 4)
drives its runs with a log-normal-spread generator parameterised by phi
(phi = 0.5 there); phi = 1.0 widens the exponent spread, which is where the
accurate (positional) bound of Part I section 2 matters.

Recipe (fixed so that every consumer sees identical bits): one NumPy PCG64
generator per matrix, ``default_rng(seed)``; draw all U values first, then all
N values, each as a flat vector of rows*cols entries; fill the matrix in
column-major order (flat index k -> row k % rows, column k // rows).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def generate(rows: int, cols: int, phi: float, seed: int) -> np.ndarray:
    """Return a ``rows x cols`` float64 matrix in Fortran (column-major) order."""
    rng = np.random.default_rng(seed)
    n = rows * cols
    u = rng.random(n)
    g = rng.standard_normal(n)
    vals = (u - 0.5) * np.exp(phi * g)
    return np.asfortranarray(vals.reshape((rows, cols), order="F"))


@dataclass(frozen=True)
class Workload:
    """One square FP64 GEMM workload: C = A B with A, B n x n column-major."""

    name: str
    n: int
    mode: str  # "fast" or "accu"
    s: int     # number of moduli
    phi: float
    seed_a: int
    seed_b: int

    def inputs(self):
        a = generate(self.n, self.n, self.phi, self.seed_a)
        b = generate(self.n, self.n, self.phi, self.seed_b)
        return a, b


# The five square workloads used by the parity tests and the benchmark.
WORKLOADS = {
    "n256_fast_s8": Workload("n256_fast_s8", 256, "fast", 8, 0.5, 123456, 123457),
    "n2048_fast_s14": Workload("n2048_fast_s14", 2048, "fast", 14, 0.5, 1, 2),
    "n8192_fast_s14": Workload("n8192_fast_s14", 8192, "fast", 14, 0.5, 1, 2),
    "n8192_accu_s14": Workload("n8192_accu_s14", 8192, "accu", 14, 1.0, 3, 4),
    "n16384_fast_s18": Workload("n16384_fast_s18", 16384, "fast", 18, 1.0, 5, 6),
    "n16384_accu_s18": Workload("n16384_accu_s18", 16384, "accu", 18, 1.0, 5, 6),
}
