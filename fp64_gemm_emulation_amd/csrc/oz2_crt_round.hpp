// oz2_crt_round.hpp -- the per-output arithmetic of the reconstruction ("Profiling Ozaki
// II: The Cost Behind Fast INT8 GEMMs", Part I section 1, red stage), callable from device
// and host code:
//   crt_accumulate  acc[k] += R_t W_t[k]  (32-bit limbs of the CRT weights, exact FMAs)
//   crt_reduce      acc -= k M with k the nearest integer to sum_t R_t W_t / M
//   crt_normalize   acc[0..L-2] -> [0, 2^32), carries moved up (the two's-complement words)
//   crt_round       RN(X) 2^scale
// The limb sums X = sum_k acc[k] 2^(32 k) stay exact integers below 2^53 in magnitude.
//
// Rounding without an integer detour.  After normalisation,
//   H_j = floor(X / 2^(32 j)) = H_{j+1} 2^32 + acc[j],   H_{L-1} = acc[L-1].
// If |H_j| < 2^21, H_{j-1} is below 2^53 and exact.  Take the largest level j >= 2 with
// |H_j| >= 2^21: then |X| >= 2^(32 j + 20), so the final unit in the last place is at least
// 2^(32 j - 32) and every rounding boundary (the doubles and the midpoints between them) is
// a multiple of 2^(32 j - 33) = 2^(32 (j - 2) + 31).  Replacing the limbs below level j - 1
// by bit 31 of acc[j-2] plus a sticky 2^30 when anything below that bit is nonzero gives a
// value Xh in the same cell of that grid as X (equal to X exactly when X lies on it), so
// RN(Xh) = RN(X); Xh = (H_j 2^64 + acc[j-1] 2^32 + hat) 2^(32 (j-2)) needs one rounding, in
// one FMA, because acc[j-1] 2^32 + hat has at most 34 significant bits.  If no level
// triggers, |H_1| < 2^53 and RN(X) = RN(H_1 2^32 + acc[0]) is again one FMA.  Levels whose
// H cannot reach 2^21 (kTopExp bounds |H_{L-1}| by 2^kTopExp) are skipped at compile time.
#pragma once
#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>

#include "oz2_params.hpp"

namespace oz2 {

template <int S>
__host__ __device__ inline void crt_accumulate(double (&acc)[CrtTable<S>::L], double rt, int t) {
#pragma unroll
  for (int k = 0; k < CrtTable<S>::L; ++k) acc[k] = fma(rt, kCrt<S>.w[t][k], acc[k]);
}

// k from the two top limb sums (see make_crt for why they suffice), then X = sum - k M.
template <int S>
__host__ __device__ inline void crt_reduce(double (&acc)[CrtTable<S>::L]) {
  constexpr int L = CrtTable<S>::L;
  double kq;
  if constexpr (L >= 2)
    kq = rint(fma(acc[L - 1], kCrt<S>.q1, acc[L - 2] * kCrt<S>.q0));
  else
    kq = rint(acc[0] * kCrt<S>.q1);
#pragma unroll
  for (int k = 0; k < L; ++k) acc[k] = fma(-kq, kCrt<S>.m[k], acc[k]);
}

// 2^e for 0 <= e < 1024, folded at compile time where e is a constant.
__host__ __device__ constexpr double pow2i(int e) {
  double x = 1.0;
  for (int k = 0; k < e; ++k) x *= 2.0;
  return x;
}

// acc[0..L-2] -> [0, 2^32) with the carries moved up; X is unchanged and acc[L-1] becomes
// floor(X / 2^(32 (L-1))).  Exact: power-of-two scalings, floor and integer sums < 2^53.
template <int L>
__host__ __device__ inline void crt_normalize(double (&acc)[L]) {
#pragma unroll
  for (int k = 0; k + 1 < L; ++k) {
    const double cy = floor(acc[k] * 0x1p-32);
    acc[k] = fma(-cy, 0x1p32, acc[k]);
    acc[k + 1] += cy;
  }
}

// RN(X) * 2^scale for normalised limbs (exact scaling unless the result is subnormal).
template <int L, int kTopExp>
__host__ __device__ inline double crt_round(const double (&a)[L], int scale) {
  if constexpr (L == 1) {
    return ldexp(a[0], scale);  // |X| < 2^53: exact
  } else {
    double h[L];
    h[L - 1] = a[L - 1];
#pragma unroll
    for (int j = L - 1; j >= 2; --j) h[j - 1] = fma(h[j], 0x1p32, a[j - 1]);
    double z = fma(h[1], 0x1p32, a[0]);
#pragma unroll
    for (int j = 2; j < L; ++j) {
      if (j == L - 1 && kTopExp < 21) continue;
      const double b = floor(a[j - 2] * 0x1p-31);
      bool sticky = fma(-b, 0x1p31, a[j - 2]) != 0.0;
#pragma unroll
      for (int k = 0; k < j - 2; ++k) sticky = sticky || a[k] != 0.0;
      const double hat = fma(b, 0x1p31, sticky ? 0x1p30 : 0.0);
      const double u = fma(a[j - 1], 0x1p32, hat);
      double zj = fma(h[j], 0x1p64, u);
      if (j > 2) zj *= pow2i(32 * (j - 2));  // exact
      if (fabs(h[j]) >= 0x1p21) z = zj;
    }
    return ldexp(z, scale);
  }
}

}  // namespace oz2
