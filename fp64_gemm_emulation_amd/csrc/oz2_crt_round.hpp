// oz2_crt_round.hpp -- the per-output arithmetic of the reconstruction ("Profiling Ozaki
// II: The Cost Behind Fast INT8 GEMMs", Part I section 1, red stage), callable from device
// and host code:
//   crt_accumulate  acc[k] += R_t W_t[k]  (kW-bit limbs of the CRT weights, exact FMAs)
//   crt_reduce      acc -= k M with k the nearest integer to sum_t R_t W_t / M
//   crt_normalize   acc[0..L-2] -> [0, 2^kW), carries moved up
//   crt_round       RN(X 2^scale), rounded once (also below the normal range)
//   crt_words       the 32-bit two's-complement words of X (validation)
// The limb sums X = sum_k acc[k] 2^(kW k) stay exact integers below 2^53 in magnitude.
//
// Rounding without an integer detour.  After normalisation,
//   H_j = floor(X / 2^(kW j)) = H_{j+1} 2^kW + acc[j],   H_{L-1} = acc[L-1].
// If |H_j| < 2^(52 - kW), H_{j-1} is below 2^53 and exact.  Take the largest level j >= 2
// with |H_j| >= 2^(52 - kW): then |X| >= 2^(kW (j - 1) + 51), so the final unit in the last
// place is at least 2^(kW (j - 1) - 1) and every rounding boundary (the doubles and the
// midpoints between them) is a multiple of 2^(kW (j - 2) + kW - 2).  Replacing the limbs below
// level j - 1 by the top two bits of acc[j-2] plus a sticky 2^(kW - 3) when anything below
// them is nonzero gives a value Xh in the same cell of that grid as X (equal to X exactly
// when X lies on it), so RN(Xh) = RN(X); Xh = (H_j 2^(2 kW) + acc[j-1] 2^kW + hat)
// 2^(kW (j-2)) needs one rounding, in one FMA, because acc[j-1] 2^kW + hat has at most
// kW + 3 significant bits.  If no level triggers, |H_1| < 2^53 and
// RN(X) = RN(H_1 2^kW + acc[0]) is again one FMA.  Levels whose H cannot reach the
// threshold (kTopExp bounds |H_{L-1}| by 2^kTopExp) are skipped at compile time.
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

// acc[0..L-2] -> [0, 2^W) with the carries moved up; X is unchanged and acc[L-1] becomes
// floor(X / 2^(W (L-1))).  Exact: power-of-two scalings, floor and integer sums < 2^53.
template <int L, int W>
__host__ __device__ inline void crt_normalize(double (&acc)[L]) {
  constexpr double kUp = pow2i(W), kDown = 1.0 / pow2i(W);
#pragma unroll
  for (int k = 0; k + 1 < L; ++k) {
    const double cy = floor(acc[k] * kDown);
    acc[k] = fma(-cy, kUp, acc[k]);
    acc[k + 1] += cy;
  }
}

// RN(X) to 53 bits for normalised limbs (X itself when |X| < 2^53).
template <int L, int W, int kTopExp>
__host__ __device__ inline double crt_round53(const double (&a)[L]) {
  if constexpr (L == 1) {
    return a[0];  // |X| < 2^53: exact
  } else {
    constexpr double kUp = pow2i(W), kUp2 = pow2i(2 * W);
    constexpr double kThr = pow2i(52 - W);
    constexpr double kTop2 = 1.0 / pow2i(W - 2), kBit = pow2i(W - 2), kSticky = pow2i(W - 3);
    double h[L];
    h[L - 1] = a[L - 1];
#pragma unroll
    for (int j = L - 1; j >= 2; --j) h[j - 1] = fma(h[j], kUp, a[j - 1]);
    double z = fma(h[1], kUp, a[0]);
#pragma unroll
    for (int j = 2; j < L; ++j) {
      if (j == L - 1 && kTopExp < 52 - W) continue;
      const double b = floor(a[j - 2] * kTop2);  // top two bits of the limb below
      bool sticky = fma(-b, kBit, a[j - 2]) != 0.0;
#pragma unroll
      for (int k = 0; k < j - 2; ++k) sticky = sticky || a[k] != 0.0;
      const double hat = fma(b, kBit, sticky ? kSticky : 0.0);
      const double u = fma(a[j - 1], kUp, hat);
      double zj = fma(h[j], kUp2, u);
      if (j > 2) zj *= pow2i(W * (j - 2));  // exact
      if (fabs(h[j]) >= kThr) z = zj;
    }
    return z;
  }
}

// The five 32-bit two's-complement words (little-endian) of X = sum_k a[k] 2^(W k) for
// normalised limbs (a[0..L-2] in [0, 2^W), |a[L-1]| < 2^40): the limbs are shifted into a
// 192-bit integer from the top down.
template <int L, int W>
__host__ __device__ inline void crt_words(const double (&a)[L], uint32_t (&out)[5]) {
  const double th = floor(a[L - 1] * 0x1p-32);
  const uint64_t top = (static_cast<uint64_t>(static_cast<int64_t>(th)) << 32) |
                       static_cast<uint32_t>(fma(-th, 0x1p32, a[L - 1]));
  uint64_t x[3] = {top, (top >> 63) != 0 ? ~0ull : 0ull, (top >> 63) != 0 ? ~0ull : 0ull};
#pragma unroll
  for (int k = L - 2; k >= 0; --k) {
    x[2] = (x[2] << W) | (x[1] >> (64 - W));
    x[1] = (x[1] << W) | (x[0] >> (64 - W));
    x[0] = x[0] << W;
    const double hi = floor(a[k] * 0x1p-32);
    const uint64_t v = (static_cast<uint64_t>(hi) << 32) | static_cast<uint32_t>(fma(-hi, 0x1p32, a[k]));
    const uint64_t s0 = x[0] + v;
    const uint64_t c0 = s0 < v ? 1ull : 0ull;
    x[0] = s0;
    const uint64_t s1 = x[1] + c0;
    x[2] += s1 < c0 ? 1ull : 0ull;
    x[1] = s1;
  }
#pragma unroll
  for (int k = 0; k < 5; ++k) out[k] = static_cast<uint32_t>(x[k / 2] >> (32 * (k % 2)));
}

// RN(X 2^scale) for a result below the normal range, rounded once.  With g = -1074 - scale > 0
// the result is the multiple of 2^-1074 nearest to X 2^scale (ties to an even multiple):
// round(|X| / 2^g) 2^-1074 with the sign of X, taken from X's exact 160-bit two's-complement
// form.  Only results below 2^-1022 come here (rare), where |X| < 2^(52 + g).
template <int L, int W>
__host__ __device__ inline double crt_round_subnormal(const double (&a)[L], int scale) {
  uint32_t w[5];
  crt_words<L, W>(a, w);
  const bool neg = (w[4] >> 31) != 0;
  uint64_t m[4] = {w[0] | (static_cast<uint64_t>(w[1]) << 32), w[2] | (static_cast<uint64_t>(w[3]) << 32), w[4], 0};
  if (neg) {  // magnitude of the 160-bit two's-complement value
    m[0] = ~m[0] + 1;
    m[1] = ~m[1] + (m[0] == 0 ? 1 : 0);
    m[2] = (~m[2] + (m[0] == 0 && m[1] == 0 ? 1 : 0)) & 0xFFFFFFFFull;
  }
  const int g = -1074 - scale;  // > 0: the bit position of the result's unit
  uint64_t y = 0;
  bool round_bit = false, sticky = false;
  if (g <= 160) {  // |X| < 2^160: beyond that the result is below half a unit, hence 0
    const int wi = g >> 6, bo = g & 63;  // y = |X| >> g (below 2^53)
    y = (m[wi] >> bo) | (bo != 0 && wi < 3 ? m[wi + 1] << (64 - bo) : 0);
    const int wr = (g - 1) >> 6, br = (g - 1) & 63;  // the bit below the unit, and all below it
    round_bit = ((m[wr] >> br) & 1u) != 0;
    sticky = (m[wr] & ((uint64_t{1} << br) - 1)) != 0;
    for (int k = 0; k < wr; ++k) sticky = sticky || m[k] != 0;
  }
  if (round_bit && (sticky || (y & 1u) != 0)) ++y;
  const double r = ldexp(static_cast<double>(y), -1074);  // exact: y <= 2^53
  return neg ? -r : r;
}

// RN(X 2^scale) for normalised limbs, rounded once: X rounded to 53 bits and scaled exactly
// when the result is normal; a result below 2^-1022 with scale < -1074 (where the
// subnormal grid is coarser than X's integer grid) takes crt_round_subnormal.  With
// scale >= -1074 a result below 2^-1022 has |X| < 2^52, so RN53(X) = X and ldexp is exact.
template <int L, int W, int kTopExp>
__host__ __device__ inline double crt_round(const double (&a)[L], int scale) {
  const double z = crt_round53<L, W, kTopExp>(a);
  if (scale < -1074 && z != 0.0) {
    // z is an integer-valued double, |z| >= 1: its unbiased exponent is floor(log2 |z|)
    const int ez = static_cast<int>((__builtin_bit_cast(uint64_t, z) >> 52) & 0x7FF) - 1023;
    if (ez + scale < -1022) return crt_round_subnormal<L, W>(a, scale);
  }
  return ldexp(z, scale);
}

}  // namespace oz2
