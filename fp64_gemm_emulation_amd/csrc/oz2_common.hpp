// oz2_common.hpp -- device helpers shared by the Ozaki II kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "oz2_params.hpp"

namespace oz2 {

constexpr int kWave = 64;

// Workspace alignment and padding of the int8 operand planes.  Rows of A_t / B_t are
// padded to kRowPad, the inner dimension to kKPad (a multiple of the 256-long
// K-permutation block used by the residue kernels).
constexpr int kRowPad = 256;
constexpr int kKPad = 256;

// Flags word bits (mirror of OZ2_FLAG_* in the public header).
constexpr unsigned kFlagNonFinite = 1u;

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ __forceinline__ int wave_max_w(int v, int width) {
  for (int off = width / 2; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// E(x): the integer with 2^(E-1) <= |x| < 2^E for finite x != 0 (subnormals included);
// kNoExp for x == 0.
__device__ __forceinline__ int exponent_of(double x) {
  return x == 0.0 ? kNoExp : __builtin_amdgcn_frexp_exp(x);
}

__device__ __forceinline__ bool is_nonfinite(double x) {
  uint64_t bits = static_cast<uint64_t>(__double_as_longlong(x));
  return ((bits >> 52) & 0x7FFu) == 0x7FFu;
}

// ceil(|x| * 2^k) for finite x, exactly, as a double (k may be any integer).
// If E(x) + k <= 0 the scaled value lies in (0, 1] and the ceiling is 1; otherwise the
// scaled value is a normal number >= 1 and ldexp is exact.
__device__ __forceinline__ double ceil_scaled_abs(double x, int ex, int k) {
  if (x == 0.0) return 0.0;
  if (ex + k <= 0) return 1.0;
  return ceil(ldexp(fabs(x), k));
}

// ceil(v / 2^sh) for an exact nonnegative integer v < 2^53 held in a double, sh >= 0.
__device__ __forceinline__ uint64_t ceil_shift(double v, int sh) {
  if (v == 0.0) return 0;
  if (sh >= 60) return 1;
  return static_cast<uint64_t>(ceil(ldexp(v, -sh)));
}

// bitlen(v - 1) = ceil(log2 v) for v >= 1.
__device__ __forceinline__ int clog2_u64(uint64_t v) {
  return v <= 1 ? 0 : 64 - __clzll(static_cast<long long>(v - 1));
}

// Position of element l (0 <= l < kKPad within a 256-block) in the K-permuted operand
// layout: lane L of a 16-lane group owns l = L + 16 k (k = 0..15) and stores them as 16
// consecutive bytes at 16 L + k.  Any permutation of the inner dimension applied to
// both operands leaves every P_t unchanged.
__host__ __device__ __forceinline__ int kperm_pos(int l) { return ((l & 15) << 4) | (l >> 4); }
__host__ __device__ __forceinline__ int kperm_inv(int pos) { return ((pos & 15) << 4) | (pos >> 4); }

}  // namespace oz2
