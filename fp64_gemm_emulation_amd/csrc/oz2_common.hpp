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

// Load of one FP64 input element; NT: with the non-temporal hint, for operands too large
// for the memory-side cache to keep between the statistics and residue passes (streamed
// reads then do not evict lines that would be reused).
template <bool NT>
__device__ __forceinline__ double load_f64(const double* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

__device__ __forceinline__ bool is_nonfinite(double x) {
  uint64_t bits = static_cast<uint64_t>(__double_as_longlong(x));
  return ((bits >> 52) & 0x7FFu) == 0x7FFu;
}

// ceil(|x| * 2^k) for finite x, exactly, as a double (k may be any integer), without
// branches: if the scaled value is at least 1 it is a normal number and ldexp is exact;
// if it lies in (0, 1) its ceiling is 1, which the max supplies even where ldexp rounds
// it into the subnormal range or to 0; x = 0 gives 0.
__device__ __forceinline__ double ceil_scaled_abs(double x, int k) {
  return fmax(ceil(ldexp(fabs(x), k)), x != 0.0 ? 1.0 : 0.0);
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

// Reductions over G consecutive lanes (a power of two, at most 64); every lane of the group
// receives the result.
template <int G>
__device__ __forceinline__ int group_max(int v) {
#pragma unroll
  for (int off = G / 2; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off, kWave));
  return v;
}

template <int G>
__device__ __forceinline__ uint64_t group_sum_u64(uint64_t v) {
  uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
#pragma unroll
  for (int off = G / 2; off > 0; off >>= 1) {
    const uint32_t lo2 = static_cast<uint32_t>(__shfl_xor(static_cast<int>(lo), off, kWave));
    const uint32_t hi2 = static_cast<uint32_t>(__shfl_xor(static_cast<int>(hi), off, kWave));
    const uint32_t sum = lo + lo2;
    hi = hi + hi2 + (sum < lo ? 1u : 0u);
    lo = sum;
  }
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Fast-mode exponent of one line ("Profiling Ozaki II: The Cost Behind Fast INT8 GEMMs",
// Part I section 2) from its statistics partials: block c has max-abs exponent e_c
// (kNoExp when all zero) and the exact integer sum of squares S_c at that exponent.  With
// e = max_c e_c (not kNoExp) and S = sum_c ceil(S_c / 4^(e - e_c)) the exponent is
// floor((tau - ceil(log2 S)) / 2) + kFBits - e; an all-zero line gets 0.  S is exact in
// uint64 (at most q 2^40 < 2^59), so the order of the sums does not matter.
// One block's term ceil(S_c / 4^(e - e_c)), 0 for an all-zero block, without branches
// (ceil_shift's for a shift clamped to 60: 0 < S_c < 2^53 then leaves a value in (0, 1)
// whose ceiling is 1, the value of every larger shift).
__device__ __forceinline__ uint64_t partial_at_line_scale(int e, int ec, double sc) {
  const double v = ec == kNoExp ? 0.0 : sc;
  return static_cast<uint64_t>(ceil(ldexp(v, -2 * min(e - ec, 30))));
}

__device__ __forceinline__ int fast_exponent(int e, uint64_t S, int tau) {
  return ((tau - clog2_u64(S)) >> 1) + kFBits - e;
}

// The same with G consecutive lanes sharing the line, lane g of the group reading blocks
// g, g + G, ... < nch of pe / ps; every lane of the group returns the exponent.
template <int G>
__device__ __forceinline__ int fast_line_exponent(const int* pe, const double* ps, int nch, int g, int tau) {
  int e = kNoExp;
  for (int c = g; c < nch; c += G) e = max(e, pe[c]);
  e = group_max<G>(e);
  if (e == kNoExp) return 0;  // uniform over the group
  uint64_t S = 0;
  for (int c = g; c < nch; c += G) S += partial_at_line_scale(e, pe[c], ps[c]);
  return fast_exponent(e, group_sum_u64<G>(S), tau);
}

// Operand planes (A_t, B_t and the accu quantized operands) are stored in the order the
// GEMM consumes them, tile-contiguous:
//   [256-row block][64-byte stage of the inner dimension][256 rows x 64 bytes],
// and inside a row's 64-byte segment the four 16-byte chunks are XOR-swizzled by
// operand_swizzle(row % 16).  One GEMM stage tile of one operand is then a contiguous
// 16 KiB block that is copied into LDS unchanged, and 16-byte fragment reads of 16
// consecutive rows at one logical chunk hit 16 distinct LDS bank groups.
//
// Within each 256-long block of the inner dimension the producer thread for "slot" L
// (0..15) owns the elements l = L + 16 k (k = 0..15) and stores them as one 16-byte chunk,
// byte k; slot L is logical chunk L % 4 of stage L / 4 of the block.  The same order is
// used for both operands, and any common permutation of the inner dimension leaves every
// P_t unchanged.
constexpr int kStageK = 64;                    // inner-dimension bytes per GEMM stage
constexpr int kStageTile = kRowPad * kStageK;  // bytes of one operand stage tile (16 KiB)

__host__ __device__ __forceinline__ int operand_swizzle(int r16) { return ((r16 >> 1) ^ (r16 >> 3)) & 3; }

// Byte offset, within one operand plane of q_pad-long rows, of the 16-byte chunk of slot
// L (0..15) of 256-block blk of row `row`.
__host__ __device__ __forceinline__ long operand_chunk_offset(int row, int blk, int slot, int q_pad) {
  const int rr = row & (kRowPad - 1);
  const long tile = static_cast<long>(row / kRowPad) * (q_pad / kStageK) + blk * (kKPad / kStageK) + (slot >> 2);
  return tile * kStageTile + rr * kStageK + 16 * ((slot & 3) ^ operand_swizzle(rr & 15));
}

// Thread mappings of the kernels that produce operand planes, chosen so that each 16-byte
// chunk store instruction of a wave writes whole cache lines of the layout above.
struct ChunkOwner {
  int row;   // operand row (a row of A, or a column of B)
  int blk;   // 256-block of the inner dimension
  int slot;  // chunk slot 0..15 within the block
};

// Rows of column-major A: workgroup = 64 rows x one 64-byte stage, grid (p_pad / 64,
// q_pad / 64).  Lane l of wave w owns row 16 w + l / 4 and physical chunk l % 4 of that
// row's stage segment: a store instruction writes 1 KiB contiguous (16 rows x 64 bytes),
// and a load instruction for one k reads 4 columns x 16 consecutive rows.
// (bx, by): the workgroup's coordinates in that grid.
__device__ __forceinline__ ChunkOwner owner_rows_of_a(int bx, int by) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int stage = by;
  const int row = bx * 64 + wave * 16 + (lane >> 2);
  return ChunkOwner{row, stage >> 2, 4 * (stage & 3) + ((lane & 3) ^ operand_swizzle(row & 15))};
}

// Columns of column-major B: workgroup = 16 columns x one 256-block, grid (r_pad / 16,
// q_pad / 256).  Lane l of wave w owns column 4 w + l / 16 and slot l % 16: a load
// instruction for one k reads 4 runs of 128 contiguous bytes, a store instruction writes
// 4 runs of 256 contiguous bytes (4 rows x 64 bytes in each of the 4 stage tiles).
// (bx, by): the workgroup's coordinates in that grid.
__device__ __forceinline__ ChunkOwner owner_cols_of_b(int bx, int by) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  return ChunkOwner{bx * 16 + wave * 4 + (lane >> 4), by, lane & 15};
}

// Byte offset of inner-dimension element l of row `row` (the inverse map, for validation).
__host__ __device__ __forceinline__ long operand_elem_offset(int row, int l, int q_pad) {
  const int w = l & (kKPad - 1);
  return operand_chunk_offset(row, l / kKPad, w & 15, q_pad) + (w >> 4);
}

}  // namespace oz2
