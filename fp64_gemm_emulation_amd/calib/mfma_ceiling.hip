// mfma_ceiling.hip -- measurement aid, not part of the GEMM emulation: the sustained
// rate of v_mfma_i32_16x16x64_i8 issued from registers only, in the form the large-grid
// mod GEMM uses it (eight waves per workgroup, two per SIMD, 16 independent 16x16
// accumulators per wave).  The operands are random bytes that change every round (byte
// rotations, a handful of VALU instructions per 16 MFMAs), as the operands of the modular
// GEMMs do; with constant or zero operands the matrix cores draw less power and run
// faster, so those would overstate what a GEMM on residues can reach.  Used by bench.py
// for the power-limited MFMA ceiling.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4i rotate_bytes(v4i x) {
  return v4i{static_cast<int>(__builtin_amdgcn_alignbyte(x[1], x[0], 1)),
             static_cast<int>(__builtin_amdgcn_alignbyte(x[2], x[1], 1)),
             static_cast<int>(__builtin_amdgcn_alignbyte(x[3], x[2], 1)),
             static_cast<int>(__builtin_amdgcn_alignbyte(x[0], x[3], 1))};
}

__global__ __launch_bounds__(512, 1) void mfma_i8_ceiling_kernel(const v4i* __restrict__ src, int rounds,
                                                                   int* __restrict__ out) {
  const int tid = threadIdx.x;
  v4i f[8];
#pragma unroll
  for (int g = 0; g < 8; ++g) f[g] = src[(blockIdx.x * 8 + g) * 512 + tid];
  v4i acc[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) acc[k] = v4i{};
  for (int it = 0; it < rounds; ++it) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        acc[mb * 4 + nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f[mb], f[4 + nb], acc[mb * 4 + nb], 0, 0, 0);
#pragma unroll
    for (int g = 0; g < 8; ++g) f[g] = rotate_bytes(f[g]);
  }
  int x = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k)
#pragma unroll
    for (int v = 0; v < 4; ++v) x ^= acc[k][v];
  out[blockIdx.x * 512 + tid] = x;
}

// The same instruction in the exact shape of the large-grid mod GEMM: one workgroup of 8
// waves per 256 x 256 output tile (the GEMM's grid), each wave 8 x 4 blocks of 16 x 16 (32
// accumulators) issued in the GEMM's order (block rows in turn, every other row's columns
// reversed), and 12 fragments (8 of A, 4 of B) that all change after every 32 MFMAs, as the
// GEMM reads new fragments for every 64-deep stage.  As in the GEMM, the waves of one row
// half (wave & 1) hold the same A fragments and the waves of one column quarter (wave >> 1)
// the same B fragments, so the two waves that share a SIMD (w, w + 4) see the same A.
// 128 KiB of LDS is held (never touched) so that one workgroup runs per CU, as for the GEMM.
// What it leaves out is the GEMM's memory traffic (copies into LDS, fragment reads) and its
// epilogue, so the GEMM's rate over this one's is the cost of those at equal MFMA work.
__global__ __launch_bounds__(512, 1) void mfma_i8_gemm_shape_kernel(const v4i* __restrict__ src, int stages,
                                                                      int* __restrict__ out) {
  __shared__ int lds_hold[128 * 1024 / 4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  v4i f[12];
#pragma unroll
  for (int g = 0; g < 12; ++g)
    f[g] = src[((blockIdx.x & 1023) * 12 + g) * 512 + (g < 8 ? wm : 2 + wn) * 64 + lane];
  v4i acc[8][4];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = v4i{};
  for (int kt = 0; kt < stages; ++kt) {
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const int mb = u / 4, nb = (mb & 1) ? 3 - u % 4 : u % 4;
      acc[mb][nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f[mb], f[8 + nb], acc[mb][nb], 0, 0, 0);
    }
#pragma unroll
    for (int g = 0; g < 12; ++g) f[g] = rotate_bytes(f[g]);
  }
  int x = 0;
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int v = 0; v < 4; ++v) x ^= acc[mb][nb][v];
  if (x == 0x7fffffff) lds_hold[tid] = x;  // keeps the LDS allocation; practically never taken
  out[blockIdx.x * 512 + tid] = x;
}

// src: blocks * 8 * 512 16-byte random words (device); out: blocks * 512 ints (device).
// One round is 16 MFMAs of 16 x 16 x 64 per wave, 8 waves: 8 * 16 * 16384 = 2^21
// multiply-adds per block.
extern "C" int oz2calib_mfma_i8(const void* src, int blocks, int rounds, int* out, void* stream) {
  if (!src || !out || blocks <= 0 || rounds <= 0) return 1;
  hipLaunchKernelGGL(mfma_i8_ceiling_kernel, dim3(blocks), dim3(512), 0, static_cast<hipStream_t>(stream),
                     static_cast<const v4i*>(src), rounds, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// src: 1024 * 12 * 512 16-byte random words (device); out: tiles * 512 ints (device).  One
// workgroup per tile, each 8 waves x 32 MFMAs of 16 x 16 x 64 per stage: stages * 2^22
// multiply-adds per tile.
extern "C" int oz2calib_mfma_i8_gemm_shape(const void* src, int tiles, int stages, int* out, void* stream) {
  if (!src || !out || tiles <= 0 || stages <= 0) return 1;
  hipLaunchKernelGGL(mfma_i8_gemm_shape_kernel, dim3(tiles), dim3(512), 0, static_cast<hipStream_t>(stream),
                     static_cast<const v4i*>(src), stages, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
