// oz2_gemm.hip -- the s main INT8 x INT8 -> INT32 GEMMs P_t = A_t B_t on CDNA4 i8 MFMA,
// one batched launch (grid z = modulus index t), with the output reduction
// R_t = P_t mod m_t fused into the epilogue ("Profiling Ozaki II: The Cost Behind Fast
// INT8 GEMMs", Part I section 1: yellow GEMMs and blue output reduction), and the accu
// bound product whose epilogue keeps only row / column maxima (same page, section 2).
//
// Exactness: |A_t|, |B_t| <= 128, so every product is at most 2^14 and every partial sum
// of a length-q dot product stays below q 2^14 < 2^31 for q < 2^17, in any order
// ("Ozaki II supplement", section 1.3).  Operand planes are int8 with the inner dimension
// contiguous (and identically K-permuted for both operands), rows padded to 256 and the
// inner dimension to 256 with zeros, so the kernel needs no bounds checks in the K loop.
#include "oz2_common.hpp"
#include "oz2_internal.hpp"

namespace oz2 {

typedef int v4i __attribute__((ext_vector_type(4)));

__constant__ int kModsDev[kMaxS] = {modulus(0),  modulus(1),  modulus(2),  modulus(3),  modulus(4),
                                    modulus(5),  modulus(6),  modulus(7),  modulus(8),  modulus(9),
                                    modulus(10), modulus(11), modulus(12), modulus(13), modulus(14),
                                    modulus(15), modulus(16), modulus(17), modulus(18), modulus(19)};

// Tile: 128 x 128 outputs per workgroup, K step 64 bytes; 4 waves in a 2 x 2 grid, each
// 64 x 64 = 4 x 4 blocks of v_mfma_i32_16x16x64_i8.  LDS rows are padded to 80 bytes so
// the 16-byte fragment reads of 16 consecutive rows hit distinct banks.
constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kBK = 64;
constexpr int kLdsPitch = kBK + 16;

// P mod m in [0, m) for |P| < 2^31 and 2 <= m <= 256.
__device__ __forceinline__ uint32_t mod_nonneg(int P, int m, double invm) {
  if (m == 256) return static_cast<uint32_t>(P) & 0xFFu;
  const int qt = static_cast<int>(floor(static_cast<double>(P) * invm));
  int rr = P - qt * m;  // off by at most one multiple of m
  rr += rr < 0 ? m : 0;
  rr -= rr >= m ? m : 0;
  return static_cast<uint32_t>(rr);
}

enum { kEpiMod = 0, kEpiRawMod = 1, kEpiBound = 2 };

template <int EPI>
__global__ __launch_bounds__(256) void gemm_i8_kernel(const int8_t* __restrict__ at, const int8_t* __restrict__ bt,
                                                      long a_plane, long b_plane, int K, uint8_t* __restrict__ res,
                                                      long r_plane, int ldr, int32_t* __restrict__ p_dump, int p,
                                                      int r, int* __restrict__ rho, int* __restrict__ gamma,
                                                      int tiles_m) {
  __shared__ __attribute__((aligned(16))) int8_t sa[kBM * kLdsPitch];
  __shared__ __attribute__((aligned(16))) int8_t sb[kBN * kLdsPitch];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int t = blockIdx.z;
  const int tile_i = static_cast<int>(blockIdx.x % static_cast<unsigned>(tiles_m));
  const int tile_j = static_cast<int>(blockIdx.x / static_cast<unsigned>(tiles_m));
  const int i0 = tile_i * kBM;
  const int j0 = tile_j * kBN;
  const int8_t* ag = at + t * a_plane + static_cast<long>(i0) * K;
  const int8_t* bg = bt + t * b_plane + static_cast<long>(j0) * K;

  v4i acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = v4i{0, 0, 0, 0};

  for (int k0 = 0; k0 < K; k0 += kBK) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = tid + 256 * h;
      const int row = c >> 2;
      const int col = (c & 3) * 16;
      const uint4 va = *reinterpret_cast<const uint4*>(ag + static_cast<long>(row) * K + k0 + col);
      const uint4 vb = *reinterpret_cast<const uint4*>(bg + static_cast<long>(row) * K + k0 + col);
      *reinterpret_cast<uint4*>(sa + row * kLdsPitch + col) = va;
      *reinterpret_cast<uint4*>(sb + row * kLdsPitch + col) = vb;
    }
    __syncthreads();
    v4i fa[4], fb[4];
    const int kofs = (lane >> 4) * 16;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
      fa[mi] = *reinterpret_cast<const v4i*>(sa + (wm * 64 + mi * 16 + (lane & 15)) * kLdsPitch + kofs);
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
      fb[ni] = *reinterpret_cast<const v4i*>(sb + (wn * 64 + ni * 16 + (lane & 15)) * kLdsPitch + kofs);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
    __syncthreads();
  }

  // acc[mi][ni][v] holds P_t[i][j] with
  //   i = i0 + 64 wm + 16 mi + 4 (lane / 16) + v,   j = j0 + 64 wn + 16 ni + lane % 16.
  const int ib = i0 + wm * 64 + 4 * (lane >> 4);
  const int jb = j0 + wn * 64 + (lane & 15);
  if constexpr (EPI == kEpiBound) {
    // rows: max over this wave's 64 columns, then over the 16 lanes sharing lane / 16
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        int mx = max(max(acc[mi][0][v], acc[mi][1][v]), max(acc[mi][2][v], acc[mi][3][v]));
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) mx = max(mx, __shfl_xor(mx, off, kWave));
        const int i = ib + mi * 16 + v;
        if ((lane & 15) == 0 && i < p) atomicMax(rho + i, mx);
      }
    }
    // columns: max over this wave's 64 rows
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      int mx = 0;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        mx = max(mx, max(max(acc[mi][ni][0], acc[mi][ni][1]), max(acc[mi][ni][2], acc[mi][ni][3])));
      mx = max(mx, __shfl_xor(mx, 16, kWave));
      mx = max(mx, __shfl_xor(mx, 32, kWave));
      const int j = jb + ni * 16;
      if (lane < 16 && j < r) atomicMax(gamma + j, mx);
    }
  } else {
    const int m = kModsDev[t];
    const double invm = 1.0 / static_cast<double>(m);
    uint8_t* rt = res + t * r_plane;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int i = ib + mi * 16;
        const int j = jb + ni * 16;
        const v4i a4 = acc[mi][ni];
        const uint32_t packed = mod_nonneg(a4[0], m, invm) | (mod_nonneg(a4[1], m, invm) << 8) |
                                (mod_nonneg(a4[2], m, invm) << 16) | (mod_nonneg(a4[3], m, invm) << 24);
        *reinterpret_cast<uint32_t*>(rt + static_cast<long>(j) * ldr + i) = packed;
        if constexpr (EPI == kEpiRawMod) {
          if (j < r) {
            int32_t* dst = p_dump + (static_cast<long>(t) * r + j) * p;
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (i + v < p) dst[i + v] = a4[v];
          }
        }
      }
    }
  }
}

hipError_t launch_gemm(const Work& w, int epi, const DumpPtrs& dump, hipStream_t st) {
  const int planes = epi == kEpiBound ? 1 : w.s;
  const int tiles_m = w.p_pad / kBM;
  dim3 grid(static_cast<unsigned>(tiles_m) * static_cast<unsigned>(w.r_pad / kBN), 1, planes);
  const long a_plane = static_cast<long>(w.p_pad) * w.q_pad;
  const long b_plane = static_cast<long>(w.r_pad) * w.q_pad;
  const long r_plane = static_cast<long>(w.r_pad) * w.p_pad;
  const int8_t* a = epi == kEpiBound ? w.abar : w.at;
  const int8_t* b = epi == kEpiBound ? w.bbar : w.bt;
  switch (epi) {
    case kEpiMod:
      hipLaunchKernelGGL(gemm_i8_kernel<kEpiMod>, grid, dim3(256), 0, st, a, b, a_plane, b_plane, w.q_pad, w.res,
                         r_plane, w.p_pad, nullptr, w.p, w.r, nullptr, nullptr, tiles_m);
      break;
    case kEpiRawMod:
      hipLaunchKernelGGL(gemm_i8_kernel<kEpiRawMod>, grid, dim3(256), 0, st, a, b, a_plane, b_plane, w.q_pad,
                         w.res, r_plane, w.p_pad, dump.pt, w.p, w.r, nullptr, nullptr, tiles_m);
      break;
    case kEpiBound:
      hipLaunchKernelGGL(gemm_i8_kernel<kEpiBound>, grid, dim3(256), 0, st, a, b, a_plane, b_plane, w.q_pad,
                         nullptr, 0L, w.p_pad, nullptr, w.p, w.r, w.rho, w.gamma, tiles_m);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace oz2
