// oz2_crt.hip -- reconstruction: X = CRT_M(R_1..R_s) in [-M/2, M/2) and C = D^-1 X E^-1
// ("Profiling Ozaki II: The Cost Behind Fast INT8 GEMMs", Part I section 1, red stage).
//
// X is computed exactly: with W_t = (M/m_t) ((M/m_t)^-1 mod m_t),
//   X = sum_t R_t W_t - k M,   k = round(sum_t R_t W_t / M).
// W_t and M are split into limbs of at most 40 bits held in doubles, so every limb sum is
// an exact FP64 integer FMA chain (each partial sum < 20 * 2^8 * 2^40 < 2^53).  k comes from the two
// top limb sums (the lower limbs cannot move the quotient across a half-integer: the
// scalings keep |X| <= 2^tau).  The lower limbs are carried into [0, 2^kW) with floor and
// the result rounded to FP64 with one
// round-to-nearest-even and scaled by 2^-(d_i + b_j) with ldexp (exact unless the result is
// subnormal); oz2_crt_round.hpp holds that step and why one FMA rounding is enough.  The
// stored value is alpha Chat when beta = 0 (C is not read) and fma(alpha, Chat, RN(beta C))
// otherwise, so alpha = 1, beta = 0 stores Chat itself.
#include "oz2_common.hpp"
#include "oz2_internal.hpp"
#include "oz2_crt_round.hpp"

namespace oz2 {

// Thread: kRowsPerThread consecutive rows i0.. of one column j; it reads kRowsPerThread
// bytes of each residue plane with one load (so each plane read of a wave covers
// 64 kRowsPerThread contiguous bytes) and writes its outputs with 16-byte stores.  (8 or
// 16 rows per thread measured no faster at n = 8192: the stage is bound by the HBM
// traffic of the s residue planes and of C.)  The residue planes are read once, with the
// non-temporal hint: 6% faster at n = 8192, s = 14 (the plain loads allocate lines that
// are never reused in the memory-side cache).  Non-temporal stores of C were slower.
constexpr int kRowsPerThread = 4;
constexpr int kCrtWords = kRowsPerThread / 4;  // 32-bit words of residues per plane and thread

template <int S, bool DUMPX>
__global__ __launch_bounds__(256) void crt_kernel(const uint8_t* __restrict__ res, long r_plane, int ldr, int p,
                                                  int r, int groups, const int* __restrict__ d,
                                                  const int* __restrict__ b, double* __restrict__ C, long ldc,
                                                  double alpha, double beta, uint32_t* __restrict__ x_dump) {
  constexpr int L = CrtTable<S>::L;
  // grid: x = column j, y = blocks of 256 row groups
  const int j = blockIdx.x;
  const int ig = blockIdx.y * blockDim.x + threadIdx.x;
  if (ig >= groups) return;
  const int i0 = ig * kRowsPerThread;
  // rows up to i0 + kRowsPerThread - 1 < p_pad: the residue planes hold them
  uint32_t rw[S][kCrtWords];
  const uint8_t* src = res + static_cast<long>(j) * ldr + i0;
#pragma unroll
  for (int t = 0; t < S; ++t) {
    if constexpr (kCrtWords == 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(src + t * r_plane);
      rw[t][0] = v.x; rw[t][1] = v.y; rw[t][2] = v.z; rw[t][3] = v.w;
    } else if constexpr (kCrtWords == 2) {
      const uint2 v = *reinterpret_cast<const uint2*>(src + t * r_plane);
      rw[t][0] = v.x; rw[t][1] = v.y;
    } else {
      rw[t][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(src + t * r_plane));
    }
  }
  // plane by plane, so each limb constant is loaded once for the thread's outputs
  double acc[kRowsPerThread][L];
#pragma unroll
  for (int v = 0; v < kRowsPerThread; ++v)
#pragma unroll
    for (int k = 0; k < L; ++k) acc[v][k] = 0.0;
#pragma unroll
  for (int t = 0; t < S; ++t) {
    double rt[kRowsPerThread];
#pragma unroll
    for (int v = 0; v < kRowsPerThread; ++v) rt[v] = static_cast<double>((rw[t][v >> 2] >> (8 * (v & 3))) & 0xFFu);
#pragma unroll
    for (int v = 0; v < kRowsPerThread; ++v) crt_accumulate<S>(acc[v], rt[v], t);
  }
  const int bj = b[j];
  double out[kRowsPerThread];
  int scale[kRowsPerThread];
  int smin = 0;
#pragma unroll
  for (int v = 0; v < kRowsPerThread; ++v) {
    const int i = min(i0 + v, p - 1);  // rows past p (last group only) are computed, not stored
    crt_reduce<S>(acc[v]);
    crt_normalize<L, CrtTable<S>::kW>(acc[v]);
    if (DUMPX && i0 + v < p) {
      uint32_t wd[5];
      crt_words<L, CrtTable<S>::kW>(acc[v], wd);
      uint32_t* xd = x_dump + (static_cast<long>(j) * p + i) * 5;
#pragma unroll
      for (int k = 0; k < 5; ++k) xd[k] = wd[k];
    }
    scale[v] = -(d[i] + bj);
    smin = min(smin, scale[v]);
    out[v] = ldexp(crt_round53<L, CrtTable<S>::kW, CrtTable<S>::kTopExp>(acc[v]), scale[v]);
  }
  // ldexp(RN53(X), scale) is RN(X 2^scale) unless the result falls below 2^-1022 with
  // scale < -1074 (crt_round); only threads with such a scale take that path, so the
  // common path stays short and its code compact.
  if (smin < -1074) {
#pragma unroll
    for (int v = 0; v < kRowsPerThread; ++v)
      out[v] = crt_round<L, CrtTable<S>::kW, CrtTable<S>::kTopExp>(acc[v], scale[v]);
  }
  double* dst = C + i0 + static_cast<long>(j) * ldc;
  if (beta != 0.0) {
#pragma unroll
    for (int v = 0; v < kRowsPerThread; ++v)
      if (i0 + v < p) out[v] = fma(alpha, out[v], beta * dst[v]);
  } else if (alpha != 1.0) {
#pragma unroll
    for (int v = 0; v < kRowsPerThread; ++v) out[v] *= alpha;
  }
  if (i0 + kRowsPerThread <= p && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
    typedef double v2d __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int v = 0; v < kRowsPerThread; v += 2) reinterpret_cast<v2d*>(dst)[v / 2] = v2d{out[v], out[v + 1]};
  } else {
#pragma unroll
    for (int v = 0; v < kRowsPerThread; ++v)
      if (i0 + v < p) dst[v] = out[v];
  }
}

template <int S>
static void launch_crt_s(const Work& w, double* C, long ldc, double alpha, double beta, const DumpPtrs& dump,
                         hipStream_t st) {
  const int groups = (w.p + kRowsPerThread - 1) / kRowsPerThread;
  if (groups == 0 || w.r == 0) return;
  const dim3 blocks(w.r, (groups + 255) / 256);
  const long r_plane = w.res_plane;
  if (dump.x != nullptr)
    hipLaunchKernelGGL((crt_kernel<S, true>), blocks, dim3(256), 0, st, w.res, r_plane, w.p_pad, w.p, w.r,
                       groups, w.d, w.b, C, ldc, alpha, beta, dump.x);
  else
    hipLaunchKernelGGL((crt_kernel<S, false>), blocks, dim3(256), 0, st, w.res, r_plane, w.p_pad, w.p, w.r,
                       groups, w.d, w.b, C, ldc, alpha, beta, nullptr);
}

template <int S>
static bool dispatch_crt(const Work& w, double* C, long ldc, double alpha, double beta, const DumpPtrs& dump,
                         hipStream_t st) {
  if constexpr (S > kMaxS) {
    return false;
  } else {
    if (w.s == S) {
      launch_crt_s<S>(w, C, ldc, alpha, beta, dump, st);
      return true;
    }
    return dispatch_crt<S + 1>(w, C, ldc, alpha, beta, dump, st);
  }
}

hipError_t launch_crt(const Work& w, double* C, long ldc, double alpha, double beta, const DumpPtrs& dump,
                      hipStream_t st) {
  if (!dispatch_crt<kMinS>(w, C, ldc, alpha, beta, dump, st)) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace oz2
