// oz2_residue.hip -- residue stage: A' = trunc(D A), B' = trunc(B E) and all s centered
// residues A_t = rho_{m_t}(A'), B_t = rho_{m_t}(B') in one pass over each FP64 element.
//
// "Profiling Ozaki II: The Cost Behind Fast INT8 GEMMs", Part II section 8 identifies the
// repeated per-modulus FP64 remainder chain as the preprocessing bottleneck and section
// 10.1 proposes converting each scaled element to an integer once and reducing it with
// fixed-divisor integer arithmetic.  This kernel goes further:
//   * the scaled, truncated value is never formed in floating point: from the FP64
//     fields (sign, 53-bit significand mu, exponent eta) |A'| = floor(mu 2^(eta + d)),
//     exactly, for any magnitude (not only below 2^63);
//   * |A'| is cut once into a 22-bit limb and NLHI 12-bit limbs, the sign is applied to
//     the limbs, and per modulus one dot product with the compile-time centered residues
//     of the limb weights gives z = A' (mod m) with |z| < 2^23 (v_mad_i32_i24);
//   * z - m round(z/m) is the centered residue for odd m; round(z/m) comes from one FP32
//     FMA that is exact at this size, and the final v_mad_i32_i24 lands the residue in
//     the low byte (the extra multiple m 2^22 it carries is 0 mod 256);
//   * m = 256 is the low byte of the signed low limb.
// No FP64 arithmetic and no integer division run inside the modulus loop.
//
// Output layout: planes A_t[t] (p_pad x q_pad) and B_t[t] (r_pad x q_pad, one row per
// column of B) int8, tile-contiguous for the GEMM (operand_chunk_offset); each thread
// stores 16 residues of one row as one 16-byte chunk.
#include <algorithm>

#include "oz2_common.hpp"
#include "oz2_internal.hpp"

namespace oz2 {

template <int T>
struct ModConst {
  static constexpr int m = modulus(T);
  static constexpr float inv = 1.0f / static_cast<float>(modulus(T));
};

// Signed limbs of A' = trunc(2^scale x): l[0] = 22 low bits, l[k] = 12-bit limb at bit
// 22 + 12 (k - 1); the sign of x is applied to every limb.  Also returns A' as an exact
// double when requested.
template <int NLHI>
__device__ __forceinline__ void scaled_limbs(double x, int scale, int (&l)[NLHI + 1], double* ap) {
  const uint64_t bits = static_cast<uint64_t>(__double_as_longlong(x));
  const bool neg = (bits >> 63) != 0;
  const int be = static_cast<int>((bits >> 52) & 0x7FF);
  uint64_t mu = bits & 0xFFFFFFFFFFFFFull;
  if (be != 0) mu |= 1ull << 52;
  if (be == 0x7FF) mu = 0;  // non-finite input: flagged in the scaling stage, treated as 0
  const int sig = (be != 0 ? be - 1075 : -1074) + scale;
  uint64_t lo, hi;
  if (sig >= 0) {
    const int sh = min(sig, 63);
    lo = mu << sh;
    hi = sh == 0 ? 0ull : mu >> (64 - sh);
  } else {
    const int sh = -sig;
    lo = sh < 64 ? mu >> sh : 0ull;
    hi = 0ull;
  }
  if (ap != nullptr) {
    const double v = sig >= 0 ? ldexp(static_cast<double>(mu), sig) : static_cast<double>(lo);
    *ap = neg ? -v : v;
  }
  // the sign is applied with a select so the compiler keeps the 24-bit range of each limb
  const int l0 = static_cast<int>(lo & ((1ull << kLimb0) - 1));
  l[0] = neg ? -l0 : l0;
#pragma unroll
  for (int k = 1; k <= NLHI; ++k) {
    const int pos = kLimb0 + kLimbHi * (k - 1);
    uint64_t f;
    if (pos + kLimbHi <= 64)
      f = lo >> pos;
    else if (pos >= 64)
      f = hi >> (pos - 64);
    else
      f = (lo >> pos) | (hi << (64 - pos));
    const int lk = static_cast<int>(f & ((1ull << kLimbHi) - 1));
    l[k] = neg ? -lk : lk;
  }
}

// a[23:0] * b[23:0] + c with signed 24-bit operands, as one full-rate v_mad_i32_i24
// (the compiler would otherwise strength-reduce constant multipliers into longer
// shift/add sequences).  b is a wave-uniform constant held in an SGPR.
__device__ __forceinline__ int mad_i24(int a, int b, int c) {
  int d;
  asm("v_mad_i32_i24 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(b), "v"(c));
  return d;
}

// Centered residue of the value held in signed limbs, for modulus index T, in the low
// byte of the returned int (higher bits are not meaningful).
template <int T, int NLHI>
__device__ __forceinline__ int residue_byte(const int (&l)[NLHI + 1]) {
  constexpr int m = ModConst<T>::m;
  if constexpr (m == 256) {
    return l[0];
  } else {
    int z = l[0];
#pragma unroll
    for (int k = 1; k <= NLHI; ++k) z = mad_i24(l[k], limb_coef(T, k), z);
    // y = 1.5 * 2^23 + round(z / m): |z| < 2^23, so z / m is within 1/(2m) of z * inv
    // and never within 1/(2m) of a half-integer (m odd): the rounding is exact.
    const float y = __builtin_fmaf(static_cast<float>(z), ModConst<T>::inv, 12582912.0f);
    // low 24 bits of y are 2^22 + round(z/m); z - m (2^22 + round(z/m)) = rho_m(z) - m 2^22
    return mad_i24(__float_as_int(y), -m, z);
  }
}

// Low bytes of a, b, c, d packed little-endian into one word with three v_perm_b32
// (selector 0x0c yields a zero byte, 0-3 pick bytes of the second operand, 4-7 of the first).
__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
  const uint32_t ab = __builtin_amdgcn_perm(static_cast<uint32_t>(b), static_cast<uint32_t>(a), 0x0c0c0400u);
  const uint32_t cd = __builtin_amdgcn_perm(static_cast<uint32_t>(d), static_cast<uint32_t>(c), 0x0c0c0400u);
  return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

template <int S, int NLHI, int T>
__device__ __forceinline__ void store_residues(const int (&l)[16][NLHI + 1], int8_t* dst, long plane) {
  if constexpr (T < S) {
    int rr[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) rr[k] = residue_byte<T, NLHI>(l[k]);
    uint4 v = make_uint4(pack4(rr[0], rr[1], rr[2], rr[3]), pack4(rr[4], rr[5], rr[6], rr[7]),
                         pack4(rr[8], rr[9], rr[10], rr[11]), pack4(rr[12], rr[13], rr[14], rr[15]));
    *reinterpret_cast<uint4*>(dst + T * plane) = v;
    store_residues<S, NLHI, T + 1>(l, dst, plane);
  }
}

// Lines that are rows of a column-major matrix (rows of A, or columns of op(B) = B^T);
// thread mapping owner_rows_of_a (the thread's 16 elements of line i are
// l = 256 blk + L + 16 k).  The validation dump of the scaled operand receives element
// (line, l) at ap_dump[line dls + l dks].
template <int S, int NLHI, bool DUMP>
__global__ __launch_bounds__(256) void residues_rows_kernel(const double* __restrict__ A, long lda, int p, int q,
                                                            const int* __restrict__ dsc, int8_t* __restrict__ at,
                                                            long plane, int q_pad, double* __restrict__ ap_dump,
                                                            long dls, long dks) {
  const ChunkOwner own = owner_rows_of_a();
  const int i = own.row;
  const bool row_ok = i < p;
  const int scale = row_ok ? dsc[i] : 0;
  int l[16][NLHI + 1];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int col = own.blk * kKPad + own.slot + 16 * k;
    const bool ok = row_ok && col < q;
    const double x = ok ? A[i + static_cast<long>(col) * lda] : 0.0;
    double apv;
    scaled_limbs<NLHI>(x, scale, l[k], DUMP ? &apv : nullptr);
    if constexpr (DUMP) {
      if (ok) ap_dump[i * dls + col * dks] = apv;
    }
  }
  store_residues<S, NLHI, 0>(l, at + operand_chunk_offset(i, own.blk, own.slot, q_pad), plane);
}

// Contiguous lines (columns of B, or rows of op(A) = A^T); thread mapping
// owner_cols_of_b.  Dump as in residues_rows_kernel.
template <int S, int NLHI, bool DUMP>
__global__ __launch_bounds__(256) void residues_cols_kernel(const double* __restrict__ B, long ldb, int q, int r,
                                                            const int* __restrict__ bsc, int8_t* __restrict__ bt,
                                                            long plane, int q_pad, double* __restrict__ bp_dump,
                                                            long dls, long dks) {
  const ChunkOwner own = owner_cols_of_b();
  const int j = own.row;
  const bool col_ok = j < r;
  const int scale = col_ok ? bsc[j] : 0;
  const double* col = B + static_cast<long>(col_ok ? j : 0) * ldb;
  int l[16][NLHI + 1];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int row = own.blk * kKPad + own.slot + 16 * k;
    const bool ok = col_ok && row < q;
    const double x = ok ? col[row] : 0.0;
    double bpv;
    scaled_limbs<NLHI>(x, scale, l[k], DUMP ? &bpv : nullptr);
    if constexpr (DUMP) {
      if (ok) bp_dump[j * dls + row * dks] = bpv;
    }
  }
  store_residues<S, NLHI, 0>(l, bt + operand_chunk_offset(j, own.blk, own.slot, q_pad), plane);
}

// Residue planes of one operand (nlines_pad rows); dump element (line, l) at
// dump[line dls + l dks].
template <int S, int NL, bool DUMP>
static void residues_lines(const Operand& o, int nlines, int nlines_pad, int q, int q_pad, const int* scale,
                           int8_t* out, long plane, double* dump, long dls, long dks, hipStream_t st) {
  if (o.contig) {
    dim3 grid(nlines_pad / 16, q_pad / kKPad);
    hipLaunchKernelGGL((residues_cols_kernel<S, NL, DUMP>), grid, dim3(256), 0, st, o.ptr, o.ld, q, nlines, scale,
                       out, plane, q_pad, dump, dls, dks);
  } else {
    dim3 grid(nlines_pad / 64, q_pad / kStageK);
    hipLaunchKernelGGL((residues_rows_kernel<S, NL, DUMP>), grid, dim3(256), 0, st, o.ptr, o.ld, nlines, q, scale,
                       out, plane, q_pad, dump, dls, dks);
  }
}

template <int S, bool ACCU>
static void launch_residues_s(const Operand& a, const Operand& b, const Work& w, const DumpPtrs& dump,
                              hipStream_t st) {
  constexpr int NL = nl_hi(S, ACCU);
  if (w.q_pad == 0) return;
  // A' dump: column-major p x q (ld p); B' dump: column-major q x r (ld q); each operand
  // runs the dumping kernel only when its own dump is requested
  // B first: its statistics were the last pass over the inputs (measured 1-2% faster)
  if (dump.bp != nullptr)
    residues_lines<S, NL, true>(b, w.r, w.r_pad, w.q, w.q_pad, w.b, w.bt, w.bt_plane, dump.bp, static_cast<long>(w.q), 1L, st);
  else
    residues_lines<S, NL, false>(b, w.r, w.r_pad, w.q, w.q_pad, w.b, w.bt, w.bt_plane, nullptr, 0L, 0L, st);
  if (dump.ap != nullptr)
    residues_lines<S, NL, true>(a, w.p, w.p_pad, w.q, w.q_pad, w.d, w.at, w.at_plane, dump.ap, 1L, static_cast<long>(w.p), st);
  else
    residues_lines<S, NL, false>(a, w.p, w.p_pad, w.q, w.q_pad, w.d, w.at, w.at_plane, nullptr, 0L, 0L, st);
}

template <int S>
static bool dispatch_residues(int s, const Operand& a, const Operand& b, const Work& w, const DumpPtrs& dump,
                              hipStream_t st) {
  if constexpr (S > kMaxS) {
    return false;
  } else {
    if (s == S) {
      if (w.accu)
        launch_residues_s<S, true>(a, b, w, dump, st);
      else
        launch_residues_s<S, false>(a, b, w, dump, st);
      return true;
    }
    return dispatch_residues<S + 1>(s, a, b, w, dump, st);
  }
}

hipError_t launch_residues(const Operand& a, const Operand& b, const Work& w, const DumpPtrs& dump,
                           hipStream_t st) {
  if (!dispatch_residues<kMinS>(w.s, a, b, w, dump, st)) return hipErrorInvalidValue;
  return hipGetLastError();
}

// Validation: operand planes (tile-contiguous layout, plane_stride bytes apart) -> dst
// [planes][rows][q], plain row-major.  Grid-stride loop: the dispatch grid size counts
// work-items in 32 bits, so the launch is capped and each thread walks the whole range.
__global__ void unpack_operands_kernel(const int8_t* __restrict__ src, long plane_stride, int rows, int q, int q_pad,
                                       int8_t* __restrict__ dst, long total) {
  const long stride = static_cast<long>(gridDim.x) * blockDim.x;
  for (long idx = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int l = static_cast<int>(idx % q);
    const long rest = idx / q;
    const int row = static_cast<int>(rest % rows);
    const long plane = rest / rows;
    dst[idx] = src[plane * plane_stride + operand_elem_offset(row, l, q_pad)];
  }
}

hipError_t launch_unpack_operands(const int8_t* src, long plane_stride, int planes, int rows, int q, int q_pad,
                                  int8_t* dst, hipStream_t st) {
  const long total = static_cast<long>(planes) * rows * q;
  if (total <= 0) return hipSuccess;
  const long blocks = std::min<long>((total + 255) / 256, 1L << 20);
  hipLaunchKernelGGL(unpack_operands_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, src, plane_stride,
                     rows, q, q_pad, dst, total);
  return hipGetLastError();
}

}  // namespace oz2
