// oz2_residue.hip -- residue stage: A' = trunc(D A), B' = trunc(B E) and all s centered
// residues A_t = rho_{m_t}(A'), B_t = rho_{m_t}(B') in one pass over each FP64 element.
//
// "Profiling Ozaki II: The Cost Behind Fast INT8 GEMMs", Part II section 8 identifies the
// repeated per-modulus FP64 remainder chain as the preprocessing bottleneck and section
// 10.1 proposes converting each scaled element to an integer once and reducing it with
// fixed-divisor integer arithmetic.  Here:
//   * A' = trunc(2^d x) is formed once, exactly, in FP64 (any magnitude the scalings
//     allow, not only below 2^63), and split with exact FP64 steps into a 22-bit low part
//     lo and H = floor(A' / 2^22), which is written as eight balanced base-256 digits
//     (signed bytes) in two words;
//   * per odd modulus, one or two v_dot4_i32_i8 with the compile-time centered residues of
//     the digit weights give z = lo + sum_k d_k rho_m(2^(22 + 8 k)) = A' (mod m),
//     |z| < 2^23;
//   * z - m round(z/m) is the centered residue; round(z/m) comes from one FP32 FMA that is
//     exact at this size, and the final v_mad_i32_i24 lands the residue in the low byte
//     (the extra multiple m 2^22 it carries is 0 mod 256);
//   * m = 256 is the low byte of lo (A' in two's complement).
// No FP64 arithmetic and no integer division run inside the modulus loop: five VALU
// instructions per odd modulus and element.
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

// A' = trunc(2^scale x) = lo + 2^22 H with lo in [0, 2^22) and H = floor(A' / 2^22) held
// as eight balanced base-256 digits (signed bytes d_0..d_7, H = sum d_k 256^k) in w0, w1:
// with C = 0x80...80, the bytes of H + C are d_k + 128, so those of (H + C) ^ C are d_k.
// Exact for |H| < 2^62 (every s up to 20 in both modes).  Also returns A' as an exact
// double when requested.
struct ScaledDigits {
  int lo;
  uint32_t w0, w1;
};

__device__ __forceinline__ ScaledDigits scaled_digits(double x, int scale, double* ap) {
  // every step below is exact: A' is an integer below 2^84 with at most 53 significant
  // bits, scalings by powers of two do not round, floor and the FMAs produce integers that
  // fit (a value that underflows in ldexp is below 1 and truncates to 0 either way)
  const double xf = __builtin_isfinite(x) ? x : 0.0;  // non-finite: flagged in the scaling stage
  const double a = trunc(ldexp(xf, scale));            // A' = trunc(2^scale x)
  if (ap != nullptr) *ap = a;
  const double h = floor(a * 0x1p-22);                 // H = floor(A' / 2^22), |H| < 2^62
  const int lo = static_cast<int>(fma(-h, 0x1p22, a));  // A' - 2^22 H in [0, 2^22)
  const double hh = floor(h * 0x1p-32);                // |hh| < 2^30
  const uint32_t hl = static_cast<uint32_t>(fma(-hh, 0x1p32, h));
  const uint64_t hb = (static_cast<uint64_t>(static_cast<uint32_t>(static_cast<int>(hh))) << 32) | hl;
  constexpr uint64_t kC = 0x8080808080808080ull;
  const uint64_t dg = (hb + kC) ^ kC;
  return ScaledDigits{lo, static_cast<uint32_t>(dg), static_cast<uint32_t>(dg >> 32)};
}

// a[23:0] * b[23:0] + c with signed 24-bit operands, as one full-rate v_mad_i32_i24
// (the compiler would otherwise strength-reduce constant multipliers into longer
// shift/add sequences).  b is a wave-uniform constant held in an SGPR.
__device__ __forceinline__ int mad_i24(int a, int b, int c) {
  int d;
  asm("v_mad_i32_i24 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(b), "v"(c));
  return d;
}

// Digit coefficients of every modulus, in SGPRs: the empty asm makes them opaque to the
// optimizer, so the dot products take them as scalar operands (the three-operand form,
// which keeps lo) instead of as literals (the two-operand form, which would copy lo into
// the accumulator before every product).
struct DigitCoefs {
  int c[kMaxS][2];
};

template <int S, int ND>
__device__ __forceinline__ DigitCoefs load_coefs() {
  DigitCoefs cf{};
#pragma unroll
  for (int t = 0; t < S; ++t) {
    cf.c[t][0] = digit_coefs(t, 0);
    cf.c[t][1] = ND > 1 ? digit_coefs(t, 1) : 0;
    asm volatile("" : "+s"(cf.c[t][0]));
    if constexpr (ND > 1) asm volatile("" : "+s"(cf.c[t][1]));
  }
  return cf;
}

// Centered residue of A' for modulus index T, in the low byte of the returned int (higher
// bits are not meaningful).  ND: 1 or 2 digit words carry H.
template <int T, int ND>
__device__ __forceinline__ int residue_byte(const ScaledDigits& g, const DigitCoefs& cf) {
  constexpr int m = ModConst<T>::m;
  if constexpr (m == 256) {
    return g.lo;  // low byte of A' in two's complement
  } else {
    // z = lo + sum_k d_k rho_m(2^(22 + 8 k)) = A' (mod m), |z| < 2^22 + 8 * 128 * 127 < 2^23.
    // The clamp flag (saturation, never reached at this size) keeps the three-operand form.
    int z = __builtin_amdgcn_sdot4(static_cast<int>(g.w0), cf.c[T][0], g.lo, true);
    if constexpr (ND > 1) z = __builtin_amdgcn_sdot4(static_cast<int>(g.w1), cf.c[T][1], z, true);
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

template <int S, int ND, int T>
__device__ __forceinline__ void store_residues(const ScaledDigits (&g)[16], const DigitCoefs& cf, int8_t* dst,
                                               long plane) {
  if constexpr (T < S) {
    int rr[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) rr[k] = residue_byte<T, ND>(g[k], cf);
    uint4 v = make_uint4(pack4(rr[0], rr[1], rr[2], rr[3]), pack4(rr[4], rr[5], rr[6], rr[7]),
                         pack4(rr[8], rr[9], rr[10], rr[11]), pack4(rr[12], rr[13], rr[14], rr[15]));
    *reinterpret_cast<uint4*>(dst + T * plane) = v;
    store_residues<S, ND, T + 1>(g, cf, dst, plane);
  }
}

// One operand of the residue stage: its lines (rows of op(A) or columns of op(B)), the
// scaling exponent of each line, and where its residue planes go.
struct ResidueOperand {
  const double* ptr;
  long ld;
  int nlines;
  const int* scale;
  int8_t* out;
  long plane;
};

// Statistics partials of one operand's lines, for the residue launch that computes the
// fast-mode exponents itself: the partials of line n at pe[n nch ..] and ps[n nch ..]
// (fast_line_exponent); the exponents are stored to out.  That launch is used for at most
// kExpInResiduesBlocks blocks per line (exponents_in_residues).
constexpr int kExpInResiduesBlocks = 16;

struct LineStats {
  const int* pe;
  const double* ps;
  int nch;
  int tau;
  int* out;
};

// One lane's share of a line's partials, when G lanes share the line: blocks g + G t.
template <int G>
struct LinePartials {
  static constexpr int K = kExpInResiduesBlocks / G;
  int e[K];
  double s[K];
};

// The loads are unconditional, from clamped in-range addresses (line 0 and block nch - 1
// exist on this path), and the unused values are replaced afterwards: with no branch
// around them the wait for these first loads does not also wait for the element loads
// issued after them.
template <int G>
__device__ __forceinline__ LinePartials<G> load_partials(const LineStats& ls, int n, bool ok, int g) {
  LinePartials<G> lp;
  const long off = static_cast<long>(ok ? n : 0) * ls.nch;
#pragma unroll
  for (int t = 0; t < LinePartials<G>::K; ++t) {
    const int c = g + t * G;
    const long at = off + min(c, ls.nch - 1);
    const int ev = ls.pe[at];
    const double sv = ls.ps[at];
    const bool in = ok && c < ls.nch;
    lp.e[t] = in ? ev : kNoExp;
    lp.s[t] = in ? sv : 0.0;
  }
  return lp;
}

// Exponent of line n from the partials the group's lanes hold (fast_line_exponent's
// arithmetic); the workgroups of the first inner-dimension block (by == 0) store it for
// the later stages.
template <int G>
__device__ __forceinline__ int line_exponent(const LinePartials<G>& lp, const LineStats& ls, int n, bool ok, int by,
                                             int g) {
  int e = kNoExp;
#pragma unroll
  for (int t = 0; t < LinePartials<G>::K; ++t) e = max(e, lp.e[t]);
  e = group_max<G>(e);
  // (no branch on an all-zero line, whose terms are all 0: a branch would move the
  // loads of the sums after the element loads)
  uint64_t S = 0;
#pragma unroll
  for (int t = 0; t < LinePartials<G>::K; ++t) S += partial_at_line_scale(e, lp.e[t], lp.s[t]);
  S = group_sum_u64<G>(S);
  const int sc = e == kNoExp ? 0 : fast_exponent(e, S, ls.tau);
  if (ok && by == 0 && g == 0) ls.out[n] = sc;
  return sc;
}

// Lines that are rows of a column-major matrix (rows of A, or columns of op(B) = B^T);
// thread mapping owner_rows_of_a for workgroup (bx, by) (the thread's 16 elements of line i
// are l = 256 blk + L + 16 k).  The validation dump of the scaled operand receives element
// (line, l) at ap_dump[line dls + l dks].  A non-finite input (read as 0) sets the flag word.
// NT: non-temporal reads of the operand (Work::stream_inputs).  FUSE: the line exponents
// come from the statistics partials (line_exponent); the partials are loaded first and
// the elements next, so that the exponent's arithmetic runs while the elements arrive.
template <int S, int ND, bool DUMP, bool NT, bool FUSE = false>
__device__ __forceinline__ void residues_rows_block(const ResidueOperand& o, int q, int q_pad, int bx, int by,
                                                    unsigned* flags, double* ap_dump, long dls, long dks,
                                                    const LineStats& ls = LineStats{}) {
  const ChunkOwner own = owner_rows_of_a(bx, by);
  const int i = own.row;
  const bool row_ok = i < o.nlines;
  const int lg = threadIdx.x & 3;  // the 4 lanes of a row are consecutive (owner_rows_of_a)
  double xs[16];
  int scale;
  if constexpr (FUSE) {
    // (unconditional loads from clamped addresses, as in load_partials; q >= 1 here)
    const LinePartials<4> lp = load_partials<4>(ls, i, row_ok, lg);
    const double* line = o.ptr + (row_ok ? i : 0);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int col = own.blk * kKPad + own.slot + 16 * k;
      const double v = load_f64<NT>(line + static_cast<long>(min(col, q - 1)) * o.ld);
      xs[k] = row_ok && col < q ? v : 0.0;
    }
    scale = line_exponent<4>(lp, ls, i, row_ok, by, lg);
  } else {
    scale = row_ok ? o.scale[i] : 0;
  }
  ScaledDigits g[16];
  bool bad = false;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int col = own.blk * kKPad + own.slot + 16 * k;
    const bool ok = row_ok && col < q;
    double x;
    if constexpr (FUSE)
      x = xs[k];
    else
      x = ok ? load_f64<NT>(o.ptr + i + static_cast<long>(col) * o.ld) : 0.0;
    bad |= !__builtin_isfinite(x);
    double apv;
    g[k] = scaled_digits(x, scale, DUMP ? &apv : nullptr);
    if constexpr (DUMP) {
      if (ok) ap_dump[i * dls + col * dks] = apv;
    }
  }
  if (bad) atomicOr(flags, kFlagNonFinite);
  store_residues<S, ND, 0>(g, load_coefs<S, ND>(), o.out + operand_chunk_offset(i, own.blk, own.slot, q_pad), o.plane);
}

// Contiguous lines (columns of B, or rows of op(A) = A^T); thread mapping owner_cols_of_b
// for workgroup (bx, by).  Dump, flag, NT and FUSE as in residues_rows_block.
template <int S, int ND, bool DUMP, bool NT, bool FUSE = false>
__device__ __forceinline__ void residues_cols_block(const ResidueOperand& o, int q, int q_pad, int bx, int by,
                                                    unsigned* flags, double* bp_dump, long dls, long dks,
                                                    const LineStats& ls = LineStats{}) {
  const ChunkOwner own = owner_cols_of_b(bx, by);
  const int j = own.row;
  const bool col_ok = j < o.nlines;
  const double* col = o.ptr + static_cast<long>(col_ok ? j : 0) * o.ld;
  const int lg = threadIdx.x & 15;  // the 16 lanes of a column are consecutive (owner_cols_of_b)
  double xs[16];
  int scale;
  if constexpr (FUSE) {
    // (unconditional loads from clamped addresses, as in load_partials; q >= 1 here)
    const LinePartials<16> lp = load_partials<16>(ls, j, col_ok, lg);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int row = own.blk * kKPad + own.slot + 16 * k;
      const double v = load_f64<NT>(col + min(row, q - 1));
      xs[k] = col_ok && row < q ? v : 0.0;
    }
    scale = line_exponent<16>(lp, ls, j, col_ok, by, lg);
  } else {
    scale = col_ok ? o.scale[j] : 0;
  }
  ScaledDigits g[16];
  bool bad = false;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int row = own.blk * kKPad + own.slot + 16 * k;
    const bool ok = col_ok && row < q;
    double x;
    if constexpr (FUSE)
      x = xs[k];
    else
      x = ok ? load_f64<NT>(col + row) : 0.0;
    bad |= !__builtin_isfinite(x);
    double bpv;
    g[k] = scaled_digits(x, scale, DUMP ? &bpv : nullptr);
    if constexpr (DUMP) {
      if (ok) bp_dump[j * dls + row * dks] = bpv;
    }
  }
  if (bad) atomicOr(flags, kFlagNonFinite);
  store_residues<S, ND, 0>(g, load_coefs<S, ND>(), o.out + operand_chunk_offset(j, own.blk, own.slot, q_pad), o.plane);
}

// One operand per launch (grid of its own thread mapping), with or without the dump.
template <int S, int ND, bool DUMP, bool CONTIG, bool NT>
__global__ __launch_bounds__(256) void residues_kernel(ResidueOperand o, int q, int q_pad, unsigned* __restrict__ flags,
                                                       double* __restrict__ dump, long dls, long dks) {
  if constexpr (CONTIG)
    residues_cols_block<S, ND, DUMP, NT>(o, q, q_pad, blockIdx.x, blockIdx.y, flags, dump, dls, dks);
  else
    residues_rows_block<S, ND, DUMP, NT>(o, q, q_pad, blockIdx.x, blockIdx.y, flags, dump, dls, dks);
}

// Both operands in one launch, for column-major A and B (the untransposed product): the
// first nb_blocks workgroups take the columns of B (grid gxb wide), the rest the rows of A
// (grid gxa wide).  One launch instead of two saves a dependent kernel start and the ramp
// and tail of a second grid, which matter at small sizes.  FUSE: the fast-mode exponents
// are computed here from the statistics partials la, lb (exponents_in_residues).
template <int S, int ND, bool NT, bool FUSE>
__global__ __launch_bounds__(256) void residues_ab_kernel(ResidueOperand a, ResidueOperand b, int q, int q_pad,
                                                          int gxa, int gxb, int nb_blocks,
                                                          unsigned* __restrict__ flags, LineStats la, LineStats lb) {
  const int k = blockIdx.x;
  if (k < nb_blocks)
    residues_cols_block<S, ND, false, NT, FUSE>(b, q, q_pad, k % gxb, k / gxb, flags, nullptr, 0, 0, lb);
  else
    residues_rows_block<S, ND, false, NT, FUSE>(a, q, q_pad, (k - nb_blocks) % gxa, (k - nb_blocks) / gxa, flags,
                                                nullptr, 0, 0, la);
}

// Grid of one operand's residue launch: (lines / 16, q_pad / 256) for contiguous lines, else
// (lines / 64, q_pad / 64), over the padded line count.
static dim3 residue_grid(bool contig, int nlines_pad, int q_pad) {
  return contig ? dim3(nlines_pad / 16, q_pad / kKPad) : dim3(nlines_pad / 64, q_pad / kStageK);
}

// Residue planes of one operand (nlines_pad rows); dump element (line, l) at
// dump[line dls + l dks] (the dumping kernels read normally: validation only).
template <int S, int NL, bool DUMP, bool NT>
static void residues_lines(const Operand& o, int nlines, int nlines_pad, int q, int q_pad, const int* scale,
                           int8_t* out, long plane, unsigned* flags, double* dump, long dls, long dks, hipStream_t st) {
  static_assert(!(DUMP && NT), "dumping kernels read normally");
  const ResidueOperand ro{o.ptr, o.ld, nlines, scale, out, plane};
  const dim3 grid = residue_grid(o.contig, nlines_pad, q_pad);
  if (o.contig)
    hipLaunchKernelGGL((residues_kernel<S, NL, DUMP, true, NT>), grid, dim3(256), 0, st, ro, q, q_pad, flags, dump,
                       dls, dks);
  else
    hipLaunchKernelGGL((residues_kernel<S, NL, DUMP, false, NT>), grid, dim3(256), 0, st, ro, q, q_pad, flags, dump,
                       dls, dks);
}

template <int S, bool ACCU, bool NT>
static void launch_residues_nt(const Operand& a, const Operand& b, const Work& w, hipStream_t st) {
  constexpr int NL = digit_words(S, ACCU);
  // untransposed operands: one launch for both (B's workgroups first: its statistics were
  // the last pass over the inputs, measured 1-2% faster)
  const dim3 ga = residue_grid(a.contig, w.p_pad, w.q_pad), gb = residue_grid(b.contig, w.r_pad, w.q_pad);
  const long nb = static_cast<long>(gb.x) * gb.y, na = static_cast<long>(ga.x) * ga.y;
  // (a one-dimensional grid keeps its work-item count below 2^32)
  if (!a.contig && b.contig && nb + na < (1L << 24)) {
    const ResidueOperand ra{a.ptr, a.ld, w.p, w.d, w.at, w.at_plane};
    const ResidueOperand rb{b.ptr, b.ld, w.r, w.b, w.bt, w.bt_plane};
    if constexpr (!ACCU && !NT) {
      if (w.exp_in_residues) {
        const LineStats la{w.part_e_a, w.part_s_a, w.nch, w.tau, w.d};
        const LineStats lb{w.part_e_b, w.part_s_b, w.nch, w.tau, w.b};
        hipLaunchKernelGGL((residues_ab_kernel<S, NL, false, true>), dim3(static_cast<unsigned>(nb + na)), dim3(256),
                           0, st, ra, rb, w.q, w.q_pad, static_cast<int>(ga.x), static_cast<int>(gb.x),
                           static_cast<int>(nb), w.flags, la, lb);
        return;
      }
    }
    hipLaunchKernelGGL((residues_ab_kernel<S, NL, NT, false>), dim3(static_cast<unsigned>(nb + na)), dim3(256), 0, st,
                       ra, rb, w.q, w.q_pad, static_cast<int>(ga.x), static_cast<int>(gb.x), static_cast<int>(nb),
                       w.flags, LineStats{}, LineStats{});
    return;
  }
  residues_lines<S, NL, false, NT>(b, w.r, w.r_pad, w.q, w.q_pad, w.b, w.bt, w.bt_plane, w.flags, nullptr, 0L, 0L, st);
  residues_lines<S, NL, false, NT>(a, w.p, w.p_pad, w.q, w.q_pad, w.d, w.at, w.at_plane, w.flags, nullptr, 0L, 0L, st);
}

template <int S, bool ACCU>
static void launch_residues_s(const Operand& a, const Operand& b, const Work& w, const DumpPtrs& dump,
                              hipStream_t st) {
  constexpr int NL = digit_words(S, ACCU);
  if (w.q_pad == 0) return;
  if (dump.ap == nullptr && dump.bp == nullptr) {
    if (w.stream_inputs)
      launch_residues_nt<S, ACCU, true>(a, b, w, st);
    else
      launch_residues_nt<S, ACCU, false>(a, b, w, st);
    return;
  }
  // A' dump: column-major p x q (ld p); B' dump: column-major q x r (ld q); each operand
  // runs the dumping kernel only when its own dump is requested
  if (dump.bp != nullptr)
    residues_lines<S, NL, true, false>(b, w.r, w.r_pad, w.q, w.q_pad, w.b, w.bt, w.bt_plane, w.flags, dump.bp,
                                       static_cast<long>(w.q), 1L, st);
  else
    residues_lines<S, NL, false, false>(b, w.r, w.r_pad, w.q, w.q_pad, w.b, w.bt, w.bt_plane, w.flags, nullptr, 0L,
                                        0L, st);
  if (dump.ap != nullptr)
    residues_lines<S, NL, true, false>(a, w.p, w.p_pad, w.q, w.q_pad, w.d, w.at, w.at_plane, w.flags, dump.ap, 1L,
                                       static_cast<long>(w.p), st);
  else
    residues_lines<S, NL, false, false>(a, w.p, w.p_pad, w.q, w.q_pad, w.d, w.at, w.at_plane, w.flags, nullptr, 0L,
                                        0L, st);
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

// Fast mode moves the exponents into the residue launch when that launch takes both
// operands (untransposed, below 2^24 workgroups) without the non-temporal hint (so the
// statistics of both ran in one launch, which clears the flag word), no A' / B' dump is
// requested (the dumping kernels read d and b), and the inner dimension has at most
// kExpInResiduesBlocks 256-blocks: every residue workgroup that covers a line recomputes
// its exponent (q / 64 of them for a row of A, q / 256 for a column of B), so those reads
// of partials grow with q^2 per line.

bool exponents_in_residues(const Operand& a, const Operand& b, const Work& w, const DumpPtrs& dump) {
  if (w.accu || w.stream_inputs || a.contig || !b.contig || dump.ap != nullptr || dump.bp != nullptr) return false;
  if (w.nch <= 0 || w.nch > kExpInResiduesBlocks || w.p <= 0 || w.r <= 0) return false;
  const dim3 ga = residue_grid(false, w.p_pad, w.q_pad), gb = residue_grid(true, w.r_pad, w.q_pad);
  return static_cast<long>(ga.x) * ga.y + static_cast<long>(gb.x) * gb.y < (1L << 24);
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
