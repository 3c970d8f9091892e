// oz2_scaling.hip -- scaling stage: the power-of-two exponents d (rows of A) and b
// (columns of B) that define D = diag(2^d) and E = diag(2^b).
//
// fast ("Profiling Ozaki II: The Cost Behind Fast INT8 GEMMs", Part I section 2 and
// Part II section 5.1): Cauchy-Schwarz bound from per-line max-abs and sum of squares,
// sums rounded upward so the bound is never underestimated.  Here the sum of squares
// is taken exactly on integers: in every kChunk-long block with max-abs exponent e_c,
// u = ceil(|a| 2^(kFBits - e_c)) and S_c = sum u^2; blocks combine as
// S = sum_c ceil(S_c / 4^(e - e_c)) with e the line's max-abs exponent.  Then
// d = floor((tau - ceil(log2 S)) / 2) + kFBits - e, the largest exponent that keeps the
// scaled squared-norm bound within the budget 2^tau split equally between the row of A
// and the column of B.
//
// accu (same page, section 2 and 5.1 "accu"): |A| and |B| quantized upward into
// integers in [0, 2^kQBits] relative to each line's max-abs exponent, one INT8 bound
// GEMM (oz2_gemm.hip), row / column maxima rho, gamma of its output, then
// d = floor((tau - ceil(log2 max(rho, 1))) / 2) + kQBits - e.  The quantized inputs are
// formed without a second pass over A and B: the max-abs pass quantizes each element
// against its block's exponent e_c while the values are in registers, and a byte pass
// divides by 2^(e - e_c) with rounding up once the line exponent e is known
// (ceil(ceil(y) / 2^k) = ceil(y / 2^k)).
#include "oz2_common.hpp"
#include "oz2_internal.hpp"

namespace oz2 {

// Lines that are rows of a column-major matrix (rows of A, or columns of op(B) = B^T):
// kStatsRowGroups x 64 lines (one per lane) x one kChunk block per workgroup; the
// kStatsColGroups waves of a row group split the block's columns, wave w reading
// l in [c kChunk + kStatsCols w, +kStatsCols).  Each load instruction reads 64
// consecutive rows of one column.  MAXONLY: only the block max-abs exponents are produced.
constexpr int kStatsRowGroups = 1;
constexpr int kStatsColGroups = 8;
constexpr int kStatsCols = kChunk / kStatsColGroups;
constexpr int kStatsThreads = kWave * kStatsRowGroups * kStatsColGroups;
constexpr long kComputeUnits = 256;  // MI355X: 8 XCDs of 32
// Workgroup (bx, c) of the row statistics: rows 64 bx.. of block c.
template <bool MAXONLY, bool NT>
__device__ __forceinline__ void stats_rows_block(const double* __restrict__ A, long lda, int p, int q, int nch,
                                                 int* __restrict__ part_e, double* __restrict__ part_s,
                                                 int8_t* __restrict__ qout, int q_pad, int bx, int c) {
  __shared__ int sh_e[kStatsRowGroups][kStatsColGroups][kWave];
  __shared__ double sh_s[kStatsRowGroups][kStatsColGroups][kWave];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = wave / kStatsColGroups;
  const int w = wave % kStatsColGroups;
  const int i = (bx * kStatsRowGroups + g) * kWave + lane;
  const int l0 = c * kChunk + w * kStatsCols;
  const bool row_ok = i < p;
  const double* base = A + (row_ok ? i : 0) + static_cast<long>(l0) * lda;

  double v[kStatsCols];
  int emax = kNoExp;
#pragma unroll
  for (int k = 0; k < kStatsCols; ++k) {
    double x = 0.0;
    if (row_ok && l0 + k < q) x = load_f64<NT>(base + static_cast<long>(k) * lda);
    x = is_nonfinite(x) ? 0.0 : x;  // (flagged by the residue stage)
    v[k] = x;
    emax = max(emax, exponent_of(x));
  }
  sh_e[g][w][lane] = emax;
  __syncthreads();
  int ec = kNoExp;
#pragma unroll
  for (int u = 0; u < kStatsColGroups; ++u) ec = max(ec, sh_e[g][u][lane]);
  if constexpr (MAXONLY) {
    if (w == 0 && row_ok) part_e[static_cast<long>(i) * nch + c] = ec;
    if (qout != nullptr) {
      // block-quantized bound input ceil(|a| 2^(kQBits - e_c)) in the operand tile layout:
      // element 32 w + k of the block goes to chunk slot k mod 16, byte 2 w + k / 16
      static_assert(kStatsColGroups == 8 && kStatsRowGroups == 1, "one row group, two bytes per wave and slot");
      __shared__ __attribute__((aligned(16))) uint16_t sq[kWave][16][8];  // read as 16-byte chunks
#pragma unroll
      for (int L = 0; L < 16; ++L) {
        uint32_t q0 = 0, q1 = 0;
        if (ec != kNoExp) {
          q0 = static_cast<uint32_t>(ceil_scaled_abs(v[L], kQBits - ec));
          q1 = static_cast<uint32_t>(ceil_scaled_abs(v[L + 16], kQBits - ec));
        }
        sq[lane][L][w] = static_cast<uint16_t>(q0 | (q1 << 8));
      }
      __syncthreads();
      // 64 rows x 16 chunks; consecutive threads fill one 64-byte row segment, then the next
      // row, so each wave stores 1 KiB of one stage tile contiguously
      const int row0 = bx * kWave;
#pragma unroll
      for (int ci = threadIdx.x; ci < kWave * 16; ci += kStatsThreads) {
        const int rrow = (ci >> 2) & (kWave - 1);
        const int rr = row0 + rrow;
        const int slot = 4 * (ci >> 8) + ((ci & 3) ^ operand_swizzle(rr & 15));
        *reinterpret_cast<uint4*>(qout + operand_chunk_offset(rr, c, slot, q_pad)) =
            *reinterpret_cast<const uint4*>(&sq[rrow][slot][0]);
      }
    }
    return;
  } else {
    double acc = 0.0;  // exact: at most kStatsCols * 2^40
    if (ec != kNoExp) {
#pragma unroll
      for (int k = 0; k < kStatsCols; ++k) {
        const double u = ceil_scaled_abs(v[k], kFBits - ec);
        acc = fma(u, u, acc);
      }
    }
    sh_s[g][w][lane] = acc;
    __syncthreads();
    if (w == 0 && row_ok) {
      // exact integer sums below 2^49: the grouping does not matter
      double tot = 0.0;
#pragma unroll
      for (int u = 0; u < kStatsColGroups; ++u) tot += sh_s[g][u][lane];
      part_e[static_cast<long>(i) * nch + c] = ec;
      part_s[static_cast<long>(i) * nch + c] = tot;
    }
  }
}

template <bool MAXONLY, bool NT>
__global__ __launch_bounds__(kStatsThreads) void stats_rows_kernel(const double* __restrict__ A, long lda, int p,
                                                                   int q, int nch, int* __restrict__ part_e,
                                                                   double* __restrict__ part_s,
                                                                   int8_t* __restrict__ qout, int q_pad) {
  stats_rows_block<MAXONLY, NT>(A, lda, p, q, nch, part_e, part_s, qout, q_pad, blockIdx.x, blockIdx.y);
}

// Contiguous lines (columns of B, or rows of op(A) = A^T): one wave per line j and
// CB consecutive blocks c; for each block, lane reads l = c kChunk + lane + 64 k,
// k = 0..3, so every load instruction is 512 contiguous bytes, and all of the wave's loads
// are issued before the first block is reduced.  CB = 2 where lines have at most 32
// blocks (more waves in flight on small grids), else 8 (one wave per block made 65536 tiny
// workgroups at n = 8192, which the dispatcher could not launch fast enough).
// One wave: line j, blocks c0 .. c0 + CB - 1.
template <bool MAXONLY, int CB, bool NT>
__device__ __forceinline__ void stats_cols_wave(const double* __restrict__ B, long ldb, int q, int r, int nch,
                                                int* __restrict__ part_e, double* __restrict__ part_s,
                                                int8_t* __restrict__ qout, int q_pad, int j, int c0) {
  const int lane = threadIdx.x & 63;
  if (c0 >= nch) return;  // whole wave
  const bool col_ok = j < r;  // columns up to the padded count when the bound input is written
  const double* col = B + static_cast<long>(col_ok ? j : 0) * ldb;
  double v[CB][4];
#pragma unroll
  for (int b = 0; b < CB; ++b)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int l = (c0 + b) * kChunk + lane + kWave * k;
      const double x = (col_ok && c0 + b < nch && l < q) ? load_f64<NT>(col + l) : 0.0;
      v[b][k] = is_nonfinite(x) ? 0.0 : x;  // (flagged by the residue stage)
    }
#pragma unroll
  for (int b = 0; b < CB; ++b) {
    const int c = c0 + b;
    if (c >= nch) break;  // whole wave
    int emax = kNoExp;
#pragma unroll
    for (int k = 0; k < 4; ++k) emax = max(emax, exponent_of(v[b][k]));
    const int ec = wave_max(emax);
    const long slot = static_cast<long>(j) * nch + c;
    if constexpr (MAXONLY) {
      if (lane == 0 && col_ok) part_e[slot] = ec;
      if (qout != nullptr) {
        // block-quantized bound input: element lane + 64 k goes to chunk slot lane mod 16,
        // byte lane / 16 + 4 k; lane L < 16 gathers the words of lanes L + 16 g and
        // transposes the 4 x 4 bytes into its chunk
        uint32_t pk = 0;
        if (ec != kNoExp) {
#pragma unroll
          for (int k = 0; k < 4; ++k)
            pk |= static_cast<uint32_t>(ceil_scaled_abs(v[b][k], kQBits - ec)) << (8 * k);
        }
        const int L = lane & 15;
        const uint32_t g0 = static_cast<uint32_t>(__shfl(static_cast<int>(pk), L, kWave));
        const uint32_t g1 = static_cast<uint32_t>(__shfl(static_cast<int>(pk), L + 16, kWave));
        const uint32_t g2 = static_cast<uint32_t>(__shfl(static_cast<int>(pk), L + 32, kWave));
        const uint32_t g3 = static_cast<uint32_t>(__shfl(static_cast<int>(pk), L + 48, kWave));
        // word k of the chunk = byte k of g0, g1, g2, g3
        const uint32_t lo01 = __builtin_amdgcn_perm(g1, g0, 0x05010400u);  // g0.b0 g1.b0 g0.b1 g1.b1
        const uint32_t hi01 = __builtin_amdgcn_perm(g1, g0, 0x07030602u);  // g0.b2 g1.b2 g0.b3 g1.b3
        const uint32_t lo23 = __builtin_amdgcn_perm(g3, g2, 0x05010400u);
        const uint32_t hi23 = __builtin_amdgcn_perm(g3, g2, 0x07030602u);
        const uint4 chunk = make_uint4(__builtin_amdgcn_perm(lo23, lo01, 0x05040100u),
                                       __builtin_amdgcn_perm(lo23, lo01, 0x07060302u),
                                       __builtin_amdgcn_perm(hi23, hi01, 0x05040100u),
                                       __builtin_amdgcn_perm(hi23, hi01, 0x07060302u));
        if (lane < 16) *reinterpret_cast<uint4*>(qout + operand_chunk_offset(j, c, L, q_pad)) = chunk;
      }
    } else {
      double acc = 0.0;
      if (ec != kNoExp) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const double u = ceil_scaled_abs(v[b][k], kFBits - ec);
          acc = fma(u, u, acc);
        }
      }
      acc = wave_sum(acc);  // exact: at most 256 * 2^40
      if (lane == 0) {
        part_e[slot] = ec;
        part_s[slot] = acc;
      }
    }
  }
}

// grid: x = column j, y = groups of 4 CB blocks; one wave per (j, CB blocks)
template <bool MAXONLY, int CB, bool NT>
__global__ __launch_bounds__(256) void stats_cols_kernel(const double* __restrict__ B, long ldb, int q, int r,
                                                         int nch, int* __restrict__ part_e,
                                                         double* __restrict__ part_s,
                                                         int8_t* __restrict__ qout, int q_pad) {
  stats_cols_wave<MAXONLY, CB, NT>(B, ldb, q, r, nch, part_e, part_s, qout, q_pad, blockIdx.x,
                                   (blockIdx.y * 4 + (threadIdx.x >> 6)) * CB);
}

// Fast-mode statistics of both operands in one launch, for column-major A and B (the
// untransposed product) that fit the memory-side cache: nb_blocks workgroups take the
// columns of B, 8 waves of (column, CB blocks) items each, and gxa x nch workgroups the rows
// of A (one stats_rows_block each).  On small products the two grids then run side by side
// instead of one after the other (n = 1024: 12.8 against 15.9 us); on large ones the merged
// kernel, then at 100 registers (four waves per SIMD against six), was slower (n = 8192:
// 0.212 against 0.178 ms), so they keep two launches.  A row workgroup reads 4x the bytes of
// a column one; when there are at least as many as compute units they go first, so that
// they do not form the launch's tail, and the kernel is held to 80 registers so that three
// workgroups share a CU.  Only the two together paid: n = 2048, 23.0 us against 23.9 (rows
// first at 100 registers) and 24.2 (columns first, at either count).  With fewer row
// workgroups columns go first (n = 1024: 12.5 against 12.9 us).
template <int CB>
__global__ __launch_bounds__(kStatsThreads) __attribute__((amdgpu_waves_per_eu(6))) void stats_ab_kernel(const double* __restrict__ A, long lda, int p,
                                                                 const double* __restrict__ B, long ldb, int r,
                                                                 int q, int nch, int gxa, int nb_blocks,
                                                                 int a_first,
                                                                 int* __restrict__ pe_a, double* __restrict__ ps_a,
                                                                 int* __restrict__ pe_b, double* __restrict__ ps_b,
                                                                 unsigned* __restrict__ flags) {
  static_assert(kStatsThreads == 8 * kWave, "8 waves per workgroup");
  // the call's non-finite flag starts here when the residue kernel computes the exponents
  // itself (no exponent launch, which otherwise clears it again)
  if (blockIdx.x == 0 && threadIdx.x == 0) *flags = 0u;
  const int na_blocks = gxa * nch;
  int k = blockIdx.x;
  bool col;  // a workgroup of B's columns; k becomes its index within its operand's grid
  if (a_first) {
    col = k >= na_blocks;
    if (col) k -= na_blocks;
  } else {
    col = k < nb_blocks;
    if (!col) k -= nb_blocks;
  }
  if (col) {
    const int groups = (nch + CB - 1) / CB;
    const long item = static_cast<long>(k) * 8 + (threadIdx.x >> 6);
    const int j = static_cast<int>(item / groups);
    if (j >= r) return;  // whole wave
    stats_cols_wave<false, CB, false>(B, ldb, q, r, nch, pe_b, ps_b, nullptr, 0, j,
                                      static_cast<int>(item % groups) * CB);
  } else {
    stats_rows_block<false, false>(A, lda, p, q, nch, pe_a, ps_a, nullptr, 0, k % gxa, k / gxa);
  }
}

// One wave per line (rows of A first, then columns of B): combine the block partials, the
// lanes taking blocks lane, lane + 64, ...
__global__ __launch_bounds__(256) void fast_exponents_kernel(int na, int nb, int nch, const int* __restrict__ pe_a,
                                                             const double* __restrict__ ps_a,
                                                             const int* __restrict__ pe_b,
                                                             const double* __restrict__ ps_b, int* __restrict__ d,
                                                             int* __restrict__ b, int tau,
                                                             unsigned* __restrict__ flags) {
  const int lane = threadIdx.x & 63;
  const int idx = blockIdx.x * 4 + (threadIdx.x >> 6);
  // the call's non-finite flag starts here (the merged statistics launch clears it too):
  // the residue stage, which runs after this kernel, sets it
  if (blockIdx.x == 0 && threadIdx.x == 0) *flags = 0u;
  if (idx >= na + nb) return;  // whole wave
  const bool is_a = idx < na;
  const int line = is_a ? idx : idx - na;
  const long off = static_cast<long>(line) * nch;
  const int out = fast_line_exponent<kWave>((is_a ? pe_a : pe_b) + off, (is_a ? ps_a : ps_b) + off, nch, lane, tau);
  if (lane == 0) {
    if (is_a)
      d[line] = out;
    else
      b[line] = out;
  }
}

// accu: line max-abs exponents from block maxima.
// Also starts the bound product's row / column maxima at 0 (the bound GEMM, which runs after
// this kernel, accumulates them with atomics).
__global__ void max_exponents_kernel(int na, int nb, int nch, const int* __restrict__ pe_a,
                                     const int* __restrict__ pe_b, int* __restrict__ e_row,
                                     int* __restrict__ f_col, int* __restrict__ rho, int* __restrict__ gamma) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= na + nb) return;
  const bool is_a = idx < na;
  const int line = is_a ? idx : idx - na;
  const int* pe = (is_a ? pe_a : pe_b) + static_cast<long>(line) * nch;
  int e = kNoExp;
  for (int c = 0; c < nch; ++c) e = max(e, pe[c]);
  if (is_a) {
    e_row[line] = e;
    rho[line] = 0;
  } else {
    f_col[line] = e;
    gamma[line] = 0;
  }
}

// accu bound inputs of lines that are rows of a column-major matrix:
// accu bound input from its block-quantized form: the statistics pass wrote
// Abar'_il = ceil(|a_il| 2^(kQBits - e_c)) with the block exponent e_c <= e_i, and
// ceil(|a| 2^(kQBits - e_i)) = ceil(Abar' / 2^(e_i - e_c)) (nested ceilings by a power of
// two).  Bytes are at most 64, so v + 2^kk - 1 stays below 256 and the four bytes of a word
// are shifted together; kk = min(e_i - e_c, 7) (a shift by 7 or more leaves v > 0 ? 1 : 0).
// grid: x = (lines x 4 chunks) / 256, y = the 4 stages of each 256-block.
__global__ __launch_bounds__(256) void requant_kernel(int8_t* __restrict__ plane, int nlines, int nch, int q_pad,
                                                      const int* __restrict__ e_line,
                                                      const int* __restrict__ part_e) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int line = t >> 2;
  if (line >= nlines) return;
  const int blk = blockIdx.y >> 2;
  const int e = e_line[line];
  const int ec = part_e[static_cast<long>(line) * nch + blk];
  if (e == kNoExp || ec == kNoExp || e == ec) return;  // zero chunk, or no shift
  const int kk = min(e - ec, 7);
  const int slot = 4 * (blockIdx.y & 3) + ((t & 3) ^ operand_swizzle(line & 15));
  uint4* ptr = reinterpret_cast<uint4*>(plane + operand_chunk_offset(line, blk, slot, q_pad));
  const uint32_t add = ((1u << kk) - 1u) * 0x01010101u;
  const uint32_t mask = (0xFFu >> kk) * 0x01010101u;
  uint4 x = *ptr;
  x.x = ((x.x + add) >> kk) & mask;
  x.y = ((x.y + add) >> kk) & mask;
  x.z = ((x.z + add) >> kk) & mask;
  x.w = ((x.w + add) >> kk) & mask;
  *ptr = x;
}

// accu exponents from the bound-product maxima.
__global__ void accu_exponents_kernel(int na, int nb, const int* __restrict__ e_row,
                                      const int* __restrict__ f_col, const int* __restrict__ rho,
                                      const int* __restrict__ gamma, int* __restrict__ d,
                                      int* __restrict__ b, int tau, unsigned* __restrict__ flags) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  // the call's non-finite flag starts here (set by the residue stage, which runs after)
  if (idx == 0) *flags = 0u;
  if (idx >= na + nb) return;
  const bool is_a = idx < na;
  const int line = is_a ? idx : idx - na;
  const int e = is_a ? e_row[line] : f_col[line];
  const int peak = is_a ? rho[line] : gamma[line];
  int out = 0;
  if (e != kNoExp) out = ((tau - clog2_u64(static_cast<uint64_t>(max(peak, 1)))) >> 1) + kQBits - e;
  if (is_a)
    d[line] = out;
  else
    b[line] = out;
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
static inline unsigned blocks_for(long n, int per) { return static_cast<unsigned>((n + per - 1) / per); }

// Block statistics of the lines of one operand (rows of op(A) or columns of op(B)).
// With qout (accu), the block-quantized bound input of every line up to nlines_pad is written
// too (zeros past nlines), in the operand tile layout of q_pad columns.  NT: non-temporal
// reads of the operand (Work::stream_inputs).
template <bool MAXONLY, bool NT>
static void stats_lines(const Operand& o, int nlines, int nlines_pad, int q, int q_pad, int nch, int* pe, double* ps,
                        int8_t* qout, hipStream_t st) {
  if (nch == 0 || nlines == 0) return;
  const int ngrid = qout != nullptr ? nlines_pad : nlines;
  if (o.contig) {
    if (nch <= 32) {
      dim3 grid(ngrid, blocks_for(nch, 4 * 2));
      hipLaunchKernelGGL((stats_cols_kernel<MAXONLY, 2, NT>), grid, dim3(256), 0, st, o.ptr, o.ld, q, nlines, nch, pe,
                         ps, qout, q_pad);
    } else {
      dim3 grid(ngrid, blocks_for(nch, 4 * 8));
      hipLaunchKernelGGL((stats_cols_kernel<MAXONLY, 8, NT>), grid, dim3(256), 0, st, o.ptr, o.ld, q, nlines, nch, pe,
                         ps, qout, q_pad);
    }
  } else {
    dim3 grid(blocks_for(ngrid, kWave * kStatsRowGroups), nch);
    hipLaunchKernelGGL((stats_rows_kernel<MAXONLY, NT>), grid, dim3(kStatsThreads), 0, st, o.ptr, o.ld, nlines, q, nch,
                       pe, ps, qout, q_pad);
  }
}

template <int CB>
static void launch_stats_ab(const Operand& a, const Operand& b, const Work& w, long nb_blocks, long gxa,
                            hipStream_t st) {
  const long na_blocks = gxa * w.nch;
  const int a_first = na_blocks >= kComputeUnits ? 1 : 0;
  hipLaunchKernelGGL((stats_ab_kernel<CB>), dim3(static_cast<unsigned>(nb_blocks + na_blocks)), dim3(kStatsThreads),
                     0, st, a.ptr, a.ld, w.p, b.ptr, b.ld, w.r, w.q, w.nch, static_cast<int>(gxa),
                     static_cast<int>(nb_blocks), a_first, w.part_e_a, w.part_s_a, w.part_e_b, w.part_s_b,
                     w.flags);
}

template <bool MAXONLY>
static hipError_t launch_stats(const Operand& a, const Operand& b, const Work& w, hipStream_t st) {
  if (!MAXONLY && !w.stream_inputs && !a.contig && b.contig && w.nch > 0 && w.p > 0 && w.r > 0) {
    // both operands in one launch (operands below 128 MiB: far fewer than 2^31 workgroups)
    const int cb = w.nch <= 32 ? 2 : 8;
    const long nb_blocks = (static_cast<long>(w.r) * ((w.nch + cb - 1) / cb) + 7) / 8;
    const long gxa = blocks_for(w.p, kWave * kStatsRowGroups);
    if (cb == 2)
      launch_stats_ab<2>(a, b, w, nb_blocks, gxa, st);
    else
      launch_stats_ab<8>(a, b, w, nb_blocks, gxa, st);
    return hipGetLastError();
  }
  int8_t* const qa = MAXONLY ? w.abar : nullptr;
  int8_t* const qb = MAXONLY ? w.bbar : nullptr;
  if (w.stream_inputs) {
    stats_lines<MAXONLY, true>(a, w.p, w.p_pad, w.q, w.q_pad, w.nch, w.part_e_a, w.part_s_a, qa, st);
    stats_lines<MAXONLY, true>(b, w.r, w.r_pad, w.q, w.q_pad, w.nch, w.part_e_b, w.part_s_b, qb, st);
  } else {
    stats_lines<MAXONLY, false>(a, w.p, w.p_pad, w.q, w.q_pad, w.nch, w.part_e_a, w.part_s_a, qa, st);
    stats_lines<MAXONLY, false>(b, w.r, w.r_pad, w.q, w.q_pad, w.nch, w.part_e_b, w.part_s_b, qb, st);
  }
  return hipGetLastError();
}

static void requant_lines(int8_t* plane, int nlines, int nch, int q_pad, const int* e_line, const int* part_e,
                          hipStream_t st) {
  if (nch == 0 || nlines == 0) return;
  hipLaunchKernelGGL(requant_kernel, dim3(blocks_for(4L * nlines, 256), 4 * nch), dim3(256), 0, st, plane, nlines,
                     nch, q_pad, e_line, part_e);
}

hipError_t launch_fast_scaling(const Operand& a, const Operand& b, const Work& w, hipStream_t st) {
  hipError_t e = launch_stats<false>(a, b, w, st);
  if (e != hipSuccess || w.exp_in_residues) return e;
  const int n = w.p + w.r;
  hipLaunchKernelGGL(fast_exponents_kernel, dim3(blocks_for(n, 4)), dim3(256), 0, st, w.p, w.r, w.nch,
                     w.part_e_a, w.part_s_a, w.part_e_b, w.part_s_b, w.d, w.b, w.tau, w.flags);
  return hipGetLastError();
}

hipError_t launch_accu_bound_inputs(const Operand& a, const Operand& b, const Work& w, hipStream_t st) {
  hipError_t e = launch_stats<true>(a, b, w, st);
  if (e != hipSuccess) return e;
  const int n = w.p + w.r;
  hipLaunchKernelGGL(max_exponents_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, st, w.p, w.r, w.nch,
                     w.part_e_a, w.part_e_b, w.e_row, w.f_col, w.rho, w.gamma);
  requant_lines(w.abar, w.p, w.nch, w.q_pad, w.e_row, w.part_e_a, st);
  requant_lines(w.bbar, w.r, w.nch, w.q_pad, w.f_col, w.part_e_b, st);
  return hipGetLastError();
}

hipError_t launch_accu_exponents(const Work& w, hipStream_t st) {
  const int n = w.p + w.r;
  hipLaunchKernelGGL(accu_exponents_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, st, w.p, w.r, w.e_row,
                     w.f_col, w.rho, w.gamma, w.d, w.b, w.tau, w.flags);
  return hipGetLastError();
}

}  // namespace oz2
