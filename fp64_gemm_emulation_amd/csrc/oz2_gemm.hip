// oz2_gemm.hip -- the s main INT8 x INT8 -> INT32 GEMMs P_t = A_t B_t on CDNA4 i8 MFMA,
// one batched launch (grid z = modulus index t), with the output reduction
// R_t = P_t mod m_t fused into the epilogue ("Profiling Ozaki II: The Cost Behind Fast
// INT8 GEMMs", Part I section 1: yellow GEMMs and blue output reduction), and the accu
// bound product whose epilogue keeps only row / column maxima (same page, section 2).
// Two kernels: gemm_w8_kernel (8 waves of v_mfma_i32_16x16x64_i8, two per SIMD) for grids
// of at least two 256 x 256 tiles per CU, and gemm_i8_kernel (one wave of
// v_mfma_i32_32x32x32_i8 per SIMD, 256 x 256 or 128 x 128 tiles) for smaller grids and
// the raw P_t validation dump.
//
// Exactness: |A_t|, |B_t| <= 128, so every product is at most 2^14 and every partial sum
// of a length-q dot product stays below q 2^14 < 2^31 for q < 2^17, in any order
// ("Ozaki II supplement", section 1.3).  Longer inner dimensions run as successive
// launches over K-blocks of kKBlock bytes; each later block adds the previous block's
// residues in its epilogue (kEpiModAcc: R_t <- (P_block + R_t) mod m_t).  A block of
// kKBlock = 2^17 is exact: for odd m the residues are at most 127 in magnitude
// (2^17 127^2 < 2^31), and for m = 256 only the low byte is used, which INT32
// wrap-around preserves.  The accu bound product needs no blocking while q 2^12 < 2^31.  Operand planes are int8 in the tile-contiguous
// layout of operand_chunk_offset (rows padded to 256, the inner dimension to 256 with
// zeros), so the kernel needs no bounds checks in the K loop.
#include <type_traits>

#include "oz2_common.hpp"
#include "oz2_internal.hpp"

namespace oz2 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// Tile: 256 x 256 outputs per workgroup, 4 waves in a 2 x 2 grid, each wave 128 x 128 =
// 4 x 4 blocks of v_mfma_i32_32x32x32_i8 (256 accumulator registers per lane).  From one
// wave per SIMD this form keeps the matrix core close to fully busy, where back-to-back
// 16x16x64 MFMAs reach only about half of it.
//
// K advances in stages of 64 bytes (two 32-deep halves).  Each stage tile of each operand
// is a contiguous 16 KiB block in memory, copied into a ring of kStages LDS buffers with
// global_load_lds_dwordx4 (1 KiB per instruction, no staging registers).  Stage X lives
// in buffer X mod kStages and is copied in two parts: its A slice during the second half
// of stage X - kStages, its B slice during the first half of stage X - kStages + 1.  Per
// stage kt and wave:
//   first half:  wait for this half's fragments; 16 MFMAs, with the 8 fragment reads of
//                the second half among the first 8 and the B-slice copies of stage
//                kt + kStages - 1 (into the buffer released at the previous middle barrier)
//                after every second one;
//   middle:      wait for both parts of stage kt + 1 and for the fragments; barrier;
//   second half: 16 MFMAs, with the 8 first-half fragment reads of stage kt + 1 among the
//                first 8 and the A-slice copies of stage kt + kStages (into the buffer of
//                stage kt, released by this barrier) after every second one.
// At most 8 LDS reads are ever outstanding, so every wait is an exact count, and each
// wait falls where the data has had half a stage of MFMAs to arrive.  Spreading the copies
// over both halves, instead of issuing them all right after the barrier, keeps the four
// waves from queueing their MFMAs behind 32 KiB of copies at the same moment: 3% faster
// at n = 8192 and 10% at n = 16384.
constexpr int kBK = kStageK;                    // 64 bytes of the inner dimension per stage
constexpr int kStages = 4;
constexpr int kTileBytes = kStageTile;          // 16 KiB per operand per stage
constexpr int kGroupM = 4;  // tile rows per group of the XCD-aware launch order
constexpr int kKBlock = 1 << 17;                // inner-dimension bytes per launch of the mod GEMM
constexpr long kSmallTileBelow = 2 * 256;       // 256 x 256 tiles (all planes) below which 128 x 128 tiles run
static_assert(static_cast<long>(kKBlock) * 127 * 127 < (1L << 31), "odd-modulus block products fit INT32");
static_assert(kRowPad == 256, "operand stage tiles are 256 rows");
static_assert(kStages == 4, "the copy schedule and its wait counts assume a ring of 4 stages");

// Constants of the output reduction R = P mod m for each modulus (index t).  The
// accumulators start at -h (h = (m - 1) / 2 for odd m, 0 for m = 256), so the epilogue
// sees P' = P - h with |P'| < 2^31:
//   y = RN(P' inv + magic) in FP64, inv = RN(1 / m), magic = 1.5 2^52 - e, is exactly
//       magic + round(P' / m): P' inv lies within 2^-22 / m of P' / m, which for odd m is
//       never closer than 1 / (2m) to a half-integer, and the sum stays in [2^52, 2^53);
//   the low 32 bits of y are then round(P' / m) - e (mod 2^32), and one v_mad_i32_i24
//       gives P' - m (round(P' / m) - e) (mod 2^24), whose low byte, with
//       e = h m^-1 (mod 256), is the centered residue of P' plus h = P mod m, in [0, m).
// Three VALU operations per output (convert, FMA, multiply-add), all at the full vector
// rate: CDNA4 issues FP64 FMAs as fast as unpacked FP32 ones.
struct ModRed {
  int m;
  int h;
  double inv;    // RN(1 / m)
  double magic;  // 1.5 2^52 - e
};

constexpr int half_of(int m) { return (m & 1) ? (m - 1) / 2 : 0; }
constexpr int shift_e(int m) {
  return (m & 1) ? static_cast<int>((static_cast<uint32_t>(half_of(m)) * inv_mod(static_cast<uint32_t>(m) & 255u, 256u)) & 255u)
                 : 0;
}
constexpr ModRed mod_red(int t) {
  return ModRed{modulus(t), half_of(modulus(t)), 1.0 / static_cast<double>(modulus(t)),
                6755399441055744.0 - static_cast<double>(shift_e(modulus(t)))};
}
constexpr bool mod_red_ok() {
  for (int t = 0; t < kMaxS; ++t) {
    const int m = modulus(t);
    if ((m & 1) && (m * shift_e(m)) % 256 != half_of(m)) return false;
  }
  return true;
}
static_assert(mod_red_ok(), "m e = h (mod 256) for every odd modulus");

__constant__ ModRed kModRed[kMaxS] = {
    mod_red(0),  mod_red(1),  mod_red(2),  mod_red(3),  mod_red(4),  mod_red(5),  mod_red(6),
    mod_red(7),  mod_red(8),  mod_red(9),  mod_red(10), mod_red(11), mod_red(12), mod_red(13),
    mod_red(14), mod_red(15), mod_red(16), mod_red(17), mod_red(18), mod_red(19)};

__device__ __forceinline__ int mad_i24(int a, int b, int c) {
  int d;
  asm("v_mad_i32_i24 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(b), "v"(c));
  return d;
}

// Low byte = P mod m for an accumulator holding P' = P - h (odd m); see ModRed.
__device__ __forceinline__ uint32_t mod_byte(int pp, const ModRed& mr) {
  const double y = __builtin_fma(static_cast<double>(pp), mr.inv, mr.magic);
  return static_cast<uint32_t>(mad_i24(static_cast<int>(__double_as_longlong(y)), -mr.m, pp));
}

// Residue bytes of the four rows held in accumulator registers 4 g .. 4 g + 3 of one
// 32 x 32 block, packed little-endian into one word.  prev: residue bytes of the previous
// K-block to add (K-blocked launches), 0 otherwise.  M256: m = 256, where P mod 256 is the
// low byte of P (h = 0).  A template parameter, so that the epilogue loops are straight-line
// code for one modulus kind (a runtime test inside them is compiled into a branch per word).
template <bool M256, bool ADD>
__device__ __forceinline__ uint32_t residue_word(const v16i& a, int g, const ModRed& mr, uint32_t prev) {
  uint32_t b0 = static_cast<uint32_t>(a[4 * g]);
  uint32_t b1 = static_cast<uint32_t>(a[4 * g + 1]);
  uint32_t b2 = static_cast<uint32_t>(a[4 * g + 2]);
  uint32_t b3 = static_cast<uint32_t>(a[4 * g + 3]);
  if constexpr (ADD) {
    b0 += prev & 0xFFu;
    b1 += (prev >> 8) & 0xFFu;
    b2 += (prev >> 16) & 0xFFu;
    b3 += prev >> 24;
  }
  if constexpr (!M256) {
    b0 = mod_byte(static_cast<int>(b0), mr);
    b1 = mod_byte(static_cast<int>(b1), mr);
    b2 = mod_byte(static_cast<int>(b2), mr);
    b3 = mod_byte(static_cast<int>(b3), mr);
  }
  const uint32_t r01 = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
  const uint32_t r23 = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
  return __builtin_amdgcn_perm(r23, r01, 0x05040100u);
}

// Residue word of a 16 x 16 block's accumulator registers (four consecutive rows of one
// column), as residue_word for the 32 x 32 blocks.
template <bool M256>
__device__ __forceinline__ uint32_t residue_word4(const v4i& a, const ModRed& mr) {
  uint32_t b0 = static_cast<uint32_t>(a[0]);
  uint32_t b1 = static_cast<uint32_t>(a[1]);
  uint32_t b2 = static_cast<uint32_t>(a[2]);
  uint32_t b3 = static_cast<uint32_t>(a[3]);
  if constexpr (!M256) {
    b0 = mod_byte(static_cast<int>(b0), mr);
    b1 = mod_byte(static_cast<int>(b1), mr);
    b2 = mod_byte(static_cast<int>(b2), mr);
    b3 = mod_byte(static_cast<int>(b3), mr);
  }
  const uint32_t r01 = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
  const uint32_t r23 = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
  return __builtin_amdgcn_perm(r23, r01, 0x05040100u);
}

// Byte-wise (a + b) mod m of two words of residues in [0, m), m <= 256.
__device__ __forceinline__ uint32_t add_mod_bytes(uint32_t a, uint32_t b, int m) {
  uint32_t out = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    int x = static_cast<int>((a >> (8 * k)) & 0xFFu) + static_cast<int>((b >> (8 * k)) & 0xFFu);
    x -= x >= m ? m : 0;
    out |= static_cast<uint32_t>(x) << (8 * k);
  }
  return out;
}

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own L2.  Give
// every XCD a contiguous range of tiles, and walk that range in groups of kGroupM tile
// rows, so the workgroups resident on one XCD share A_t row panels and B_t column panels.
__device__ __forceinline__ void tile_coords(unsigned wg, int tiles_m, int tiles_n, int& ti, int& tj) {
  const unsigned ntiles = static_cast<unsigned>(tiles_m) * static_cast<unsigned>(tiles_n);
  unsigned id = wg;
  if ((ntiles & 7u) == 0) id = (wg & 7u) * (ntiles >> 3) + (wg >> 3);
  const unsigned group_size = static_cast<unsigned>(kGroupM) * tiles_n;
  const unsigned group = id / group_size;
  const unsigned first_m = group * kGroupM;
  const unsigned gm = min(static_cast<unsigned>(tiles_m) - first_m, static_cast<unsigned>(kGroupM));
  const unsigned in_group = id - group * group_size;
  ti = static_cast<int>(first_m + in_group % gm);
  tj = static_cast<int>(in_group / gm);
}

// s_waitcnt with one counter constrained (gfx9 encoding: vmcnt bits [3:0] and [15:14],
// expcnt [6:4], lgkmcnt [11:8]; the others left at their maxima).
#define OZ2_WAIT_VMCNT(N) __builtin_amdgcn_s_waitcnt(((N) & 0xF) | (((N) >> 4) << 14) | (0x7 << 4) | (0xF << 8))
#define OZ2_WAIT_LGKMCNT(N) __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (((N) & 0xF) << 8))
#define OZ2_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

typedef __attribute__((address_space(3))) void* lds_ptr_t;

enum { kEpiMod = 0, kEpiRawMod = 1, kEpiBound = 2, kEpiModAcc = 3 };

// K: padded inner dimension (row length of the operand planes); stages kt0 .. kt0 + nk - 1
// of it are multiplied.  TB: 32 x 32 MFMA blocks per wave and dimension; the workgroup
// tile is 64 TB x 64 TB (TB = 4: 256 x 256, one workgroup per CU; TB = 2: 128 x 128 for
// small products, two workgroups per CU so that one's epilogue overlaps the other's
// MFMAs).  A 128-row tile reads one half of the 256-row stage tiles, which is contiguous.
template <int EPI, int TB>
__global__ __launch_bounds__(256, TB == 4 ? 1 : 2) void gemm_i8_kernel(
    const int8_t* __restrict__ at, const int8_t* __restrict__ bt, long a_plane, long b_plane, int K, int kt0, int nk,
    uint8_t* __restrict__ res, long r_plane, int ldr, int32_t* __restrict__ p_dump, int p, int r,
    int* __restrict__ rho, int* __restrict__ gamma, int tiles_m, int tiles_n) {
  static_assert(TB == 4 || TB == 2, "tile shapes: 256 x 256 or 128 x 128");
  constexpr int WT = 32 * TB;                // wave tile edge
  constexpr int BT = 2 * WT;                 // workgroup tile edge
  constexpr int kSlice = BT * kBK;           // bytes of one operand per stage in LDS
  constexpr int kStageLds = 2 * kSlice;      // A then B
  constexpr int kCopies = kSlice / 4 / 1024; // 1 KiB copies per wave and operand per stage (= TB)
  constexpr int kLoads = 2 * kCopies;        // outstanding copy instructions per wave per stage
  constexpr int kPairs = TB * TB / 2;        // MFMA pairs per 32-deep half
  constexpr int kFeed = kPairs / 2 > 0 ? kPairs / 2 : 1;  // pairs that carry the reads / copies
  constexpr int kReadsPer = 2 * TB / kFeed;  // fragment reads issued after each of those pairs
  constexpr int kCopyEvery = kPairs / kCopies;  // MFMA pairs per copy within one half
  __shared__ __attribute__((aligned(1024))) int8_t smem[kStages * kStageLds];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: kept in SGPRs
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int t = blockIdx.z;
  int tile_i, tile_j;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tile_i, tile_j);
  const int i0 = tile_i * BT;
  const int j0 = tile_j * BT;

  // Copies: the tile's rows i0 .. i0 + BT - 1 lie in 256-row block i0 / 256 at byte offset
  // 64 (i0 % 256) of each 16 KiB stage tile.  Wave w moves bytes [kSlice/4 w + 1024 g, +1024)
  // of the tile's slice (g < kCopies for A, again for B); lane l lands at byte 16 l.
  const long a_base = static_cast<long>(i0 / kRowPad) * kRowPad * K + (i0 % kRowPad) * kBK;
  const long b_base = static_cast<long>(j0 / kRowPad) * kRowPad * K + (j0 % kRowPad) * kBK;
  const int8_t* const ga = at + t * a_plane + a_base + static_cast<long>(kt0) * kTileBytes + wave * (kSlice / 4) + 16 * lane;
  const int8_t* const gb = bt + t * b_plane + b_base + static_cast<long>(kt0) * kTileBytes + wave * (kSlice / 4) + 16 * lane;
  auto copy1 = [&](int kbuf, int ksrc, int g) {
    const int c = g % kCopies;
    const long src = static_cast<long>(ksrc) * kTileBytes + c * 1024;
    int8_t* dst = smem + (kbuf % kStages) * kStageLds + wave * (kSlice / 4) + c * 1024;
    if (g < kCopies)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(ga + src), (lds_ptr_t)dst, 16, 0, 0);
    else
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(gb + src), (lds_ptr_t)(dst + kSlice), 16, 0, 0);
  };

  // Accumulators start at -h for the mod epilogues (see ModRed), at 0 for the bound.
  // The modulus constants are loaded here and pinned in scalar registers: loaded in the
  // epilogue, their latency would stall every wave at the end of every tile.
  ModRed mr{0, 0, 0.0, 0.0};
  if constexpr (EPI != kEpiBound) {
    mr = kModRed[t];
    asm volatile("" : "+s"(mr.m), "+s"(mr.h), "+s"(mr.inv), "+s"(mr.magic));
  }
  const int init = -mr.h;
  v16i acc[TB][TB];
#pragma unroll
  for (int mb = 0; mb < TB; ++mb)
#pragma unroll
    for (int nb = 0; nb < TB; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mb][nb][v] = init;

  // Fragment of a 32-row block for one 32-deep half: lane l reads row 32 blk + l % 32,
  // logical 16-byte chunk 2 half + l / 32 (the same for A and B, so the K positions that
  // one MFMA pairs up agree).  f0 holds the first half's TB A and TB B fragments, f1 the
  // second half's.
  const int frow = lane & 31;
  const int fsw = operand_swizzle(frow & 15);
  const int fk = lane >> 5;
  const int8_t* const fa = smem + wm * WT * kBK + frow * kBK;
  const int8_t* const fb = smem + kSlice + wn * WT * kBK + frow * kBK;
  v4i f0[2 * TB], f1[2 * TB];
  auto read1 = [&](int kbuf, int half, v4i (&x)[2 * TB], int g) {
    const int off = (kbuf % kStages) * kStageLds + 16 * ((2 * half + fk) ^ fsw);
    if (g < TB) x[g] = *reinterpret_cast<const v4i*>(fa + off + g * 32 * kBK);
    else x[g] = *reinterpret_cast<const v4i*>(fb + off + (g - TB) * 32 * kBK);
  };
  // MFMA pair g of a half: blocks (g / (TB/2), 2 (g % (TB/2))) and the next column block
  auto mfma2 = [&](const v4i (&x)[2 * TB], int g) {
    const int mb = g / (TB / 2), nb = 2 * (g % (TB / 2));
    acc[mb][nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(x[mb], x[TB + nb], acc[mb][nb], 0, 0, 0);
    acc[mb][nb + 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(x[mb], x[TB + nb + 1], acc[mb][nb + 1], 0, 0, 0);
  };

  if (nk > 0) {
    // Prologue: stages 0..kStages-2 and the A slice of stage kStages-1 in flight (clamped
    // to the last stage for short K), wait for stage 0, read its first-half fragments.
#pragma unroll
    for (int kt = 0; kt < kStages - 1; ++kt)
#pragma unroll
      for (int g = 0; g < kLoads; ++g) copy1(kt, min(kt, nk - 1), g);
#pragma unroll
    for (int g = 0; g < kCopies; ++g) copy1(kStages - 1, min(kStages - 1, nk - 1), g);
    OZ2_WAIT_VMCNT((kStages - 2) * kLoads + kCopies);
    __builtin_amdgcn_s_barrier();
    OZ2_SCHED_FENCE();
#pragma unroll
    for (int g = 0; g < 2 * TB; ++g) read1(0, 0, f0, g);
    OZ2_SCHED_FENCE();
    // The body is branch-free: every copy is always issued, its source stage clamped to
    // nk - 1, into a buffer that nothing reads any more (the B slice into the buffer of
    // stage kt - 1, the A slice into that of stage kt, after the barriers that end their
    // reads).  When stage kt + 1 is waited for in the middle of stage kt, the younger
    // copies are exactly both parts of stages kt + 2 and kt + 3 (kStages = 4): 2 kLoads
    // instructions.  Past the last stage, the first-half reads fetch a buffer that is not
    // used again.
    for (int kt = 0; kt < nk; ++kt) {
      OZ2_WAIT_LGKMCNT(0);
      OZ2_SCHED_FENCE();
#pragma unroll
      for (int g = 0; g < kPairs; ++g) {
        mfma2(f0, g);
        if (g < kFeed) {
#pragma unroll
          for (int u = 0; u < kReadsPer; ++u) read1(kt, 1, f1, kReadsPer * g + u);
        }
        if (g % kCopyEvery == kCopyEvery - 1)
          copy1(kt + kStages - 1, min(kt + kStages - 1, nk - 1), kCopies + g / kCopyEvery);
        OZ2_SCHED_FENCE();
      }
      OZ2_WAIT_VMCNT(2 * kLoads);
      OZ2_WAIT_LGKMCNT(0);
      OZ2_SCHED_FENCE();
      __builtin_amdgcn_s_barrier();
      OZ2_SCHED_FENCE();
      const int kn = min(kt + kStages, nk - 1);
#pragma unroll
      for (int g = 0; g < kPairs; ++g) {
        mfma2(f1, g);
        if (g < kFeed) {
#pragma unroll
          for (int u = 0; u < kReadsPer; ++u) read1(kt + 1, 0, f0, kReadsPer * g + u);
        }
        if (g % kCopyEvery == kCopyEvery - 1) copy1(kt, kn, g / kCopyEvery);
        OZ2_SCHED_FENCE();
      }
    }
    // no LDS copy may still be in flight when the workgroup's LDS is released
    OZ2_WAIT_VMCNT(0);
    OZ2_WAIT_LGKMCNT(0);
  }

  // acc[mb][nb][v] holds P_t[i][j] (minus h in the mod epilogues) with
  //   i = i0 + WT wm + 32 mb + 8 (v / 4) + 4 (lane / 32) + v % 4,
  //   j = j0 + WT wn + 32 nb + lane % 32.
  const int ib = i0 + wm * WT + 4 * (lane >> 5);
  const int jb = j0 + wn * WT + (lane & 31);
  if constexpr (EPI == kEpiBound) {
    // rows: max over this wave's columns, then over the 32 lanes sharing lane / 32
#pragma unroll
    for (int mb = 0; mb < TB; ++mb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        int mx = 0;
#pragma unroll
        for (int nb = 0; nb < TB; ++nb) mx = max(mx, acc[mb][nb][v]);
#pragma unroll
        for (int off = 16; off > 0; off >>= 1) mx = max(mx, __shfl_xor(mx, off, kWave));
        const int i = ib + mb * 32 + 8 * (v >> 2) + (v & 3);
        if ((lane & 31) == 0 && i < p) atomicMax(rho + i, mx);
      }
    }
    // columns: max over this wave's rows
#pragma unroll
    for (int nb = 0; nb < TB; ++nb) {
      int mx = 0;
#pragma unroll
      for (int mb = 0; mb < TB; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = max(mx, acc[mb][nb][v]);
      mx = max(mx, __shfl_xor(mx, 32, kWave));
      const int j = jb + nb * 32;
      if (lane < 32 && j < r) atomicMax(gamma + j, mx);
    }
  } else {
    uint8_t* rt = res + t * r_plane;
    const bool m256 = mr.m == 256;
    if constexpr (EPI == kEpiMod) {
      // The tile's BT x BT residue bytes go through LDS (the copy ring is free once every
      // wave has passed its K loop and waited for its own copies) so that every store
      // instruction writes whole 256-byte column segments: a lane's own words cover 32
      // columns 8 bytes at a time.  Staging layout: word (il / 4) of tile column jl at
      // word WC jl + ((il / 4) xor (jl mod 32)), so the 32 lanes of a half-wave, which hold
      // 32 consecutive columns, write 32 distinct banks; a 16-byte read of logical chunk c
      // finds its 4 words in chunk c xor ((jl mod 32) / 4), permuted by xor (jl mod 4).
      constexpr int WC = BT / 4;            // words per tile column
      static_assert(WC >= 32 && BT * BT <= kStages * kStageLds, "staging fits the ring");
      uint32_t* const stage = reinterpret_cast<uint32_t*>(smem);
      __builtin_amdgcn_s_barrier();
      const int jl0 = wn * WT + (lane & 31);
      const int wl0 = (wm * WT + 4 * (lane >> 5)) >> 2;
      auto stage_all = [&](auto m256) {
#pragma unroll
        for (int mb = 0; mb < TB; ++mb)
#pragma unroll
          for (int nb = 0; nb < TB; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int jl = jl0 + 32 * nb;
              const int wl = wl0 + 8 * mb + 2 * g;
              stage[WC * jl + (wl ^ (jl & 31))] = residue_word<decltype(m256)::value, false>(acc[mb][nb], g, mr, 0u);
            }
      };
      if (m256)
        stage_all(std::true_type{});
      else
        stage_all(std::false_type{});
      __syncthreads();
      constexpr int kTpc = BT / 16;         // threads per column (16 bytes each)
      constexpr int kCols = 256 / kTpc;     // columns per pass of the workgroup
      const int c = tid % kTpc;
#pragma unroll 4
      for (int pass = 0; pass < BT / kCols; ++pass) {
        const int jl = pass * kCols + tid / kTpc;
        const v4i d = *reinterpret_cast<const v4i*>(stage + WC * jl + 4 * (c ^ ((jl & 31) >> 2)));
        const int sw = jl & 3;              // logical word k sits at position k xor sw
        int x0 = d[0], x1 = d[1], x2 = d[2], x3 = d[3];
        if (sw & 1) {
          const int y0 = x0, y2 = x2;
          x0 = x1; x1 = y0; x2 = x3; x3 = y2;
        }
        if (sw & 2) {
          const int y0 = x0, y1 = x1;
          x0 = x2; x1 = x3; x2 = y0; x3 = y1;
        }
        *reinterpret_cast<v4i*>(rt + static_cast<long>(j0 + jl) * ldr + i0 + 16 * c) = v4i{x0, x1, x2, x3};
      }
    } else {
      // validation dump and K-blocked launches: direct 4-byte stores
      auto store_all = [&](auto m256) {
#pragma unroll
      for (int mb = 0; mb < TB; ++mb) {
#pragma unroll
        for (int nb = 0; nb < TB; ++nb) {
          const int j = jb + nb * 32;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int i = ib + mb * 32 + 8 * g;
            uint32_t* const rp = reinterpret_cast<uint32_t*>(rt + static_cast<long>(j) * ldr + i);
            uint32_t prev = 0u;
            if constexpr (EPI == kEpiModAcc) prev = *rp;
            *rp = residue_word<decltype(m256)::value, EPI == kEpiModAcc>(acc[mb][nb], g, mr, prev);
            if constexpr (EPI == kEpiRawMod) {
              if (j < r) {
                int32_t* dst = p_dump + (static_cast<long>(t) * r + j) * p;
#pragma unroll
                for (int v = 0; v < 4; ++v)
                  if (i + v < p) dst[i + v] = acc[mb][nb][4 * g + v] + mr.h;
              }
            }
          }
        }
      }
      };
      if (m256)
        store_all(std::true_type{});
      else
        store_all(std::false_type{});
    }
  }
}

// The mod GEMM for large grids on v_mfma_i32_16x16x64_i8: 256 x 256 outputs per
// workgroup, 8 waves (two per SIMD) in a 2 x 4 grid, each 128 x 64 outputs = 8 x 4 blocks
// of 16 x 16 (128 accumulator registers, so two waves fit a SIMD and interleave their
// MFMAs).  Under the board's power limit this form sustains more int8 operations per
// second than one wave of 32x32x32 per SIMD: it reads and writes half the accumulator bytes
// per multiply-add.  One stage (64 bytes of K) is one MFMA step for all 32 blocks.  Per
// stage kt and wave: wait for this stage's fragments and for the copies of stage kt + 1;
// barrier (after which nothing reads the buffer of stage kt); 32 MFMAs with the 12
// fragment reads of stage kt + 1 after every second one of the first 24, and the 4 copies
// of stage kt + kStages into the buffer of stage kt after MFMAs 4, 12, 20, 28.  The
// younger copies when stage kt + 1 is waited for are those of stages kt + 2 and kt + 3.
// Fragments: lane l reads row 16 b + l % 16 at logical chunk l / 16 of the stage (the
// same for A and B, so the K positions one MFMA pairs up agree); the operand swizzle puts
// the 16 rows of each chunk in distinct bank groups.  Accumulator register v of lane l of
// a block holds row 4 (l / 16) + v, column l % 16.
// EPI: kEpiMod (residues R_t), kEpiModAcc (a later K-block: R_t <- (P_block + R_t) mod m_t)
// or kEpiBound (the accu bound product: row and column maxima of the single plane,
// accumulators from 0).  Stages kt0 .. kt0 + nk - 1 of the inner dimension are multiplied.
template <int EPI>
__global__ __launch_bounds__(512, 1) void gemm_w8_kernel(const int8_t* __restrict__ at, const int8_t* __restrict__ bt,
                                                         long a_plane, long b_plane, int K, int kt0, int nk,
                                                         uint8_t* __restrict__ res, long r_plane, int ldr,
                                                         int* __restrict__ rho, int* __restrict__ gamma, int p, int r,
                                                         int tiles_m, int tiles_n) {
  static_assert(EPI == kEpiMod || EPI == kEpiModAcc || EPI == kEpiBound, "epilogues of the 8-wave GEMM");
  constexpr int BT = 256;
  constexpr int kSlice = BT * kBK;             // 16 KiB per operand per stage
  constexpr int kStageLds = 2 * kSlice;        // A then B
  constexpr int kWaves = 8;
  constexpr int kCopiesW = kStageLds / 1024 / kWaves;  // 1 KiB copies per wave per stage (4)
  constexpr int MB = 8, NB = 4;                // 16 x 16 blocks per wave
  constexpr int kFr = MB + NB;                 // fragment reads per wave per stage (12)
  static_assert(kCopiesW == 4 && kStages == 4, "copy schedule and wait counts");
  __shared__ __attribute__((aligned(1024))) int8_t smem[kStages * kStageLds];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Waves w and w + 4 share a SIMD (waves go to SIMDs round-robin) and interleave their
  // MFMAs there; giving them the same 128 rows (wm) and different columns lets the A
  // operand the matrix core sees stay unchanged across both waves' MFMAs of one block row.
  // Under the board's power limit, fewer operand bits switching per MFMA is clock: with the
  // block order below, 1.3% shorter GEMM stage than partners sharing columns with a
  // row-major order (n = 8192, s = 14).
  const int wm = wave & 1;                     // rows 128 wm
  const int wn = wave >> 1;                    // columns 64 wn
  const int t = blockIdx.z;
  int tile_i, tile_j;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tile_i, tile_j);
  const int i0 = tile_i * BT;
  const int j0 = tile_j * BT;
  ModRed mr{0, 0, 0.0, 0.0};
  if constexpr (EPI != kEpiBound) {
    mr = kModRed[t];
    asm volatile("" : "+s"(mr.m), "+s"(mr.h), "+s"(mr.inv), "+s"(mr.magic));
  }

  // Copies: waves 0-3 move the A slice, waves 4-7 the B slice; wave w moves bytes
  // [4096 (w mod 4) + 1024 c, +1024) of it, lane l at byte 16 l.
  const int8_t* const gsrc = (wave < 4 ? at + t * a_plane + static_cast<long>(i0) * K
                                       : bt + t * b_plane + static_cast<long>(j0) * K) +
                             static_cast<long>(kt0) * kTileBytes + (wave & 3) * 4096 + 16 * lane;
  int8_t* const gdst = smem + (wave >= 4 ? kSlice : 0) + (wave & 3) * 4096;
  auto copy1 = [&](int kbuf, int ksrc, int c) {
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(gsrc + static_cast<long>(ksrc) * kTileBytes + c * 1024),
                                     (lds_ptr_t)(gdst + (kbuf % kStages) * kStageLds + c * 1024), 16, 0, 0);
  };
  const int frow = lane & 15;
  const int fch = (lane >> 4) ^ operand_swizzle(frow);
  const int8_t* const fa = smem + (wm * 128 + frow) * kBK + 16 * fch;
  const int8_t* const fb = smem + kSlice + (wn * 64 + frow) * kBK + 16 * fch;
  auto read1 = [&](int kbuf, v4i (&x)[kFr], int g) {
    const int off = (kbuf % kStages) * kStageLds;
    if (g < MB) x[g] = *reinterpret_cast<const v4i*>(fa + off + g * 16 * kBK);
    else x[g] = *reinterpret_cast<const v4i*>(fb + off + (g - MB) * 16 * kBK);
  };
  v4i acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = v4i{-mr.h, -mr.h, -mr.h, -mr.h};
  v4i x0[kFr], x1[kFr];
  // One stage: MFMAs on x, reads of stage kt + 1 into y, copies of stage kt + kStages.
  auto stage = [&](int kt, v4i (&x)[kFr], v4i (&y)[kFr]) {
    OZ2_WAIT_LGKMCNT(0);
    OZ2_WAIT_VMCNT(2 * kCopiesW);
    OZ2_SCHED_FENCE();
    __builtin_amdgcn_s_barrier();
    OZ2_SCHED_FENCE();
    const int kn = min(kt + kStages, nk - 1);
#pragma unroll
    for (int u = 0; u < MB * NB; ++u) {
      // block rows in order, the columns of every other row reversed (a snake): each step
      // changes one operand fragment, and the B fragment stays across a row change
      const int mb = u / NB, nb = (mb & 1) ? NB - 1 - u % NB : u % NB;
      acc[mb][nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(x[mb], x[MB + nb], acc[mb][nb], 0, 0, 0);
      if (u % 2 == 1 && u / 2 < kFr) read1(kt + 1, y, u / 2);
      if (u % 8 == 4) copy1(kt, kn, u / 8);
      OZ2_SCHED_FENCE();
    }
  };

  if (nk > 0) {
#pragma unroll
    for (int kt = 0; kt < kStages; ++kt)
#pragma unroll
      for (int c = 0; c < kCopiesW; ++c) copy1(kt, min(kt, nk - 1), c);
    OZ2_WAIT_VMCNT((kStages - 1) * kCopiesW);
    __builtin_amdgcn_s_barrier();
    OZ2_SCHED_FENCE();
#pragma unroll
    for (int g = 0; g < kFr; ++g) read1(0, x0, g);
    OZ2_SCHED_FENCE();
    // nk is a multiple of kStages (the inner dimension is padded to 256): even
    for (int kt = 0; kt < nk; kt += 2) {
      stage(kt, x0, x1);
      stage(kt + 1, x1, x0);
    }
    // Copies still in flight now are at most those issued in the last two stages, into the
    // buffers of stages nk - 2 and nk - 1; the mod epilogue stages its residues through the
    // other two and waits for these only after that.
    OZ2_WAIT_VMCNT(2 * kCopiesW);
    OZ2_WAIT_LGKMCNT(0);
  }

  if constexpr (EPI == kEpiBound) {
    OZ2_WAIT_VMCNT(0);
    // rows: max over this wave's 4 column blocks, then over the 16 lanes of each row group
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        int mx = 0;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) mx = max(mx, acc[mb][nb][v]);
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) mx = max(mx, __shfl_xor(mx, off, kWave));
        const int i = i0 + wm * 128 + 16 * mb + 4 * (lane >> 4) + v;
        if ((lane & 15) == 0 && i < p) atomicMax(rho + i, mx);
      }
    }
    // columns: max over this wave's 8 row blocks and 4 registers, then over the 4 row groups
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      int mx = 0;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int v = 0; v < 4; ++v) mx = max(mx, acc[mb][nb][v]);
      mx = max(mx, __shfl_xor(mx, 16, kWave));
      mx = max(mx, __shfl_xor(mx, 32, kWave));
      const int j = j0 + wn * 64 + 16 * nb + (lane & 15);
      if (lane < 16 && j < r) atomicMax(gamma + j, mx);
    }
    return;
  }
  // Epilogue: residue words through the first two stage buffers of the LDS ring (those of
  // stages nk - 4 and nk - 3, whose copies have landed) as in gemm_i8_kernel, so that every
  // store instruction writes whole 256-byte column segments.
  constexpr int WC = BT / 4;
  static_assert(BT * BT <= 2 * kStageLds, "staging fits the first two stage buffers");
  uint32_t* const stg = reinterpret_cast<uint32_t*>(smem);
  __builtin_amdgcn_s_barrier();
  const int jl0 = wn * 64 + (lane & 15);
  const int wl0 = wm * 32 + (lane >> 4);
  auto stage_all = [&](auto m256) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int jl = jl0 + 16 * nb;
        const int wl = wl0 + 4 * mb;
        stg[WC * jl + (wl ^ (jl & 31))] = residue_word4<decltype(m256)::value>(acc[mb][nb], mr);
      }
  };
  if (mr.m == 256)
    stage_all(std::true_type{});
  else
    stage_all(std::false_type{});
  // the last copies have landed before anything leaves the LDS ring (and before the
  // workgroup's LDS can be released); no global store is in flight yet
  OZ2_WAIT_VMCNT(0);
  __syncthreads();
  uint8_t* const rt = res + t * r_plane;
  constexpr int kTpc = BT / 16;                // threads per column
  constexpr int kCols = 512 / kTpc;            // columns per pass
  constexpr int kPasses = BT / kCols;
  const int c = tid % kTpc;
  // all reads first: their latencies overlap instead of preceding one store each
  v4i d[kPasses];
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int jl = pass * kCols + tid / kTpc;
    d[pass] = *reinterpret_cast<const v4i*>(stg + WC * jl + 4 * (c ^ ((jl & 31) >> 2)));
  }
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int jl = pass * kCols + tid / kTpc;
    const int sw = jl & 3;
    int x0w = d[pass][0], x1w = d[pass][1], x2w = d[pass][2], x3w = d[pass][3];
    if (sw & 1) {
      const int y0 = x0w, y2 = x2w;
      x0w = x1w; x1w = y0; x2w = x3w; x3w = y2;
    }
    if (sw & 2) {
      const int y0 = x0w, y1 = x1w;
      x0w = x2w; x1w = x3w; x2w = y0; x3w = y1;
    }
    v4i* const dst = reinterpret_cast<v4i*>(rt + static_cast<long>(j0 + jl) * ldr + i0 + 16 * c);
    if constexpr (EPI == kEpiModAcc) {
      // add the previous K-blocks' residues byte by byte: both are below m, one subtraction
      const v4i prev = *dst;
      x0w = static_cast<int>(add_mod_bytes(static_cast<uint32_t>(x0w), static_cast<uint32_t>(prev[0]), mr.m));
      x1w = static_cast<int>(add_mod_bytes(static_cast<uint32_t>(x1w), static_cast<uint32_t>(prev[1]), mr.m));
      x2w = static_cast<int>(add_mod_bytes(static_cast<uint32_t>(x2w), static_cast<uint32_t>(prev[2]), mr.m));
      x3w = static_cast<int>(add_mod_bytes(static_cast<uint32_t>(x3w), static_cast<uint32_t>(prev[3]), mr.m));
    }
    *dst = v4i{x0w, x1w, x2w, x3w};
  }
}

template <int EPI, int TB>
static void launch_tile(dim3 grid, hipStream_t st, const int8_t* a, const int8_t* b, long a_plane, long b_plane, int K,
                        int kt0, int nk, uint8_t* res, long r_plane, int ldr, int32_t* pd, int p, int r, int* rho,
                        int* gamma, int tiles_m, int tiles_n) {
  hipLaunchKernelGGL((gemm_i8_kernel<EPI, TB>), grid, dim3(256), 0, st, a, b, a_plane, b_plane, K, kt0, nk, res,
                     r_plane, ldr, pd, p, r, rho, gamma, tiles_m, tiles_n);
}

template <int TB>
static hipError_t launch_gemm_tb(const Work& w, int epi, const DumpPtrs& dump, hipStream_t st) {
  constexpr int BT = 64 * TB;
  const int planes = epi == kEpiBound ? 1 : w.s;
  const int tiles_m = w.p_pad / BT;
  const int tiles_n = w.r_pad / BT;
  dim3 grid(static_cast<unsigned>(tiles_m) * static_cast<unsigned>(tiles_n), 1, planes);
  const long a_plane = w.at_plane;
  const long b_plane = w.bt_plane;
  const long r_plane = w.res_plane;
  const int nk = w.q_pad / kBK;
  if (epi == kEpiBound) {
    if constexpr (TB == 4)
      hipLaunchKernelGGL(gemm_w8_kernel<kEpiBound>, grid, dim3(512), 0, st, w.abar, w.bbar, a_plane, b_plane, w.q_pad,
                         0, nk, nullptr, 0L, w.p_pad, w.rho, w.gamma, w.p, w.r, tiles_m, tiles_n);
    else
      launch_tile<kEpiBound, TB>(grid, st, w.abar, w.bbar, a_plane, b_plane, w.q_pad, 0, nk, nullptr, 0L, w.p_pad,
                                 nullptr, w.p, w.r, w.rho, w.gamma, tiles_m, tiles_n);
    return hipGetLastError();
  }
  if (epi != kEpiMod && epi != kEpiRawMod) return hipErrorInvalidValue;
  // the raw P_t dump covers one block only (the entry points refuse it for longer q)
  constexpr int kBlockStages = kKBlock / kBK;
  if (epi == kEpiRawMod && nk > kBlockStages) return hipErrorInvalidValue;
  for (int kt0 = 0; kt0 == 0 || kt0 < nk; kt0 += kBlockStages) {
    const int nkb = nk - kt0 < kBlockStages ? nk - kt0 : kBlockStages;
    if (kt0 > 0 && TB == 4)
      hipLaunchKernelGGL(gemm_w8_kernel<kEpiModAcc>, grid, dim3(512), 0, st, w.at, w.bt, a_plane, b_plane, w.q_pad, kt0,
                         nkb, w.res, r_plane, w.p_pad, nullptr, nullptr, w.p, w.r, tiles_m, tiles_n);
    else if (kt0 > 0)
      launch_tile<kEpiModAcc, TB>(grid, st, w.at, w.bt, a_plane, b_plane, w.q_pad, kt0, nkb, w.res, r_plane, w.p_pad,
                                  nullptr, w.p, w.r, nullptr, nullptr, tiles_m, tiles_n);
    else if (epi == kEpiRawMod)
      launch_tile<kEpiRawMod, TB>(grid, st, w.at, w.bt, a_plane, b_plane, w.q_pad, 0, nkb, w.res, r_plane, w.p_pad,
                                  dump.pt, w.p, w.r, nullptr, nullptr, tiles_m, tiles_n);
    else if constexpr (TB == 4)
      hipLaunchKernelGGL(gemm_w8_kernel<kEpiMod>, grid, dim3(512), 0, st, w.at, w.bt, a_plane, b_plane, w.q_pad, 0,
                         nkb, w.res, r_plane, w.p_pad, nullptr, nullptr, w.p, w.r, tiles_m, tiles_n);
    else
      launch_tile<kEpiMod, TB>(grid, st, w.at, w.bt, a_plane, b_plane, w.q_pad, 0, nkb, w.res, r_plane, w.p_pad,
                               nullptr, w.p, w.r, nullptr, nullptr, tiles_m, tiles_n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// 256 x 256 tiles (gemm_w8_kernel for the mod, K-block and bound epilogues, gemm_i8_kernel
// for the raw P_t dump) unless that grid gives fewer
// than two workgroups per CU, where the exposed per-tile prologue / epilogue and the
// partly empty last round dominate and the 128 x 128-tile gemm_i8_kernel runs.
hipError_t launch_gemm(const Work& w, int epi, const DumpPtrs& dump, hipStream_t st) {
  const long planes = epi == kEpiBound ? 1 : w.s;
  const long big_tiles = static_cast<long>(w.p_pad / 256) * (w.r_pad / 256) * planes;
  if (big_tiles < kSmallTileBelow) return launch_gemm_tb<2>(w, epi, dump, st);
  return launch_gemm_tb<4>(w, epi, dump, st);
}

}  // namespace oz2
