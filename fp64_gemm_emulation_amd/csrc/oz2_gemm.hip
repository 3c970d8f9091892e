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


// Tile: 256 x 256 outputs per workgroup, 4 waves in a 2 x 2 grid, each wave 128 x 128 =
// 8 x 8 blocks of v_mfma_i32_16x16x64_i8 (256 accumulator registers per lane).
//
// K advances in stages of 64 bytes.  Operands go from global memory straight into a ring
// of kStages LDS buffers with global_load_lds_dwordx4 (no staging registers), so up to
// four stages are in flight and the load latency is covered by several stages of MFMAs.
// In LDS each 256 x 64-byte operand tile is stored row-major with its four 16-byte
// chunks XOR-swizzled by bits 2..3 of the row: one load instruction fills 1 KiB
// contiguously (16 rows), and the 16-byte fragment reads of 16 consecutive rows touch 16
// distinct bank groups.  Per stage and wave: MFMAs of the first half of the tile rows;
// wait for the next stage's loads and synchronize; refill the buffer just consumed with
// the stage four ahead; read the next stage's fragments while the second half's MFMAs
// run.
constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 64;
constexpr int kStages = 4;
constexpr int kTileBytes = kBM * kBK;          // 16 KiB per operand per stage
constexpr int kStageBytes = 2 * kTileBytes;    // A then B
constexpr int kLoadsPerStage = 8;              // global_load_lds per wave per stage (4 A + 4 B)
constexpr int kGroupM = 4;  // tile rows per group of the XCD-aware launch order

// Constants of the output reduction R = P mod m for each modulus (index t):
// c16 = 2^16 mod m, inv = RN(1/m) in FP32.
struct ModRed {
  int m;
  int c16;
  float inv;
};
__constant__ ModRed kModRed[kMaxS] = {
#define OZ2_MR(T) {modulus(T), static_cast<int>(pow2_mod(16, modulus(T))), 1.0f / static_cast<float>(modulus(T))}
    OZ2_MR(0),  OZ2_MR(1),  OZ2_MR(2),  OZ2_MR(3),  OZ2_MR(4),  OZ2_MR(5),  OZ2_MR(6),
    OZ2_MR(7),  OZ2_MR(8),  OZ2_MR(9),  OZ2_MR(10), OZ2_MR(11), OZ2_MR(12), OZ2_MR(13),
    OZ2_MR(14), OZ2_MR(15), OZ2_MR(16), OZ2_MR(17), OZ2_MR(18), OZ2_MR(19)
#undef OZ2_MR
};

__device__ __forceinline__ int mad_i24(int a, int b, int c) {
  int d;
  asm("v_mad_i32_i24 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(b), "v"(c));
  return d;
}

// P mod m in [0, m) for |P| < 2^31, 2 <= m <= 256.  For odd m: P = a 2^16 + b gives
// z = a (2^16 mod m) + b = P (mod m) with |z| < 2^23, so round(z / m) is exact from one
// FP32 FMA (z / m is never within 1/(2m) of a half-integer), and z - m round(z/m) is
// the centered residue, moved to [0, m).
__device__ __forceinline__ uint32_t mod_nonneg(int P, const ModRed& mr) {
  if (mr.m == 256) return static_cast<uint32_t>(P) & 0xFFu;
  const int z = mad_i24(P >> 16, mr.c16, P & 0xFFFF);
  const float y = __builtin_fmaf(static_cast<float>(z), mr.inv, 12582912.0f);
  int r = mad_i24(__float_as_int(y), -mr.m, z) + (mr.m << 22);  // low 24 bits of y: 2^22 + round(z/m)
  r += (r >> 31) & mr.m;
  return static_cast<uint32_t>(r);
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

// s_waitcnt with only the vector-memory counter constrained: vmcnt <= N (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] left at their maxima).
#define OZ2_WAIT_VMCNT(N) __builtin_amdgcn_s_waitcnt(((N) & 0xF) | (((N) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

typedef __attribute__((address_space(3))) void* lds_ptr_t;

enum { kEpiMod = 0, kEpiRawMod = 1, kEpiBound = 2 };

template <int EPI>
__global__ __launch_bounds__(256, 1) void gemm_i8_kernel(const int8_t* __restrict__ at, const int8_t* __restrict__ bt,
                                                         long a_plane, long b_plane, int K,
                                                         uint8_t* __restrict__ res, long r_plane, int ldr,
                                                         int32_t* __restrict__ p_dump, int p, int r,
                                                         int* __restrict__ rho, int* __restrict__ gamma,
                                                         int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) int8_t smem[kStages * kStageBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: kept in SGPRs
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int t = blockIdx.z;
  int tile_i, tile_j;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tile_i, tile_j);
  const int i0 = tile_i * kBM;
  const int j0 = tile_j * kBN;

  // DMA: wave w fills rows [64 w + 16 j, +16) of each operand tile, j = 0..3; lane l
  // lands at row 16 j + l / 4, physical chunk l % 4, and so fetches logical chunk
  // (l % 4) ^ ((l / 16) % 4) of that row.  Uniform bases live in SGPRs; each lane keeps
  // one 32-bit offset (a tile spans at most 256 rows of K < 2^17 bytes).
  const int8_t* const ga = at + t * a_plane + static_cast<long>(i0 + 64 * wave) * K;
  const int8_t* const gb = bt + t * b_plane + static_cast<long>(j0 + 64 * wave) * K;
  const unsigned loff = static_cast<unsigned>((lane >> 2) * K + 16 * ((lane & 3) ^ ((lane >> 4) & 3)));
  auto dma = [&](int kbuf, int ksrc) {
    int8_t* sa = smem + (kbuf % kStages) * kStageBytes + wave * 64 * kBK;
    const long k0 = static_cast<long>(ksrc) * kBK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const long rowk = static_cast<long>(16 * j) * K + k0;
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(ga + rowk + loff),
                                       (lds_ptr_t)(sa + j * 16 * kBK), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(gb + rowk + loff),
                                       (lds_ptr_t)(sa + kTileBytes + j * 16 * kBK), 16, 0, 0);
    }
  };

  // fragment reads: row R = 128 w + 16 blk + lane % 16, logical chunk lane / 16
  const int fofs = (lane & 15) * kBK + 16 * ((lane >> 4) ^ ((lane >> 2) & 3));
  const int8_t* const fa0 = smem + wm * 128 * kBK + fofs;
  const int8_t* const fb0 = smem + kTileBytes + wn * 128 * kBK + fofs;

  v4i acc[8][8];
#pragma unroll
  for (int mi = 0; mi < 8; ++mi)
#pragma unroll
    for (int ni = 0; ni < 8; ++ni) acc[mi][ni] = v4i{0, 0, 0, 0};

  v4i fa0r[8], fb0r[8], fa1r[8], fb1r[8];
  auto lread_b = [&](int kt, v4i (&xb)[8]) {
    const int buf = (kt % kStages) * kStageBytes;
#pragma unroll
    for (int ni = 0; ni < 8; ++ni) xb[ni] = *reinterpret_cast<const v4i*>(fb0 + buf + ni * 16 * kBK);
  };
  auto lread_a = [&](int kt, v4i (&xa)[8], int m_lo) {
    const int buf = (kt % kStages) * kStageBytes;
#pragma unroll
    for (int mi = m_lo; mi < m_lo + 4; ++mi) xa[mi] = *reinterpret_cast<const v4i*>(fa0 + buf + mi * 16 * kBK);
  };
  auto mfma_rows = [&](const v4i (&xa)[8], const v4i (&xb)[8], int m_lo) {
#pragma unroll
    for (int mi = m_lo; mi < m_lo + 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 8; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xa[mi], xb[ni], acc[mi][ni], 0, 0, 0);
  };
  auto sync = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
  };

  // K / kBK is a multiple of 4 (the inner dimension is padded to 256), so the stage loop
  // runs in pairs and needs no tail.  The body is branch-free: the refill for stage
  // kt + 4 is always issued, from stage min(kt + 4, nk - 1), into the buffer of stage kt,
  // which nothing reads after the barrier; so exactly two stages of loads are always
  // outstanding behind the one the next barrier needs.
  const int nk = K / kBK;
  // one stage: MFMAs of rows 0..3 with the current fragments; wait for stage kt + 1 and
  // synchronize; refill the buffer of stage kt; read stage kt + 1's B fragments and rows
  // 0..3 of its A fragments; MFMAs of rows 4..7; read rows 4..7 of stage kt + 1's A
  // fragments (covered by the next stage's first half).
  auto stage = [&](int kt, v4i (&ca)[8], v4i (&cb)[8], v4i (&na)[8], v4i (&nb)[8]) {
    mfma_rows(ca, cb, 0);
    __builtin_amdgcn_sched_barrier(0);
    OZ2_WAIT_VMCNT(2 * kLoadsPerStage);
    sync();
    dma(kt, min(kt + 4, nk - 1));
    lread_b(kt + 1, nb);
    lread_a(kt + 1, na, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfma_rows(ca, cb, 4);
    lread_a(kt + 1, na, 4);
  };

  if (nk > 0) {
    // prologue: stages 0..3 in flight (clamped for short K), wait for stage 0
#pragma unroll
    for (int kt = 0; kt < kStages; ++kt) dma(kt, min(kt, nk - 1));
    OZ2_WAIT_VMCNT(3 * kLoadsPerStage);
    sync();
    lread_b(0, fb0r);
    lread_a(0, fa0r, 0);
    lread_a(0, fa0r, 4);
    for (int kt = 0; kt < nk; kt += 2) {
      stage(kt, fa0r, fb0r, fa1r, fb1r);
      stage(kt + 1, fa1r, fb1r, fa0r, fb0r);
    }
    // no LDS DMA may still be in flight when the workgroup's LDS is released
    OZ2_WAIT_VMCNT(0);
  }

  // acc[mi][ni][v] holds P_t[i][j] with
  //   i = i0 + 128 wm + 16 mi + 4 (lane / 16) + v,   j = j0 + 128 wn + 16 ni + lane % 16.
  const int ib = i0 + wm * 128 + 4 * (lane >> 4);
  const int jb = j0 + wn * 128 + (lane & 15);
  if constexpr (EPI == kEpiBound) {
    // rows: max over this wave's 128 columns, then over the 16 lanes sharing lane / 16
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        int mx = 0;
#pragma unroll
        for (int ni = 0; ni < 8; ++ni) mx = max(mx, acc[mi][ni][v]);
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) mx = max(mx, __shfl_xor(mx, off, kWave));
        const int i = ib + mi * 16 + v;
        if ((lane & 15) == 0 && i < p) atomicMax(rho + i, mx);
      }
    }
    // columns: max over this wave's 128 rows
#pragma unroll
    for (int ni = 0; ni < 8; ++ni) {
      int mx = 0;
#pragma unroll
      for (int mi = 0; mi < 8; ++mi)
        mx = max(mx, max(max(acc[mi][ni][0], acc[mi][ni][1]), max(acc[mi][ni][2], acc[mi][ni][3])));
      mx = max(mx, __shfl_xor(mx, 16, kWave));
      mx = max(mx, __shfl_xor(mx, 32, kWave));
      const int j = jb + ni * 16;
      if (lane < 16 && j < r) atomicMax(gamma + j, mx);
    }
  } else {
    const ModRed mr = kModRed[t];
    uint8_t* rt = res + t * r_plane;
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) {
#pragma unroll
      for (int ni = 0; ni < 8; ++ni) {
        const int i = ib + mi * 16;
        const int j = jb + ni * 16;
        const v4i a4 = acc[mi][ni];
        const uint32_t r01 = __builtin_amdgcn_perm(mod_nonneg(a4[1], mr), mod_nonneg(a4[0], mr), 0x0c0c0400u);
        const uint32_t r23 = __builtin_amdgcn_perm(mod_nonneg(a4[3], mr), mod_nonneg(a4[2], mr), 0x0c0c0400u);
        *reinterpret_cast<uint32_t*>(rt + static_cast<long>(j) * ldr + i) = __builtin_amdgcn_perm(r23, r01, 0x05040100u);
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
  const int tiles_n = w.r_pad / kBN;
  dim3 grid(static_cast<unsigned>(tiles_m) * static_cast<unsigned>(tiles_n), 1, planes);
  const long a_plane = static_cast<long>(w.p_pad) * w.q_pad;
  const long b_plane = static_cast<long>(w.r_pad) * w.q_pad;
  const long r_plane = static_cast<long>(w.r_pad) * w.p_pad;
  const int8_t* a = epi == kEpiBound ? w.abar : w.at;
  const int8_t* b = epi == kEpiBound ? w.bbar : w.bt;
  switch (epi) {
    case kEpiMod:
      hipLaunchKernelGGL(gemm_i8_kernel<kEpiMod>, grid, dim3(256), 0, st, a, b, a_plane, b_plane, w.q_pad, w.res,
                         r_plane, w.p_pad, nullptr, w.p, w.r, nullptr, nullptr, tiles_m, tiles_n);
      break;
    case kEpiRawMod:
      hipLaunchKernelGGL(gemm_i8_kernel<kEpiRawMod>, grid, dim3(256), 0, st, a, b, a_plane, b_plane, w.q_pad,
                         w.res, r_plane, w.p_pad, dump.pt, w.p, w.r, nullptr, nullptr, tiles_m, tiles_n);
      break;
    case kEpiBound:
      hipLaunchKernelGGL(gemm_i8_kernel<kEpiBound>, grid, dim3(256), 0, st, a, b, a_plane, b_plane, w.q_pad,
                         nullptr, 0L, w.p_pad, nullptr, w.p, w.r, w.rho, w.gamma, tiles_m, tiles_n);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace oz2
