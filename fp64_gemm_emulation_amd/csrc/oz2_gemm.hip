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

// Tile: 256 x 256 outputs per workgroup, 4 waves in a 2 x 2 grid, each wave 128 x 128 =
// 8 x 8 blocks of v_mfma_i32_16x16x64_i8 (256 accumulator registers per lane).  K advances
// in stages of 64 bytes held in a double-buffered LDS ring; the next stage is fetched
// into registers while the current one feeds the MFMAs, so one barrier per stage
// suffices.  LDS rows are padded to 80 bytes: the 16-byte fragment reads of 16
// consecutive rows then fall on 16 distinct 16-byte bank groups.
constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 64;
constexpr int kStage16 = kBM * kBK / 16 / 256;  // 16-byte chunks per thread per operand
constexpr int kPitch = kBK + 16;
constexpr int kStageBytes = (kBM + kBN) * kPitch;
constexpr int kGroupM = 4;  // tile rows per group of the XCD-aware launch order

// P mod m in [0, m) for |P| < 2^31 and 2 <= m <= 256.
__device__ __forceinline__ uint32_t mod_nonneg(int P, int m, double invm) {
  if (m == 256) return static_cast<uint32_t>(P) & 0xFFu;
  const int qt = static_cast<int>(floor(static_cast<double>(P) * invm));
  int rr = P - qt * m;  // off by at most one multiple of m
  rr += rr < 0 ? m : 0;
  rr -= rr >= m ? m : 0;
  return static_cast<uint32_t>(rr);
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

enum { kEpiMod = 0, kEpiRawMod = 1, kEpiBound = 2 };

template <int EPI>
__global__ __launch_bounds__(256, 1) void gemm_i8_kernel(const int8_t* __restrict__ at, const int8_t* __restrict__ bt,
                                                         long a_plane, long b_plane, int K,
                                                         uint8_t* __restrict__ res, long r_plane, int ldr,
                                                         int32_t* __restrict__ p_dump, int p, int r,
                                                         int* __restrict__ rho, int* __restrict__ gamma,
                                                         int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) int8_t smem[2 * kStageBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int t = blockIdx.z;
  int tile_i, tile_j;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tile_i, tile_j);
  const int i0 = tile_i * kBM;
  const int j0 = tile_j * kBN;
  const int8_t* ag = at + t * a_plane + static_cast<long>(i0) * K;
  const int8_t* bg = bt + t * b_plane + static_cast<long>(j0) * K;

  // staging: thread copies 16-byte chunks (row srow + kRowStep h, column scol) of both operands
  constexpr int kChunksPerRow = kBK / 16;
  constexpr int kRowStep = 256 / kChunksPerRow;
  const int srow = tid / kChunksPerRow;
  const int scol = (tid % kChunksPerRow) * 16;
  const int8_t* ga = ag + static_cast<long>(srow) * K + scol;
  const int8_t* gb = bg + static_cast<long>(srow) * K + scol;
  const long gstep = static_cast<long>(kRowStep) * K;
  int8_t* const la = smem + srow * kPitch + scol;
  int8_t* const lb = smem + kBM * kPitch + srow * kPitch + scol;

  v4i acc[8][8];
#pragma unroll
  for (int mi = 0; mi < 8; ++mi)
#pragma unroll
    for (int ni = 0; ni < 8; ++ni) acc[mi][ni] = v4i{0, 0, 0, 0};

  const int frow = lane & 15;
  const int fk = (lane >> 4) * 16;
  const int8_t* const fa0 = smem + (wm * 128 + frow) * kPitch + fk;
  const int8_t* const fb0 = smem + kBM * kPitch + (wn * 128 + frow) * kPitch + fk;

  const int nk = K / kBK;
  v4i ra[kStage16], rb[kStage16];
  if (nk > 0) {
#pragma unroll
    for (int h = 0; h < kStage16; ++h) {
      ra[h] = *reinterpret_cast<const v4i*>(ga + h * gstep);
      rb[h] = *reinterpret_cast<const v4i*>(gb + h * gstep);
    }
#pragma unroll
    for (int h = 0; h < kStage16; ++h) {
      *reinterpret_cast<v4i*>(la + h * kRowStep * kPitch) = ra[h];
      *reinterpret_cast<v4i*>(lb + h * kRowStep * kPitch) = rb[h];
    }
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = (kt & 1) * kStageBytes;
    const bool more = kt + 1 < nk;
    if (more) {  // prefetch the next stage into registers
      const long k1 = static_cast<long>(kt + 1) * kBK;
#pragma unroll
      for (int h = 0; h < kStage16; ++h) {
        ra[h] = *reinterpret_cast<const v4i*>(ga + h * gstep + k1);
        rb[h] = *reinterpret_cast<const v4i*>(gb + h * gstep + k1);
      }
    }
    v4i fa[8], fb[8];
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) fa[mi] = *reinterpret_cast<const v4i*>(fa0 + cur + mi * 16 * kPitch);
#pragma unroll
    for (int ni = 0; ni < 8; ++ni) fb[ni] = *reinterpret_cast<const v4i*>(fb0 + cur + ni * 16 * kPitch);
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
      for (int ni = 0; ni < 8; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
    if (more) {
      const int nxt = kStageBytes - cur;
#pragma unroll
      for (int h = 0; h < kStage16; ++h) {
        *reinterpret_cast<v4i*>(la + nxt + h * kRowStep * kPitch) = ra[h];
        *reinterpret_cast<v4i*>(lb + nxt + h * kRowStep * kPitch) = rb[h];
      }
    }
    __syncthreads();
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
    const int m = kModsDev[t];
    const double invm = 1.0 / static_cast<double>(m);
    uint8_t* rt = res + t * r_plane;
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) {
#pragma unroll
      for (int ni = 0; ni < 8; ++ni) {
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
