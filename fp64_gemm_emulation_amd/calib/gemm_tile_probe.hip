// gemm_tile_probe.hip -- measurement aid, not part of the GEMM emulation: a mod GEMM in the
// form of the library's (oz2_gemm.hip, whose helpers it uses) launched on caller-supplied int8
// operand planes with 256 x 256 or 128 x 128 output tiles, to time what the tile edge costs
// the GEMM stage.  A GEMM fused with the CRT ("Ozaki II supplement", section 3.2: reconstruction stays
// a substantial stage) must keep every output's s residues on chip until its last modulus:
// s bytes per output are 896 KiB for a 256 x 256 tile at s = 14, beyond the 160 KiB of LDS
// and the register file, while a 128 x 128 tile holds them in 224 VGPRs per lane.  The
// 128 x 128 GEMM alone (here even with two workgroups per CU) is therefore a lower bound on
// the time of such a fused kernel.
#include "../csrc/oz2_gemm.hip"

namespace oz2 {

// A mod GEMM on v_mfma_i32_16x16x64_i8 built like the library's gemm_w8_kernel (same operand
// layout, copy ring, fragment order and epilogue) with its tile edge as a parameter: BT x BT
// outputs per workgroup (BT = 256: one workgroup per CU; BT = 128: two, i.e. two waves per
// SIMD), 4 waves in a 2 x 2 grid, each (BT/2) x (BT/2) outputs = MB x MB blocks of 16 x 16.
// (As the large-grid GEMM itself, BT = 256 was measured 35% slower than gemm_w8_kernel at
// n = 8192, s = 14: its one wave per SIMD waits on its own copies, fragment reads and
// barriers with no second wave to keep the matrix core busy.)  Per stage kt and wave:
// wait for this stage's fragments and the copies of stage kt + 1; barrier (after which
// nothing reads the buffer of stage kt); MB^2 MFMAs with the 2 MB fragment reads of stage
// kt + 1 spread over the first three quarters of them and the copies of stage kt + kStages
// into the buffer of stage kt spread over all of them.  Waves 0-1 copy the A slice, 2-3
// the B slice.  Fragments, accumulator layout and epilogues as in gemm_w8_kernel.
template <int EPI, int BT>
__global__ __launch_bounds__(256, BT == 256 ? 1 : 2) void gemm_w4_kernel(
    const int8_t* __restrict__ at, const int8_t* __restrict__ bt, long a_plane, long b_plane, int K, int kt0, int nk,
    uint8_t* __restrict__ res, long r_plane, int ldr, int* __restrict__ rho, int* __restrict__ gamma, int p, int r,
    int tiles_m, int tiles_n) {
  static_assert(EPI == kEpiMod || EPI == kEpiModAcc || EPI == kEpiBound, "epilogues of the 4-wave GEMM");
  static_assert(BT == 256 || BT == 128, "tile edges 256 or 128");
  constexpr int kSlice = BT * kBK;                      // bytes of one operand per stage
  constexpr int kStageLds = 2 * kSlice;                 // A then B
  constexpr int kCopiesW = kStageLds / 1024 / 4;        // 1 KiB copies per wave per stage (8 or 4)
  constexpr int MB = BT / 32;                           // 16 x 16 blocks per wave and dimension
  constexpr int kFr = 2 * MB;                           // fragment reads per wave per stage
  constexpr int kMfma = MB * MB;                        // MFMAs per wave per stage
  constexpr int kReadEvery = (3 * kMfma / 4) / kFr > 0 ? (3 * kMfma / 4) / kFr : 1;
  constexpr int kCopyEvery = kMfma / kCopiesW;
  static_assert(kReadEvery * kFr <= kMfma && kCopyEvery * kCopiesW == kMfma, "read and copy schedule");
  static_assert(kStages == 4, "copy schedule and wait counts");
  __shared__ __attribute__((aligned(1024))) int8_t smem[kStages * kStageLds];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1;                    // rows (BT/2) wm
  const int wn = wave & 1;                     // columns (BT/2) wn
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
  // Copies: the tile's rows i0 .. i0 + BT - 1 are contiguous in each 16 KiB stage tile of
  // their 256-row block, from byte 64 (i0 mod 256); wave w moves bytes [(kSlice/2)(w mod 2)
  // + 1024 c, +1024) of the A (w < 2) or B slice, lane l at byte 16 l.
  const long a_base = static_cast<long>(i0 / kRowPad) * kRowPad * K + (i0 % kRowPad) * kBK;
  const long b_base = static_cast<long>(j0 / kRowPad) * kRowPad * K + (j0 % kRowPad) * kBK;
  const int8_t* const gsrc = (wave < 2 ? at + t * a_plane + a_base : bt + t * b_plane + b_base) +
                             static_cast<long>(kt0) * kTileBytes + (wave & 1) * (kSlice / 2) + 16 * lane;
  int8_t* const gdst = smem + (wave >= 2 ? kSlice : 0) + (wave & 1) * (kSlice / 2);
  auto copy1 = [&](int kbuf, int ksrc, int c) {
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(gsrc + static_cast<long>(ksrc) * kTileBytes + c * 1024),
                                     (lds_ptr_t)(gdst + (kbuf % kStages) * kStageLds + c * 1024), 16, 0, 0);
  };
  const int frow = lane & 15;
  const int fch = (lane >> 4) ^ operand_swizzle(frow);
  const int8_t* const fa = smem + (wm * (BT / 2) + frow) * kBK + 16 * fch;
  const int8_t* const fb = smem + kSlice + (wn * (BT / 2) + frow) * kBK + 16 * fch;
  auto read1 = [&](int kbuf, v4i (&x)[kFr], int g) {
    const int off = (kbuf % kStages) * kStageLds;
    if (g < MB) x[g] = *reinterpret_cast<const v4i*>(fa + off + g * 16 * kBK);
    else x[g] = *reinterpret_cast<const v4i*>(fb + off + (g - MB) * 16 * kBK);
  };
  v4i acc[MB][MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < MB; ++nb) acc[mb][nb] = v4i{-mr.h, -mr.h, -mr.h, -mr.h};
  v4i x0[kFr], x1[kFr];
  auto stage = [&](int kt, v4i (&x)[kFr], v4i (&y)[kFr]) {
    OZ2_WAIT_LGKMCNT(0);
    OZ2_WAIT_VMCNT(2 * kCopiesW);
    OZ2_SCHED_FENCE();
    __builtin_amdgcn_s_barrier();
    OZ2_SCHED_FENCE();
    const int kn = min(kt + kStages, nk - 1);
#pragma unroll
    for (int u = 0; u < kMfma; ++u) {
      const int mb = u / MB, nb = u % MB;
      acc[mb][nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(x[mb], x[MB + nb], acc[mb][nb], 0, 0, 0);
      if (u % kReadEvery == kReadEvery - 1 && u / kReadEvery < kFr) read1(kt + 1, y, u / kReadEvery);
      if (u % kCopyEvery == kCopyEvery / 2) copy1(kt, kn, u / kCopyEvery);
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
    OZ2_WAIT_VMCNT(0);
    OZ2_WAIT_LGKMCNT(0);
  }

  if constexpr (EPI == kEpiBound) {
    // rows: max over this wave's column blocks, then over the 16 lanes of each row group
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        int mx = 0;
#pragma unroll
        for (int nb = 0; nb < MB; ++nb) mx = max(mx, acc[mb][nb][v]);
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) mx = max(mx, __shfl_xor(mx, off, kWave));
        const int i = i0 + wm * (BT / 2) + 16 * mb + 4 * (lane >> 4) + v;
        if ((lane & 15) == 0 && i < p) atomicMax(rho + i, mx);
      }
    }
    // columns: max over this wave's row blocks and 4 registers, then over the 4 row groups
#pragma unroll
    for (int nb = 0; nb < MB; ++nb) {
      int mx = 0;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int v = 0; v < 4; ++v) mx = max(mx, acc[mb][nb][v]);
      mx = max(mx, __shfl_xor(mx, 16, kWave));
      mx = max(mx, __shfl_xor(mx, 32, kWave));
      const int j = j0 + wn * (BT / 2) + 16 * nb + (lane & 15);
      if (lane < 16 && j < r) atomicMax(gamma + j, mx);
    }
    return;
  }
  // Epilogue: residue words through the (now free) LDS ring in the XOR-swizzled column
  // layout of gemm_w8_kernel, so that every store instruction writes whole column segments.
  constexpr int WC = BT / 4;                   // words per tile column
  static_assert(WC >= 32 && BT * BT / 4 <= kStages * kStageLds, "staging fits the ring");
  uint32_t* const stg = reinterpret_cast<uint32_t*>(smem);
  __builtin_amdgcn_s_barrier();
  const int jl0 = wn * (BT / 2) + (lane & 15);
  const int wl0 = wm * (BT / 8) + (lane >> 4);
  auto stage_all = [&](auto m256) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int nb = 0; nb < MB; ++nb) {
        const int jl = jl0 + 16 * nb;
        const int wl = wl0 + 4 * mb;
        stg[WC * jl + (wl ^ (jl & 31))] = residue_word4<decltype(m256)::value>(acc[mb][nb], mr);
      }
      OZ2_SCHED_FENCE();  // one block row at a time: keeps the accumulator reads from piling up
    }
  };
  if (mr.m == 256)
    stage_all(std::true_type{});
  else
    stage_all(std::false_type{});
  __syncthreads();
  uint8_t* const rt = res + t * r_plane;
  constexpr int kTpc = BT / 16;                // threads per column (16 bytes each)
  constexpr int kCols = 256 / kTpc;            // columns per pass
  const int c = tid % kTpc;
#pragma unroll 4
  for (int pass = 0; pass < BT / kCols; ++pass) {
    const int jl = pass * kCols + tid / kTpc;
    const v4i d = *reinterpret_cast<const v4i*>(stg + WC * jl + 4 * (c ^ ((jl & 31) >> 2)));
    const int sw = jl & 3;
    int x0w = d[0], x1w = d[1], x2w = d[2], x3w = d[3];
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
      const v4i prev = *dst;
      x0w = static_cast<int>(add_mod_bytes(static_cast<uint32_t>(x0w), static_cast<uint32_t>(prev[0]), mr.m));
      x1w = static_cast<int>(add_mod_bytes(static_cast<uint32_t>(x1w), static_cast<uint32_t>(prev[1]), mr.m));
      x2w = static_cast<int>(add_mod_bytes(static_cast<uint32_t>(x2w), static_cast<uint32_t>(prev[2]), mr.m));
      x3w = static_cast<int>(add_mod_bytes(static_cast<uint32_t>(x3w), static_cast<uint32_t>(prev[3]), mr.m));
    }
    *dst = v4i{x0w, x1w, x2w, x3w};
  }
}

}  // namespace oz2

// at, bt: s planes of n x n int8 in the operand tile layout (any bytes: random data stands in
// for residues); res: s planes of n x n bytes.  n a multiple of 256, 1 <= s <= 20, tile 256
// or 128.  Returns 0, 1 for invalid arguments, 2 for a launch error.
extern "C" int oz2calib_gemm_tiles(const void* at, const void* bt, int n, int s, int tile, void* res, void* stream) {
  using namespace oz2;
  if (at == nullptr || bt == nullptr || res == nullptr || n <= 0 || n % 256 != 0 || s < 1 || s > kMaxS) return 1;
  const long plane = static_cast<long>(n) * n;
  const int nk = n / kBK;
  const auto* a = static_cast<const int8_t*>(at);
  const auto* b = static_cast<const int8_t*>(bt);
  auto* r = static_cast<uint8_t*>(res);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (tile == 256) {
    const int tm = n / 256;
    hipLaunchKernelGGL((gemm_w4_kernel<kEpiMod, 256>), dim3(tm * tm, 1, s), dim3(256), 0, st, a, b, plane, plane, n, 0,
                       nk, r, plane, n, nullptr, nullptr, n, n, tm, tm);
  } else if (tile == 128) {
    const int tm = n / 128;
    hipLaunchKernelGGL((gemm_w4_kernel<kEpiMod, 128>), dim3(tm * tm, 1, s), dim3(256), 0, st, a, b, plane, plane, n, 0,
                       nk, r, plane, n, nullptr, nullptr, n, n, tm, tm);
  } else {
    return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
