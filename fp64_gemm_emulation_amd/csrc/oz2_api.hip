// oz2_api.hip -- the C ABI declared in include/oz2.h: argument checks, workspace layout,
// the four stage launches on the caller's stream, stage timing and validation dumps.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <vector>

#include "oz2.h"
#include "oz2_common.hpp"
#include "oz2_internal.hpp"

namespace {

using oz2::Work;

constexpr size_t kAlign = 256;
// Largest p and r: keeps every launch within the grid limits (at most 2^32 - 1 work-items
// along x, 65535 blocks along y) for every kernel.
constexpr long kMaxDim = 1L << 23;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
long round_up(long v, long m) { return (v + m - 1) / m * m; }

struct Layout {
  int p_pad, r_pad, q_pad, nch;
  long at_plane, bt_plane, res_plane;
  size_t off_flags, off_d, off_b, off_pea, off_psa, off_peb, off_psb, off_e, off_f, off_rho, off_gamma, off_at,
      off_bt, off_res, total;
};

Layout make_layout(int p, int q, int r, int s) {
  Layout L{};
  L.p_pad = static_cast<int>(round_up(std::max(p, 1), oz2::kRowPad));
  L.r_pad = static_cast<int>(round_up(std::max(r, 1), oz2::kRowPad));
  L.q_pad = static_cast<int>(round_up(q, oz2::kKPad));
  L.nch = (q + oz2::kChunk - 1) / oz2::kChunk;
  size_t off = 0;
  auto take = [&off](size_t bytes) {
    size_t o = off;
    off += align_up(std::max<size_t>(bytes, 1));
    return o;
  };
  L.off_flags = take(sizeof(unsigned));
  L.off_d = take(sizeof(int) * static_cast<size_t>(p));
  L.off_b = take(sizeof(int) * static_cast<size_t>(r));
  L.off_pea = take(sizeof(int) * static_cast<size_t>(p) * L.nch);
  L.off_psa = take(sizeof(double) * static_cast<size_t>(p) * L.nch);
  L.off_peb = take(sizeof(int) * static_cast<size_t>(r) * L.nch);
  L.off_psb = take(sizeof(double) * static_cast<size_t>(r) * L.nch);
  L.off_e = take(sizeof(int) * static_cast<size_t>(p));
  L.off_f = take(sizeof(int) * static_cast<size_t>(r));
  L.off_rho = take(sizeof(int) * static_cast<size_t>(p));
  L.off_gamma = take(sizeof(int) * static_cast<size_t>(r));
  // planes are packed back to back (padding them apart measured no faster at n = 8192)
  L.at_plane = static_cast<long>(L.p_pad) * L.q_pad;
  L.bt_plane = static_cast<long>(L.r_pad) * L.q_pad;
  L.res_plane = static_cast<long>(L.r_pad) * L.p_pad;
  L.off_at = take(static_cast<size_t>(s) * L.at_plane);
  L.off_bt = take(static_cast<size_t>(s) * L.bt_plane);
  L.off_res = take(static_cast<size_t>(s) * L.res_plane);
  L.total = off;
  return L;
}

// Operands (A and B together) above this size are read with the non-temporal hint in the
// statistics and residue passes: the 256 MB memory-side cache cannot keep them from one
// pass to the next, and streamed reads that allocate there only evict the residue planes
// and the other operand's tail.  Smaller operands are read normally, so the residue pass
// finds them in that cache.
constexpr double kStreamInputsBytes = 128.0 * (1 << 20);

Work bind(const Layout& L, char* base, int p, int q, int r, int s, bool accu) {
  Work w{};
  w.stream_inputs = 8.0 * (static_cast<double>(p) * q + static_cast<double>(q) * r) > kStreamInputsBytes;
  w.p = p;
  w.q = q;
  w.r = r;
  w.s = s;
  w.accu = accu;
  w.p_pad = L.p_pad;
  w.r_pad = L.r_pad;
  w.q_pad = L.q_pad;
  w.nch = L.nch;
  w.tau = 0;
  w.flags = reinterpret_cast<unsigned*>(base + L.off_flags);
  w.d = reinterpret_cast<int*>(base + L.off_d);
  w.b = reinterpret_cast<int*>(base + L.off_b);
  w.part_e_a = reinterpret_cast<int*>(base + L.off_pea);
  w.part_s_a = reinterpret_cast<double*>(base + L.off_psa);
  w.part_e_b = reinterpret_cast<int*>(base + L.off_peb);
  w.part_s_b = reinterpret_cast<double*>(base + L.off_psb);
  w.e_row = reinterpret_cast<int*>(base + L.off_e);
  w.f_col = reinterpret_cast<int*>(base + L.off_f);
  w.rho = reinterpret_cast<int*>(base + L.off_rho);
  w.gamma = reinterpret_cast<int*>(base + L.off_gamma);
  w.at = reinterpret_cast<int8_t*>(base + L.off_at);
  w.bt = reinterpret_cast<int8_t*>(base + L.off_bt);
  w.abar = w.at;  // consumed by the bound GEMM before the residues overwrite plane 0
  w.bbar = w.bt;
  w.res = reinterpret_cast<uint8_t*>(base + L.off_res);
  w.at_plane = L.at_plane;
  w.bt_plane = L.bt_plane;
  w.res_plane = L.res_plane;
  return w;
}

constexpr int tau_table(int s) {
  switch (s) {
#define OZ2_TAU_CASE(S) \
  case S:               \
    return oz2::tau_of(S);
    OZ2_TAU_CASE(2) OZ2_TAU_CASE(3) OZ2_TAU_CASE(4) OZ2_TAU_CASE(5) OZ2_TAU_CASE(6) OZ2_TAU_CASE(7)
    OZ2_TAU_CASE(8) OZ2_TAU_CASE(9) OZ2_TAU_CASE(10) OZ2_TAU_CASE(11) OZ2_TAU_CASE(12) OZ2_TAU_CASE(13)
    OZ2_TAU_CASE(14) OZ2_TAU_CASE(15) OZ2_TAU_CASE(16) OZ2_TAU_CASE(17) OZ2_TAU_CASE(18) OZ2_TAU_CASE(19)
    OZ2_TAU_CASE(20)
#undef OZ2_TAU_CASE
    default:
      return -1;
  }
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const auto pa = reinterpret_cast<uintptr_t>(a);
  const auto pb = reinterpret_cast<uintptr_t>(b);
  return na > 0 && nb > 0 && pa < pb + nb && pb < pa + na;
}

// One call: C (p x r) = alpha op(A) op(B) + beta C, op(A) p x q, op(B) q x r.
struct Call {
  int transa, transb;
  int p, q, r;
  double alpha;
  const double* A;
  int lda;
  const double* B;
  int ldb;
  double beta;
  double* C;
  int ldc;
  int s, mode;
};

int validate(const Call& c, const oz2_dump_t* dump) {
  if (c.s < OZ2_MIN_S || c.s > OZ2_MAX_S) return OZ2_ERR_ARG;
  if (c.mode != OZ2_FAST && c.mode != OZ2_ACCU) return OZ2_ERR_ARG;
  if ((c.transa != OZ2_OP_N && c.transa != OZ2_OP_T) || (c.transb != OZ2_OP_N && c.transb != OZ2_OP_T))
    return OZ2_ERR_ARG;
  if (c.p < 0 || c.q < 0 || c.r < 0 || c.p > kMaxDim || c.r > kMaxDim) return OZ2_ERR_ARG;
  if (c.q > OZ2_MAX_Q) return OZ2_ERR_UNSUPPORTED;
  // the raw P_t dump holds int32 products, exact only without K-blocking
  if (dump != nullptr && dump->P != nullptr && c.q > OZ2_MAX_Q_P_DUMP) return OZ2_ERR_UNSUPPORTED;
  // one GEMM launch puts every 256 x 256 output tile of a plane along grid x (256
  // work-items each): keep that work-item count in 32 bits
  if (static_cast<uint64_t>(round_up(std::max(c.p, 1), oz2::kRowPad) / oz2::kRowPad) *
          static_cast<uint64_t>(round_up(std::max(c.r, 1), oz2::kRowPad) / oz2::kRowPad) * 256u >= (1ull << 32))
    return OZ2_ERR_UNSUPPORTED;
  // stored shapes: A is p x q (N) or q x p (T); B is q x r (N) or r x q (T)
  const int a_rows = c.transa == OZ2_OP_N ? c.p : c.q, a_cols = c.transa == OZ2_OP_N ? c.q : c.p;
  const int b_rows = c.transb == OZ2_OP_N ? c.q : c.r, b_cols = c.transb == OZ2_OP_N ? c.r : c.q;
  if (c.lda < std::max(1, a_rows) || c.ldb < std::max(1, b_rows) || c.ldc < std::max(1, c.p)) return OZ2_ERR_ARG;
  if (c.p == 0 || c.r == 0) return OZ2_OK;
  if (c.C == nullptr) return OZ2_ERR_ARG;
  if (c.q > 0 && (c.A == nullptr || c.B == nullptr)) return OZ2_ERR_ARG;
  const size_t c_bytes = sizeof(double) * (static_cast<size_t>(c.ldc) * (c.r - 1) + c.p);
  if (c.q > 0) {
    const size_t a_bytes = sizeof(double) * (static_cast<size_t>(c.lda) * (a_cols - 1) + a_rows);
    const size_t b_bytes = sizeof(double) * (static_cast<size_t>(c.ldb) * (b_cols - 1) + b_rows);
    if (overlaps(c.C, c_bytes, c.A, a_bytes) || overlaps(c.C, c_bytes, c.B, b_bytes)) return OZ2_ERR_ARG;
  }
  return OZ2_OK;
}

// ---------------------------------------------------------------------------
// Library state: workspace and timing
// ---------------------------------------------------------------------------
struct Owned {
  void* ptr = nullptr;
  size_t bytes = 0;
};

struct State {
  std::vector<Owned> owned;  // library-owned workspace, one per device ordinal
  void* user = nullptr;
  size_t user_bytes = 0;
  // timing
  bool timing = false;
  int timing_max = 0;
  int timing_n = 0;
  int last_timed = -1;  // event set of the most recent timed call
  std::vector<hipEvent_t> events;  // 5 per timed call
  // last call (for flags)
  hipStream_t last_stream = nullptr;
  unsigned* last_flags = nullptr;
};

State g;

// Workspace of ozaki2_dgemm_noalloc: a fixed device array, one copy per GPU the library
// runs on (it exists from the module's load on that GPU until the process ends).  In host
// code `scratch` names a host-side stand-in, not device memory: its device address is
// resolved once per device with hipGetSymbolAddress and only that address is used.
static __device__ __align__(256) unsigned char scratch[OZ2_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};  // per device ordinal; filled on the first call there

// The scratch array's device address on the current device (no allocation).
int scratch_workspace(char** base) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return OZ2_ERR_HIP;
  if (dev >= kMaxDevices) return OZ2_ERR_UNSUPPORTED;
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return OZ2_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *base = static_cast<char*>(g_scratch_ptr[dev]);
  return OZ2_OK;
}

int acquire_workspace(size_t need, char** base) {
  if (g.user != nullptr) {
    if (g.user_bytes < need) return OZ2_ERR_WORKSPACE;
    *base = static_cast<char*>(g.user);
    return OZ2_OK;
  }
  // the buffer of the device current at this call (each device gets its own)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return OZ2_ERR_HIP;
  if (g.owned.size() <= static_cast<size_t>(dev)) g.owned.resize(static_cast<size_t>(dev) + 1);
  Owned& o = g.owned[static_cast<size_t>(dev)];
  if (o.bytes < need) {
    if (o.ptr != nullptr) {
      if (hipDeviceSynchronize() != hipSuccess) return OZ2_ERR_HIP;
      (void)hipFree(o.ptr);
      o.ptr = nullptr;
      o.bytes = 0;
    }
    if (hipMalloc(&o.ptr, need) != hipSuccess) {
      o.ptr = nullptr;
      (void)hipGetLastError();
      return OZ2_ERR_WORKSPACE;
    }
    o.bytes = need;
  }
  *base = static_cast<char*>(o.ptr);
  return OZ2_OK;
}

struct Recorder {
  hipEvent_t* ev = nullptr;
  hipStream_t st;
  explicit Recorder(hipStream_t s) : st(s) {
    if (g.timing && g.timing_n < g.timing_max) {
      ev = &g.events[5 * static_cast<size_t>(g.timing_n)];
      g.last_timed = g.timing_n;
      ++g.timing_n;
    }
  }
  hipError_t mark(int k) { return ev != nullptr ? hipEventRecord(ev[k], st) : hipSuccess; }
};

#define OZ2_TRY(expr)                         \
  do {                                        \
    if ((expr) != hipSuccess) return OZ2_ERR_HIP; \
  } while (0)

int copy_rows_2d(void* dst, size_t dpitch, const void* src, size_t spitch, size_t width, size_t height,
                 hipStream_t st) {
  if (width == 0 || height == 0) return OZ2_OK;
  OZ2_TRY(hipMemcpy2DAsync(dst, dpitch, src, spitch, width, height, hipMemcpyDeviceToDevice, st));
  return OZ2_OK;
}

// use_scratch: the workspace is the fixed scratch array (ozaki2_dgemm_noalloc), checked
// against its size before any HIP call; otherwise the caller's or the library's buffer.
int run(const Call& c, void* stream, const oz2_dump_t* dump, bool use_scratch = false) {
  int rc = validate(c, dump);
  if (rc != OZ2_OK) return rc;
  const int p = c.p, q = c.q, r = c.r, s = c.s, mode = c.mode;
  if (p == 0 || r == 0) return OZ2_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool accu = mode == OZ2_ACCU;
  const Layout lay = make_layout(p, q, r, s);
  char* base = nullptr;
  if (use_scratch) {
    if (lay.total > OZ2_NOALLOC_SCRATCH_BYTES) return OZ2_ERR_WORKSPACE;
    if ((rc = scratch_workspace(&base)) != OZ2_OK) return rc;
  } else if ((rc = acquire_workspace(lay.total, &base)) != OZ2_OK) {
    return rc;
  }
  Work w = bind(lay, base, p, q, r, s, accu);
  w.tau = tau_table(s);
  oz2_dump_t dz{};
  if (dump != nullptr) dz = *dump;
  oz2::DumpPtrs dp;
  dp.ap = dz.Ap;
  dp.bp = dz.Bp;
  dp.pt = dz.P;
  dp.x = dz.X;

  Recorder rec(st);
  OZ2_TRY(rec.mark(0));
  // rows of op(A) are contiguous when A is transposed; columns of op(B) unless B is
  const oz2::Operand opa{c.A, c.lda, c.transa == OZ2_OP_T};
  const oz2::Operand opb{c.B, c.ldb, c.transb == OZ2_OP_N};
  w.exp_in_residues = oz2::exponents_in_residues(opa, opb, w, dp);
  // --- scaling ---
  if (!accu) {
    OZ2_TRY(oz2::launch_fast_scaling(opa, opb, w, st));
  } else {
    OZ2_TRY(oz2::launch_accu_bound_inputs(opa, opb, w, st));
    if (dz.Abar != nullptr) OZ2_TRY(oz2::launch_unpack_operands(w.abar, w.at_plane, 1, p, q, w.q_pad, dz.Abar, st));
    if (dz.Bbar != nullptr) OZ2_TRY(oz2::launch_unpack_operands(w.bbar, w.bt_plane, 1, r, q, w.q_pad, dz.Bbar, st));
    OZ2_TRY(oz2::launch_gemm(w, 2, dp, st));
    OZ2_TRY(oz2::launch_accu_exponents(w, st));
    if (dz.e != nullptr) OZ2_TRY(hipMemcpyAsync(dz.e, w.e_row, sizeof(int) * p, hipMemcpyDeviceToDevice, st));
    if (dz.f != nullptr) OZ2_TRY(hipMemcpyAsync(dz.f, w.f_col, sizeof(int) * r, hipMemcpyDeviceToDevice, st));
    if (dz.rho != nullptr) OZ2_TRY(hipMemcpyAsync(dz.rho, w.rho, sizeof(int) * p, hipMemcpyDeviceToDevice, st));
    if (dz.gamma != nullptr)
      OZ2_TRY(hipMemcpyAsync(dz.gamma, w.gamma, sizeof(int) * r, hipMemcpyDeviceToDevice, st));
  }
  OZ2_TRY(rec.mark(1));
  // --- residues ---
  OZ2_TRY(oz2::launch_residues(opa, opb, w, dp, st));
  // (d and b are final here: for small fast-mode products the residue launch computes them)
  if (dz.d != nullptr) OZ2_TRY(hipMemcpyAsync(dz.d, w.d, sizeof(int) * p, hipMemcpyDeviceToDevice, st));
  if (dz.b != nullptr) OZ2_TRY(hipMemcpyAsync(dz.b, w.b, sizeof(int) * r, hipMemcpyDeviceToDevice, st));
  if (dz.At != nullptr) OZ2_TRY(oz2::launch_unpack_operands(w.at, w.at_plane, s, p, q, w.q_pad, dz.At, st));
  if (dz.Bt != nullptr) OZ2_TRY(oz2::launch_unpack_operands(w.bt, w.bt_plane, s, r, q, w.q_pad, dz.Bt, st));
  OZ2_TRY(rec.mark(2));
  // --- GEMMs + output reduction ---
  OZ2_TRY(oz2::launch_gemm(w, dz.P != nullptr ? 1 : 0, dp, st));
  if (dz.R != nullptr) {
    for (int t = 0; t < s; ++t) {
      rc = copy_rows_2d(dz.R + static_cast<size_t>(t) * r * p, p,
                        w.res + static_cast<size_t>(t) * w.res_plane, w.p_pad, p, r, st);
      if (rc != OZ2_OK) return rc;
    }
  }
  OZ2_TRY(rec.mark(3));
  // --- CRT + inverse scaling ---
  OZ2_TRY(oz2::launch_crt(w, c.C, c.ldc, c.alpha, c.beta, dp, st));
  OZ2_TRY(rec.mark(4));
  g.last_stream = st;
  g.last_flags = w.flags;
  return OZ2_OK;
}

}  // namespace

extern "C" {

int ozaki2_dgemm(int p, int q, int r, const double* A, int lda, const double* B, int ldb, double* C, int ldc, int s,
                 int mode, void* stream) {
  const Call c{OZ2_OP_N, OZ2_OP_N, p, q, r, 1.0, A, lda, B, ldb, 0.0, C, ldc, s, mode};
  return run(c, stream, nullptr);
}

int ozaki2_dgemm_ex(int transa, int transb, int p, int q, int r, double alpha, const double* A, int lda,
                    const double* B, int ldb, double beta, double* C, int ldc, int s, int mode, void* stream) {
  const Call c{transa, transb, p, q, r, alpha, A, lda, B, ldb, beta, C, ldc, s, mode};
  return run(c, stream, nullptr);
}

int ozaki2_dgemm_noalloc(int p, int q, int r, const double* A, int lda, const double* B, int ldb, double* C, int ldc,
                         int s, int mode, void* stream) {
  const Call c{OZ2_OP_N, OZ2_OP_N, p, q, r, 1.0, A, lda, B, ldb, 0.0, C, ldc, s, mode};
  return run(c, stream, nullptr, true);
}

int ozaki2_dgemm_debug(int p, int q, int r, const double* A, int lda, const double* B, int ldb, double* C, int ldc,
                       int s, int mode, void* stream, const oz2_dump_t* dump) {
  const Call c{OZ2_OP_N, OZ2_OP_N, p, q, r, 1.0, A, lda, B, ldb, 0.0, C, ldc, s, mode};
  return run(c, stream, dump);
}

size_t ozaki2_workspace_size(int p, int q, int r, int s, int mode) {
  if (s < OZ2_MIN_S || s > OZ2_MAX_S || (mode != OZ2_FAST && mode != OZ2_ACCU)) return 0;
  if (p <= 0 || r <= 0 || q < 0 || q > OZ2_MAX_Q || p > kMaxDim || r > kMaxDim) return 0;
  return make_layout(p, q, r, s).total;
}

int ozaki2_set_workspace(void* dev_ptr, size_t bytes) {
  if (dev_ptr != nullptr && (reinterpret_cast<uintptr_t>(dev_ptr) % kAlign) != 0) return OZ2_ERR_ARG;
  g.user = dev_ptr;
  g.user_bytes = dev_ptr != nullptr ? bytes : 0;
  return OZ2_OK;
}

int ozaki2_release(void) {
  int rc = OZ2_OK;
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) rc = OZ2_ERR_HIP;
  if (!g.events.empty() && hipDeviceSynchronize() != hipSuccess) rc = OZ2_ERR_HIP;
  for (size_t dev = 0; dev < g.owned.size(); ++dev) {
    Owned& o = g.owned[dev];
    if (o.ptr == nullptr) continue;
    // synchronize and free on the device that owns the buffer
    if (hipSetDevice(static_cast<int>(dev)) != hipSuccess || hipDeviceSynchronize() != hipSuccess ||
        hipFree(o.ptr) != hipSuccess)
      rc = OZ2_ERR_HIP;
    o.ptr = nullptr;
    o.bytes = 0;
  }
  if (!g.owned.empty() && hipSetDevice(cur) != hipSuccess) rc = OZ2_ERR_HIP;
  for (hipEvent_t e : g.events) (void)hipEventDestroy(e);
  g.events.clear();
  g.timing = false;
  g.timing_max = g.timing_n = 0;
  g.last_timed = -1;
  g.last_flags = nullptr;
  g.last_stream = nullptr;
  return rc;
}

int ozaki2_timing_begin(int max_calls) {
  if (max_calls < 1) return OZ2_ERR_ARG;
  const size_t need = 5 * static_cast<size_t>(max_calls);
  while (g.events.size() < need) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return OZ2_ERR_HIP;
    g.events.push_back(e);
  }
  g.timing = true;
  g.timing_max = max_calls;
  g.timing_n = 0;
  return OZ2_OK;
}

int ozaki2_timing_end(double* stage_ms, int* ncalls) {
  if (stage_ms == nullptr || ncalls == nullptr) return OZ2_ERR_ARG;
  for (int k = 0; k < 4; ++k) stage_ms[k] = 0.0;
  const int n = g.timing_n;
  g.timing = false;
  *ncalls = n;
  if (n == 0) return OZ2_OK;
  if (hipEventSynchronize(g.events[5 * static_cast<size_t>(n) - 1]) != hipSuccess) return OZ2_ERR_HIP;
  for (int c = 0; c < n; ++c) {
    for (int k = 0; k < 4; ++k) {
      float ms = 0.0f;
      if (hipEventElapsedTime(&ms, g.events[5 * static_cast<size_t>(c) + k],
                              g.events[5 * static_cast<size_t>(c) + k + 1]) != hipSuccess)
        return OZ2_ERR_HIP;
      stage_ms[k] += ms;
    }
  }
  g.timing_n = 0;
  return OZ2_OK;
}

int ozaki2_get_stage_ms(float* ms) {
  if (ms == nullptr || g.last_timed < 0 || 5 * static_cast<size_t>(g.last_timed) + 4 >= g.events.size())
    return OZ2_ERR_ARG;
  hipEvent_t* ev = &g.events[5 * static_cast<size_t>(g.last_timed)];
  if (hipEventSynchronize(ev[4]) != hipSuccess) return OZ2_ERR_HIP;
  for (int k = 0; k < 4; ++k)
    if (hipEventElapsedTime(&ms[k], ev[k], ev[k + 1]) != hipSuccess) return OZ2_ERR_HIP;
  return OZ2_OK;
}

int ozaki2_get_flags(unsigned* flags) {
  if (flags == nullptr) return OZ2_ERR_ARG;
  *flags = 0;
  if (g.last_flags == nullptr) return OZ2_OK;
  unsigned v = 0;
  if (hipMemcpyAsync(&v, g.last_flags, sizeof(v), hipMemcpyDeviceToHost, g.last_stream) != hipSuccess)
    return OZ2_ERR_HIP;
  if (hipStreamSynchronize(g.last_stream) != hipSuccess) return OZ2_ERR_HIP;
  *flags = v;
  return OZ2_OK;
}

int ozaki2_moduli(int s, int* out) {
  if (s < OZ2_MIN_S || s > OZ2_MAX_S || out == nullptr) return OZ2_ERR_ARG;
  for (int t = 0; t < s; ++t) out[t] = oz2::modulus(t);
  return OZ2_OK;
}

int ozaki2_tau(int s) { return tau_table(s); }

const char* ozaki2_status_string(int status) {
  switch (status) {
    case OZ2_OK:
      return "ok";
    case OZ2_ERR_ARG:
      return "invalid argument";
    case OZ2_ERR_UNSUPPORTED:
      return "unsupported: q above OZ2_MAX_Q, a launch grid beyond its limits, or a P_t dump with q above OZ2_MAX_Q_P_DUMP";
    case OZ2_ERR_WORKSPACE:
      return "workspace too small (a caller buffer, or the fixed scratch of ozaki2_dgemm_noalloc: "
             "OZ2_NOALLOC_SCRATCH_BYTES) or device allocation failed";
    case OZ2_ERR_HIP:
      return "HIP runtime or kernel launch error";
    default:
      return "unknown status";
  }
}

}  // extern "C"
