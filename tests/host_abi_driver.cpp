// Host driver of the library's C ABI paths that run before any HIP call: argument
// validation of every product entry point, the workspace arithmetic, the moduli / tau
// tables and the status strings.  Built with AddressSanitizer and UndefinedBehaviorSanitizer
// on the host code only (tests/test_sanitizers.py) and run without a GPU: every call here
// must return before the HIP runtime is touched.  Prints "ok" and exits 0 when every
// return value is the documented one.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "oz2.h"

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    std::printf("FAIL %s: got %d want %d\n", what, got, want);
    ++failures;
  }
}

int main() {
  // never dereferenced: every call below fails validation or has no work
  double* A = reinterpret_cast<double*>(uintptr_t{0x10000});
  double* B = reinterpret_cast<double*>(uintptr_t{0x20000000});
  double* C = reinterpret_cast<double*>(uintptr_t{0x40000000});
  const int n = 8;
  expect(ozaki2_dgemm(n, n, n, A, n, B, n, C, n, 1, OZ2_FAST, nullptr), OZ2_ERR_ARG, "s below range");
  expect(ozaki2_dgemm(n, n, n, A, n, B, n, C, n, 21, OZ2_FAST, nullptr), OZ2_ERR_ARG, "s above range");
  expect(ozaki2_dgemm(n, n, n, A, n, B, n, C, n, 8, 7, nullptr), OZ2_ERR_ARG, "mode");
  expect(ozaki2_dgemm(-1, n, n, A, n, B, n, C, n, 8, OZ2_FAST, nullptr), OZ2_ERR_ARG, "negative p");
  expect(ozaki2_dgemm(n, -1, n, A, n, B, n, C, n, 8, OZ2_FAST, nullptr), OZ2_ERR_ARG, "negative q");
  expect(ozaki2_dgemm(n, n, -5, A, n, B, n, C, n, 8, OZ2_FAST, nullptr), OZ2_ERR_ARG, "negative r");
  expect(ozaki2_dgemm(n, n, n, A, n - 1, B, n, C, n, 8, OZ2_FAST, nullptr), OZ2_ERR_ARG, "lda");
  expect(ozaki2_dgemm(n, n, n, A, n, B, n - 1, C, n, 8, OZ2_FAST, nullptr), OZ2_ERR_ARG, "ldb");
  expect(ozaki2_dgemm(n, n, n, A, n, B, n, C, n - 1, 8, OZ2_FAST, nullptr), OZ2_ERR_ARG, "ldc");
  expect(ozaki2_dgemm(n, n, n, nullptr, n, B, n, C, n, 8, OZ2_FAST, nullptr), OZ2_ERR_ARG, "A null");
  expect(ozaki2_dgemm(n, n, n, A, n, nullptr, n, C, n, 8, OZ2_FAST, nullptr), OZ2_ERR_ARG, "B null");
  expect(ozaki2_dgemm(n, n, n, A, n, B, n, nullptr, n, 8, OZ2_FAST, nullptr), OZ2_ERR_ARG, "C null");
  expect(ozaki2_dgemm(n, n, n, A, n, B, n, A + 3, n, 8, OZ2_FAST, nullptr), OZ2_ERR_ARG, "C overlaps A");
  expect(ozaki2_dgemm(n, n, n, A, n, B, n, B + 60, n, 8, OZ2_FAST, nullptr), OZ2_ERR_ARG, "C overlaps B");
  expect(ozaki2_dgemm(n, 524288, n, A, n, B, 524288, C, n, 8, OZ2_FAST, nullptr), OZ2_ERR_UNSUPPORTED, "q");
  expect(ozaki2_dgemm(1 << 24, n, n, A, 1 << 24, B, n, C, 1 << 24, 8, OZ2_FAST, nullptr), OZ2_ERR_ARG, "huge p");
  expect(ozaki2_dgemm(0, n, n, A, n, B, n, C, n, 8, OZ2_FAST, nullptr), OZ2_OK, "p = 0");
  expect(ozaki2_dgemm(n, n, 0, A, n, B, n, C, n, 8, OZ2_ACCU, nullptr), OZ2_OK, "r = 0");
  expect(ozaki2_dgemm(0, 0, 0, nullptr, 1, nullptr, 1, nullptr, 1, 8, OZ2_FAST, nullptr), OZ2_OK, "empty");
  // the grid bound: p_pad / 256 * r_pad / 256 * 256 work-items must stay below 2^32
  expect(ozaki2_dgemm(1 << 23, 4, 1 << 20, A, 1 << 23, B, 4, C, 1 << 23, 8, OZ2_FAST, nullptr), OZ2_ERR_UNSUPPORTED,
         "grid too large");
  // transposed forms and alpha / beta
  expect(ozaki2_dgemm_ex(2, OZ2_OP_N, n, n, n, 1.0, A, n, B, n, 0.0, C, n, 8, OZ2_FAST, nullptr), OZ2_ERR_ARG,
         "transa");
  expect(ozaki2_dgemm_ex(OZ2_OP_N, -1, n, n, n, 1.0, A, n, B, n, 0.0, C, n, 8, OZ2_FAST, nullptr), OZ2_ERR_ARG,
         "transb");
  expect(ozaki2_dgemm_ex(OZ2_OP_T, OZ2_OP_N, 4, 16, n, 1.0, A, 15, B, 16, 0.0, C, 4, 8, OZ2_FAST, nullptr),
         OZ2_ERR_ARG, "lda of transposed A");
  expect(ozaki2_dgemm_ex(OZ2_OP_N, OZ2_OP_T, 4, 16, n, 1.0, A, 4, B, n - 1, 0.0, C, 4, 8, OZ2_FAST, nullptr),
         OZ2_ERR_ARG, "ldb of transposed B");
  expect(ozaki2_dgemm_ex(OZ2_OP_T, OZ2_OP_T, 0, 16, n, 2.0, A, 16, B, n, 1.0, C, 1, 8, OZ2_ACCU, nullptr), OZ2_OK,
         "empty transposed");
  // validation dumps
  oz2_dump_t dump;
  std::memset(&dump, 0, sizeof dump);
  dump.P = reinterpret_cast<int32_t*>(uintptr_t{0x80000000});
  expect(ozaki2_dgemm_debug(n, 131072, n, A, n, B, 131072, C, n, 8, OZ2_FAST, nullptr, &dump), OZ2_ERR_UNSUPPORTED,
         "raw P dump beyond one K-block");
  expect(ozaki2_dgemm_debug(n, n, n, A, n, B, n, C, n, 1, OZ2_FAST, nullptr, &dump), OZ2_ERR_ARG, "debug s");
  expect(ozaki2_dgemm_debug(0, n, n, A, n, B, n, C, n, 8, OZ2_FAST, nullptr, nullptr), OZ2_OK, "debug empty");
  // the allocation-free entry point: validation, then its fixed scratch
  expect(ozaki2_dgemm_noalloc(n, n, n, A, n, B, n, C, n, 1, OZ2_FAST, nullptr), OZ2_ERR_ARG, "noalloc s");
  expect(ozaki2_dgemm_noalloc(n, n, n, A, n, B, n, C, n - 1, 8, OZ2_FAST, nullptr), OZ2_ERR_ARG, "noalloc ldc");
  expect(ozaki2_dgemm_noalloc(4096, 4096, 4096, A, 4096, B, 4096, C, 4096, 14, OZ2_FAST, nullptr),
         OZ2_ERR_WORKSPACE, "noalloc beyond the scratch");
  expect(ozaki2_dgemm_noalloc(0, n, n, A, n, B, n, C, n, 8, OZ2_FAST, nullptr), OZ2_OK, "noalloc empty");
  // workspace arithmetic over a range of sizes, up to the largest accepted rows
  size_t prev = 0;
  for (int p = 1; p <= (1 << 23); p *= 2) {
    const size_t w = ozaki2_workspace_size(p, 300, 257, 20, OZ2_ACCU);
    if (w == 0 || w < prev) {
      std::printf("FAIL workspace size not growing at p = %d\n", p);
      ++failures;
    }
    prev = w;
  }
  expect(static_cast<int>(ozaki2_workspace_size(8, 8, 8, 1, OZ2_FAST)), 0, "workspace size of an invalid s");
  expect(static_cast<int>(ozaki2_workspace_size(8, 524288, 8, 8, OZ2_FAST)), 0, "workspace size beyond OZ2_MAX_Q");
  if (ozaki2_workspace_size(2048, 2048, 2048, 20, OZ2_ACCU) > OZ2_NOALLOC_SCRATCH_BYTES) {
    std::printf("FAIL n = 2048 must fit the allocation-free scratch at every s\n");
    ++failures;
  }
  // caller workspace: must be 256-byte aligned; NULL reverts to the library's
  expect(ozaki2_set_workspace(reinterpret_cast<void*>(uintptr_t{0x1001}), 4096), OZ2_ERR_ARG, "misaligned workspace");
  expect(ozaki2_set_workspace(nullptr, 0), OZ2_OK, "workspace reset");
  // tables and strings
  int mods[OZ2_MAX_S];
  expect(ozaki2_moduli(1, mods), OZ2_ERR_ARG, "moduli s = 1");
  expect(ozaki2_moduli(8, nullptr), OZ2_ERR_ARG, "moduli null");
  expect(ozaki2_moduli(OZ2_MAX_S, mods), OZ2_OK, "moduli");
  expect(mods[0], 256, "first modulus");
  expect(mods[OZ2_MAX_S - 1], 173, "twentieth modulus");
  int prev_tau = 0;
  for (int s = OZ2_MIN_S; s <= OZ2_MAX_S; ++s) {
    const int t = ozaki2_tau(s);
    if (t <= prev_tau) {
      std::printf("FAIL tau not increasing at s = %d\n", s);
      ++failures;
    }
    prev_tau = t;
  }
  expect(ozaki2_tau(21), -1, "tau beyond range");
  for (int st = -1; st <= 5; ++st) {
    const char* msg = ozaki2_status_string(st);
    if (msg == nullptr || std::strlen(msg) == 0) {
      std::printf("FAIL status string %d\n", st);
      ++failures;
    }
  }
  expect(ozaki2_get_flags(nullptr), OZ2_ERR_ARG, "flags null");
  unsigned flags = 99;
  expect(ozaki2_get_flags(&flags), OZ2_OK, "flags before any call");
  expect(static_cast<int>(flags), 0, "flags value before any call");
  expect(ozaki2_timing_end(nullptr, nullptr), OZ2_ERR_ARG, "timing end null");
  expect(ozaki2_get_stage_ms(nullptr), OZ2_ERR_ARG, "stage ms null");
  float ms[4];
  expect(ozaki2_get_stage_ms(ms), OZ2_ERR_ARG, "stage ms before any timed call");
  expect(ozaki2_timing_begin(0), OZ2_ERR_ARG, "timing begin 0");
  if (failures != 0) return 1;
  std::printf("ok\n");
  return 0;
}
