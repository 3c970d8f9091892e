/*
 * oz2.h -- C ABI of the Ozaki Scheme II FP64 GEMM emulation for AMD MI355X (gfx950).
 *
 * The library computes C ~= A * B for FP64 matrices with s exact INT8 x INT8 -> INT32
 * modular GEMMs and Chinese-Remainder reconstruction, following the pipeline of
 * "Profiling Ozaki II: The Cost Behind Fast INT8 GEMMs", Part I section 1 (stage table),
 * and "Ozaki II supplement: INT8 range conditions and paper performance results",
 * section 1.1:
 *
 *   D, E      power-of-two row / column scalings from a bound (fast or accu)
 *   A' = trunc(D A),  B' = trunc(B E)
 *   A_t = rho_{m_t}(A'),  B_t = rho_{m_t}(B')      centered int8 residues, t = 1..s
 *   P_t = A_t B_t                                  int8 x int8 -> int32, exact for q < 2^17
 *                                                  (longer q: blocked, each block reduced mod m_t)
 *   R_t = P_t mod m_t                              nonnegative, uint8
 *   X   = CRT(R_1..R_s) in [-M/2, M/2),  M = prod m_t
 *   C   = D^-1 X E^-1
 *
 * Moduli: the first s pairwise-coprime integers taken greedily downward from 256
 * (256, 255, 253, 251, 247, 241, 239, 233, 229, 227, 223, 217, 211, 199, 197, ...).
 *
 * Conventions for every entry point:
 *   - Matrices are column-major FP64: A is p x q with leading dimension lda >= max(1,p),
 *     B is q x r with ldb >= max(1,q), C is p x r with ldc >= max(1,p) (ozaki2_dgemm_ex
 *     also takes transposed A and B).
 *   - Matrix and workspace pointers are DEVICE pointers on the current HIP device.
 *     C must not overlap A, B or the workspace.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Work is
 *     enqueued asynchronously on it; no entry point synchronizes unless stated.
 *   - Arguments are validated before anything is enqueued; on an error return nothing
 *     has been launched and C is untouched.
 *   - Not thread-safe: calls share one library workspace and one timing state; calls on
 *     different streams that share a workspace must be ordered by the caller.
 *   - ozaki2_dgemm and ozaki2_dgemm_ex enqueue kernels only (no allocation, memory set or
 *     copy) once their workspace exists, so a call can be captured in a HIP graph when a
 *     caller workspace is set (or an earlier call of the same or larger size has created
 *     the library's); the graph keeps the workspace pointer, which must stay valid.
 */
#ifndef OZ2_H
#define OZ2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bound used to choose D and E ("Profiling Ozaki II", Part I section 2). */
typedef enum {
  OZ2_FAST = 0, /* Cauchy-Schwarz bound from row/column max-abs and sums of squares */
  OZ2_ACCU = 1  /* positional bound from one extra upward-quantized |A| |B| INT8 GEMM */
} oz2_mode_t;

/* Status codes returned by every int-valued entry point. */
enum {
  OZ2_OK = 0,
  OZ2_ERR_ARG = 1,         /* invalid size, leading dimension, pointer, s or mode */
  OZ2_ERR_UNSUPPORTED = 2, /* q > OZ2_MAX_Q, a size whose launch grid would not fit, or a raw P_t
                              dump requested with q > OZ2_MAX_Q_P_DUMP */
  OZ2_ERR_WORKSPACE = 3,   /* caller workspace or the fixed scratch of ozaki2_dgemm_noalloc too small,
                              or device allocation failed */
  OZ2_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
};

#define OZ2_MIN_S 2
#define OZ2_MAX_S 20
/* One INT32 dot product of int8 residues is exact while q 128^2 < 2^31, i.e. q < 2^17
 * ("Ozaki II supplement", section 1.3).  Longer inner dimensions are split into blocks of
 * 2^17 whose partial products are reduced mod m_t before they are combined, which is exact
 * for any q (odd m_t: residues are at most 127 in magnitude; m_t = 256: only the low byte
 * of a block sum is used); the limit below comes from the accu bound product, whose INT32 entries
 * are at most q 64^2. */
#define OZ2_MAX_Q 524287
/* Largest q for which the raw P_t dump of ozaki2_dgemm_debug is defined (exact INT32). */
#define OZ2_MAX_Q_P_DUMP 131071
/* X is dumped as a 160-bit two's-complement integer in 5 little-endian 32-bit limbs. */
#define OZ2_X_LIMBS 5

/* Flag bits reported by ozaki2_get_flags. */
#define OZ2_FLAG_NONFINITE 1u /* A or B held Inf/NaN; affected entries of C are unspecified */

/*
 * ozaki2_dgemm -- C = A * B emulated with s INT8 modular GEMMs (the whole pipeline above).
 *   p, q, r : sizes (>= 0; p == 0 or r == 0 is a no-op; q == 0 writes C = 0).
 *   s       : number of moduli, OZ2_MIN_S..OZ2_MAX_S.
 *   mode    : OZ2_FAST or OZ2_ACCU.
 * Uses the workspace set by ozaki2_set_workspace, else a library-owned buffer on the
 * current device (one per device) that is allocated (or grown) on first need and kept
 * until ozaki2_release(); growing it synchronizes the current device.
 * Returns OZ2_OK, OZ2_ERR_ARG, OZ2_ERR_UNSUPPORTED, OZ2_ERR_WORKSPACE or OZ2_ERR_HIP.
 */
int ozaki2_dgemm(int p, int q, int r, const double* A, int lda, const double* B, int ldb,
                 double* C, int ldc, int s, int mode, void* stream);

/*
 * ozaki2_dgemm_noalloc -- the product of ozaki2_dgemm (same arguments, kernels and result)
 * for callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  It allocates nothing (no hipMalloc,
 * hipFree or allocating library call) and ignores ozaki2_set_workspace: its workspace is a
 * fixed device array of OZ2_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, which
 * exists from the library's load on that GPU until the process ends.  The first call on a
 * device resolves the array's address there (hipGetSymbolAddress, no allocation).
 *   Size limit: a product whose ozaki2_workspace_size exceeds OZ2_NOALLOC_SCRATCH_BYTES is
 *   rejected with OZ2_ERR_WORKSPACE before anything is launched (square products:
 *   n = 2048 fits for every s, n = 3072 up to s = 9, n = 4096 up to s = 5).
 *   Sharing: every call on one GPU uses that GPU's one array, so calls that may overlap on
 *   one GPU (different streams, or host threads) race and must be ordered by the caller.
 *   The kernels clear what must start at zero themselves; nothing carries over between
 *   calls.
 * Returns OZ2_OK, OZ2_ERR_ARG, OZ2_ERR_UNSUPPORTED, OZ2_ERR_WORKSPACE or OZ2_ERR_HIP.
 */
#define OZ2_NOALLOC_SCRATCH_BYTES (256ull << 20)
int ozaki2_dgemm_noalloc(int p, int q, int r, const double* A, int lda, const double* B, int ldb,
                         double* C, int ldc, int s, int mode, void* stream);

/* Operation applied to an input matrix by ozaki2_dgemm_ex. */
typedef enum {
  OZ2_OP_N = 0, /* the matrix as stored */
  OZ2_OP_T = 1  /* its transpose */
} oz2_op_t;

/*
 * ozaki2_dgemm_ex -- C = alpha op(A) op(B) + beta C, the product emulated as in
 * ozaki2_dgemm with op(A) (p x q) and op(B) (q x r) in place of A and B.
 *   transa : OZ2_OP_N: A is p x q, lda >= max(1,p);  OZ2_OP_T: A is q x p, lda >= max(1,q).
 *   transb : OZ2_OP_N: B is q x r, ldb >= max(1,q);  OZ2_OP_T: B is r x q, ldb >= max(1,r).
 *   C      : p x r, ldc >= max(1,p).  With Chat the emulated product (the value ozaki2_dgemm
 *            stores), each entry becomes alpha * Chat when beta == 0 (C is then not read,
 *            so it may hold anything) and fma(alpha, Chat, beta * C) otherwise.
 * alpha = 1, beta = 0 with OZ2_OP_N twice is exactly ozaki2_dgemm.  The scalings are those
 * of op(A) and op(B): rows of op(A) and columns of op(B).  Same workspace, errors and
 * ordering rules as ozaki2_dgemm; transa/transb outside oz2_op_t give OZ2_ERR_ARG.
 */
int ozaki2_dgemm_ex(int transa, int transb, int p, int q, int r, double alpha, const double* A, int lda,
                    const double* B, int ldb, double beta, double* C, int ldc, int s, int mode, void* stream);

/* Bytes of device workspace ozaki2_dgemm / ozaki2_dgemm_debug need for these sizes
 * (0 if the arguments are invalid or describe no work). */
size_t ozaki2_workspace_size(int p, int q, int r, int s, int mode);

/* Use a caller-owned device buffer (256-byte aligned, `bytes` long) as the workspace of
 * every following call, whichever device is current (it must be memory of the device the
 * calls run on).  dev_ptr == NULL reverts to the library-owned buffers.  The caller keeps
 * ownership and must keep the buffer alive while calls using it are in flight. */
int ozaki2_set_workspace(void* dev_ptr, size_t bytes);

/* Free the library-owned workspaces (synchronizing each device that holds one) and the
 * timing events (synchronizing the current device). */
int ozaki2_release(void);

/*
 * Validation dumps for ozaki2_dgemm_debug.  Every member is a device pointer the
 * caller owns; NULL members are skipped.  Layouts (t = modulus index 0..s-1):
 *   d[p], b[r]           int32 scaling exponents: D = diag(2^d), E = diag(2^b)
 *   Ap[p*q]              A' as exact FP64 integers, column-major, ld p
 *   Bp[q*r]              B' as exact FP64 integers, column-major, ld q
 *   At[s*p*q]            A_t[i][l] at At[(t*p + i)*q + l]
 *   Bt[s*r*q]            B_t[l][j] at Bt[(t*r + j)*q + l]
 *   P[s*r*p]             P_t[i][j] at P[(t*r + j)*p + i]   (int32; only for q <= OZ2_MAX_Q_P_DUMP)
 *   R[s*r*p]             R_t[i][j] at R[(t*r + j)*p + i]   (uint8)
 *   X[r*p*5]             X[i][j] at X[(j*p + i)*5 + k], k = 0..4: the 32-bit words of X as a
 *                        160-bit two's-complement integer, least significant first
 * accu mode only (ignored in fast mode):
 *   e[p], f[r]           max-abs exponents of rows of A / columns of B (E(x): 2^(E-1) <= |x| < 2^E;
 *                        INT32_MIN for an all-zero line)
 *   Abar[p*q]            upward-quantized |A|, Abar[i*q + l] in [0, 64]
 *   Bbar[r*q]            upward-quantized |B|, Bbar[j*q + l] in [0, 64]
 *   rho[p], gamma[r]     row / column maxima of the bound product Abar * Bbar^T
 */
typedef struct oz2_dump {
  int32_t* d;
  int32_t* b;
  double* Ap;
  double* Bp;
  int8_t* At;
  int8_t* Bt;
  int32_t* P;
  uint8_t* R;
  uint32_t* X;
  int32_t* e;
  int32_t* f;
  int8_t* Abar;
  int8_t* Bbar;
  int32_t* rho;
  int32_t* gamma;
} oz2_dump_t;

/* Same computation and result C as ozaki2_dgemm, also writing every intermediate named
 * in `dump` (which may be NULL).  Slower (extra kernels and copies); for validation. */
int ozaki2_dgemm_debug(int p, int q, int r, const double* A, int lda, const double* B, int ldb,
                       double* C, int ldc, int s, int mode, void* stream, const oz2_dump_t* dump);

/*
 * Stage timing.  ozaki2_timing_begin(max_calls) pre-creates events for up to max_calls
 * subsequent ozaki2_dgemm calls; each timed call records HIP events on its stream between
 * the four stages.  ozaki2_timing_end synchronizes on the last recorded event and returns
 * the per-stage sums in milliseconds over the timed calls:
 *   stage_ms[0] scaling   (fast: statistics + exponents; accu: bound inputs, bound GEMM, exponents)
 *   stage_ms[1] residues  (scale, truncate and all s centered int8 residues of A and B; for small
 *                          untransposed fast-mode products, whose exponents this launch computes
 *                          from the statistics, also the exponents)
 *   stage_ms[2] gemm      (the batched s INT8 GEMMs with the fused mod-m epilogue)
 *   stage_ms[3] crt       (CRT reconstruction and inverse scaling into C)
 * and in *ncalls the number of calls timed.  Timing is then switched off.
 */
int ozaki2_timing_begin(int max_calls);
int ozaki2_timing_end(double* stage_ms, int* ncalls);

/* The four stage times in milliseconds (same order as above) of the most recent call that
 * was timed (made while ozaki2_timing_begin was in effect; untimed calls record no events).
 * Synchronizes on that call's last event.  OZ2_ERR_ARG if ms is NULL or no call has been
 * timed since the library's events were created, OZ2_ERR_HIP on a runtime error. */
int ozaki2_get_stage_ms(float* ms);

/* Synchronizes the stream of the last call and returns its flag word (OZ2_FLAG_*). */
int ozaki2_get_flags(unsigned* flags);

/* The s moduli used for s (writes s ints) and tau = floor(log2(M/2 - 1)), the
 * reconstruction budget the scalings keep |(A'B')_ij| <= 2^tau within. */
int ozaki2_moduli(int s, int* out);
int ozaki2_tau(int s);

/* Static description of a status code. */
const char* ozaki2_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* OZ2_H */
