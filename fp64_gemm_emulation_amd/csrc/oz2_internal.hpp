// oz2_internal.hpp -- host-side launch interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace oz2 {

// Device pointers into one call's workspace (see the layout in oz2_api.hip).
struct Work {
  int p, q, r, s;
  bool accu;
  int p_pad, r_pad, q_pad;  // rows of A_t / B_t padded to kRowPad, inner dim to kKPad
  int nch;                  // number of kChunk-long blocks along q
  int tau;
  bool stream_inputs;       // FP64 operand reads with the non-temporal hint (large operands)
  bool exp_in_residues;     // fast mode: the residue launch computes d and b from the statistics
                            // partials (no exponent launch); see exponents_in_residues
  unsigned* flags;          // 1 word
  int* d;                   // [p]   row exponents of A
  int* b;                   // [r]   column exponents of B
  int* part_e_a;            // [p * nch]
  double* part_s_a;         // [p * nch]
  int* part_e_b;            // [r * nch]
  double* part_s_b;         // [r * nch]
  int* e_row;               // [p]   accu: max-abs exponents of rows of A
  int* f_col;               // [r]   accu: max-abs exponents of columns of B
  int* rho;                 // [p]   accu: row maxima of the bound product
  int* gamma;               // [r]   accu: column maxima of the bound product
  int8_t* at;               // s planes of p_pad x q_pad, tile-contiguous (operand_chunk_offset)
  int8_t* bt;               // s planes of r_pad x q_pad, same layout
  long at_plane, bt_plane;  // byte strides between the planes of A_t / B_t
  long res_plane;           // byte stride between the planes of R_t
  int8_t* abar;             // [p_pad][q_pad]     accu bound inputs (alias of A_t plane 0)
  int8_t* bbar;             // [r_pad][q_pad]     (alias of B_t plane 0)
  uint8_t* res;             // [s][r_pad][p_pad]  R_t, column-major planes
};

// One FP64 input operand as the kernels see it: its "lines" are the rows of op(A) or the
// columns of op(B), each q long.  contig: every line is contiguous in memory (columns of
// a column-major matrix, element k of line n at ptr[n ld + k]); otherwise a line is a
// row of a column-major matrix (element k of line n at ptr[n + k ld]).
struct Operand {
  const double* ptr;
  long ld;
  bool contig;
};

// Optional validation outputs written while the pipeline runs.
struct DumpPtrs {
  double* ap = nullptr;     // A' column-major, ld p
  double* bp = nullptr;     // B' column-major, ld q
  int32_t* pt = nullptr;    // P_t [s][r][p]
  uint32_t* x = nullptr;    // X   [r][p][5]
};

// scaling stage
hipError_t launch_fast_scaling(const Operand& a, const Operand& b, const Work& w, hipStream_t st);
hipError_t launch_accu_bound_inputs(const Operand& a, const Operand& b, const Work& w, hipStream_t st);
hipError_t launch_accu_exponents(const Work& w, hipStream_t st);

// residue stage
// Whether the fast-mode exponents can be computed inside the residue launch for these
// operands (small untransposed products with short inner dimensions, no A' / B' dumps).
bool exponents_in_residues(const Operand& a, const Operand& b, const Work& w, const DumpPtrs& dump);
hipError_t launch_residues(const Operand& a, const Operand& b, const Work& w, const DumpPtrs& dump,
                           hipStream_t st);

// GEMM stage: epi 0 = R_t only, 1 = R_t and raw P_t dump, 2 = accu bound (rho, gamma)
hipError_t launch_gemm(const Work& w, int epi, const DumpPtrs& dump, hipStream_t st);

// reconstruction stage
// C = alpha Chat + beta C (C not read when beta == 0)
hipError_t launch_crt(const Work& w, double* C, long ldc, double alpha, double beta, const DumpPtrs& dump,
                      hipStream_t st);

// validation helper: operand planes in the tile-contiguous layout (padded) -> dst
// [planes][rows][q], plain row-major
hipError_t launch_unpack_operands(const int8_t* src, long plane_stride, int planes, int rows, int q, int q_pad,
                                  int8_t* dst, hipStream_t st);

}  // namespace oz2
