// Host driver for the per-output reconstruction arithmetic of the HIP library
// (fp64_gemm_emulation_amd/csrc/oz2_crt_round.hpp), so that a CPU test can check it
// against exact integer arithmetic.  Reads lines "s scale R_0 .. R_{s-1}" (residues
// R_t in [0, m_t)) and prints, per line, the five 32-bit two's-complement words of X and
// the bits of RN(X) 2^scale, all in hex.
#include <cstdio>
#include <cstring>

#include "oz2_crt_round.hpp"

template <int S>
static void one(int scale, const unsigned* res) {
  constexpr int L = oz2::CrtTable<S>::L;
  double acc[L];
  for (int k = 0; k < L; ++k) acc[k] = 0.0;
  for (int t = 0; t < S; ++t) oz2::crt_accumulate<S>(acc, static_cast<double>(res[t]), t);
  oz2::crt_reduce<S>(acc);
  constexpr int W = oz2::CrtTable<S>::kW;
  oz2::crt_normalize<L, W>(acc);
  uint32_t w[5];
  oz2::crt_words<L, W>(acc, w);
  const double z = oz2::crt_round<L, W, oz2::CrtTable<S>::kTopExp>(acc, scale);
  unsigned long long bits;
  std::memcpy(&bits, &z, sizeof bits);
  std::printf("%08x %08x %08x %08x %08x %016llx\n", w[0], w[1], w[2], w[3], w[4], bits);
}

template <int S>
static bool dispatch(int s, int scale, const unsigned* res) {
  if constexpr (S > oz2::kMaxS) {
    return false;
  } else {
    if (s == S) {
      one<S>(scale, res);
      return true;
    }
    return dispatch<S + 1>(s, scale, res);
  }
}

int main() {
  int s, scale;
  unsigned res[oz2::kMaxS];
  while (std::scanf("%d %d", &s, &scale) == 2) {
    if (s < oz2::kMinS || s > oz2::kMaxS) return 2;
    for (int t = 0; t < s; ++t)
      if (std::scanf("%u", &res[t]) != 1) return 3;
    if (!dispatch<oz2::kMinS>(s, scale, res)) return 4;
  }
  return 0;
}
