// oz2_params.hpp -- compile-time constants of the Ozaki II emulation.
//
// Everything here is derived at compile time from two definitions:
//   * the moduli: pairwise coprime, at most 256 so centered residues fit int8
//     ("Ozaki II supplement: INT8 range conditions and paper performance results",
//     section 1.2), taken greedily downward from 256;
//   * M = prod m_t and the reconstruction range [-M/2, M/2) of the CRT
//     ("Profiling Ozaki II: The Cost Behind Fast INT8 GEMMs", Part I section 1).
// The scalings keep |(A'B')_ij| <= 2^tau with tau = floor(log2(M/2 - 1)).
#pragma once

#include <cstdint>

namespace oz2 {

constexpr int kMinS = 2;
constexpr int kMaxS = 20;

// Fast-mode bound: |a| quantized upward to kFBits fractional bits relative to the
// max-abs exponent of its kChunk-long block; accu-mode bound inputs are integers
// in [0, 2^kQBits].
constexpr int kFBits = 20;
constexpr int kChunk = 256;
constexpr int kQBits = 6;
constexpr int kNoExp = -(1 << 30);  // exponent of an all-zero line / block

// ---------------------------------------------------------------------------
// Moduli
// ---------------------------------------------------------------------------
constexpr int gcd_c(int a, int b) {
  while (b != 0) {
    int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

struct ModTable {
  int m[kMaxS];
};

constexpr ModTable make_moduli() {
  ModTable tab{};
  int n = 0;
  for (int c = 256; n < kMaxS && c >= 2; --c) {
    bool ok = true;
    for (int k = 0; k < n; ++k)
      if (gcd_c(c, tab.m[k]) != 1) ok = false;
    if (ok) tab.m[n++] = c;
  }
  return tab;
}

inline constexpr ModTable kModTable = make_moduli();
constexpr int modulus(int t) { return kModTable.m[t]; }

static_assert(modulus(0) == 256 && modulus(1) == 255 && modulus(7) == 233 && modulus(13) == 199,
              "greedy pairwise-coprime moduli from 256");

// ---------------------------------------------------------------------------
// Small fixed-width unsigned big integers (little-endian 32-bit limbs)
// ---------------------------------------------------------------------------
constexpr int kBigLimbs = 6;  // 192 bits > log2(M) for s <= 20 (about 155.4)

struct Big {
  uint32_t w[kBigLimbs];
};

constexpr Big big_one() {
  Big b{};
  b.w[0] = 1;
  return b;
}

constexpr Big big_mul_small(Big a, uint32_t m) {
  uint64_t carry = 0;
  for (int k = 0; k < kBigLimbs; ++k) {
    uint64_t v = static_cast<uint64_t>(a.w[k]) * m + carry;
    a.w[k] = static_cast<uint32_t>(v);
    carry = v >> 32;
  }
  return a;
}

constexpr Big big_shr1(Big a) {
  for (int k = 0; k < kBigLimbs; ++k) {
    uint32_t hi = (k + 1 < kBigLimbs) ? a.w[k + 1] : 0u;
    a.w[k] = (a.w[k] >> 1) | (hi << 31);
  }
  return a;
}

constexpr Big big_dec(Big a) {  // a - 1, a >= 1
  for (int k = 0; k < kBigLimbs; ++k) {
    if (a.w[k] != 0) {
      a.w[k] -= 1;
      break;
    }
    a.w[k] = 0xFFFFFFFFu;
  }
  return a;
}

constexpr int big_bitlen(Big a) {
  for (int k = kBigLimbs - 1; k >= 0; --k) {
    if (a.w[k] != 0) {
      int b = 0;
      uint32_t v = a.w[k];
      while (v) {
        ++b;
        v >>= 1;
      }
      return 32 * k + b;
    }
  }
  return 0;
}

constexpr uint32_t big_mod_small(Big a, uint32_t m) {
  uint64_t r = 0;
  for (int k = kBigLimbs - 1; k >= 0; --k) r = ((r << 32) | a.w[k]) % m;
  return static_cast<uint32_t>(r);
}

// prod_{t < S, t != skip} m_t
constexpr Big product_except(int S, int skip) {
  Big b = big_one();
  for (int t = 0; t < S; ++t)
    if (t != skip) b = big_mul_small(b, static_cast<uint32_t>(modulus(t)));
  return b;
}

constexpr Big modulus_product(int S) { return product_except(S, -1); }

// tau = floor(log2(M/2 - 1))
constexpr int tau_of(int S) { return big_bitlen(big_dec(big_shr1(modulus_product(S)))) - 1; }

constexpr uint32_t inv_mod(uint32_t a, uint32_t m) {
  a %= m;
  for (uint32_t x = 1; x < m; ++x)
    if ((a * x) % m == 1) return x;
  return 0;
}

constexpr uint32_t pow2_mod(int e, uint32_t m) {
  uint32_t r = 1 % m;
  for (int k = 0; k < e; ++k) r = (r * 2) % m;
  return r;
}

static_assert(tau_of(2) == 14 && tau_of(8) == 62 && tau_of(14) == 109 && tau_of(18) == 139,
              "tau = floor(log2(M/2 - 1))");

// ---------------------------------------------------------------------------
// Residue kernel: digit layout of A' and per-modulus constants
// ---------------------------------------------------------------------------
// A' = lo + 2^kLoBits H with lo in [0, 2^kLoBits) and H = floor(A' / 2^kLoBits) held as
// balanced base-256 digits d_k in [-128, 127].  For an odd modulus m the reduced value
// z = lo + sum_k d_k c_k (c_k the centered residue of 2^(kLoBits + 8 k), |c_k| <= 127)
// satisfies |z| < 2^22 + 8 * 128 * 127 < 2^23, so it is exact in FP32 and its nearest
// quotient by m can be taken in FP32.
constexpr int kLoBits = 22;

// Bit length bound of |A'|: fast keeps ||2^d_i A(i,:)||_2 <= 2^(tau/2); accu keeps
// |A'| < 2^(floor(tau/2) + kQBits).
constexpr int max_bits(int S, bool accu) { return accu ? tau_of(S) / 2 + kQBits : tau_of(S) / 2 + 1; }

// Words of four digits that carry H: four balanced digits hold |H| < 2^31, eight |H| < 2^63.
constexpr int digit_words(int S, bool accu) { return max_bits(S, accu) - kLoBits <= 30 ? 1 : 2; }
static_assert(max_bits(kMaxS, true) - kLoBits <= 62, "two digit words hold H");

constexpr int centered_small(uint32_t r, uint32_t m) {
  return (r > (m - 1) / 2) ? static_cast<int>(r) - static_cast<int>(m) : static_cast<int>(r);
}

// The four signed-byte coefficients rho_m(2^(kLoBits + 8 k)), k = 4 w .. 4 w + 3, of digit
// word w for modulus index t, packed little-endian.
constexpr int digit_coefs(int t, int w) {
  uint32_t packed = 0;
  for (int k = 0; k < 4; ++k) {
    const uint32_t m = static_cast<uint32_t>(modulus(t));
    const int c = centered_small(pow2_mod(kLoBits + 8 * (4 * w + k), m), m);
    packed |= (static_cast<uint32_t>(c) & 0xFFu) << (8 * k);
  }
  return static_cast<int>(packed);
}

// ---------------------------------------------------------------------------
// CRT constants: X = sum_t R_t W_t - k M, W_t = (M / m_t) * ((M / m_t)^-1 mod m_t).
// W_t and M are split into L limbs of kW <= 40 bits (the fewest limbs of at most 40 bits
// that hold M), stored in doubles, so the weighted sums are exact FP64 integer FMAs:
// every partial sum stays below 20 * 2^8 * 2^40 < 2^53.  k is the nearest integer to
// sum_t R_t W_t / M, estimated from the two top limb sums alone,
// k = rint(acc[L-1] q1 + acc[L-2] q0) with q1 = 2^(kW (L-1)) / M, q0 = 2^(kW (L-2)) / M.
// The limbs left out add less than 20 * 255 * 2^(kW (L-2)) * (1 + 2^-kW) / M
// <= 5100 * 2^-kW (M > 2^(kW (L-1))) to the quotient, below 4e-5 wherever L >= 3, and the
// scalings keep |X| <= 2^tau, which puts the exact quotient at least 0.014 from a
// half-integer for every s: the estimate rounds to k.
// ---------------------------------------------------------------------------
constexpr int crt_bits(int S) { return big_bitlen(modulus_product(S)); }
constexpr int crt_limbs(int S) { return (crt_bits(S) + 39) / 40; }
constexpr int crt_width(int S) { return (crt_bits(S) + crt_limbs(S) - 1) / crt_limbs(S); }

// bits [lo, lo + n) of a, n <= 40
constexpr uint64_t big_bits(Big a, int lo, int n) {
  uint64_t v = 0;
  for (int b = 0; b < n; ++b) {
    const int pos = lo + b;
    if (pos < 32 * kBigLimbs && ((a.w[pos / 32] >> (pos % 32)) & 1u)) v |= 1ull << b;
  }
  return v;
}

template <int S>
struct CrtTable {
  static constexpr int L = crt_limbs(S);
  static constexpr int kW = crt_width(S);
  // |floor(X / 2^(kW (L-1)))| <= 2^kTopExp for |X| <= 2^tau
  static constexpr int kTopExp = tau_of(S) - kW * (L - 1);
  double w[S][L];
  double m[L];
  double q1, q0;
};

template <int S>
constexpr CrtTable<S> make_crt() {
  CrtTable<S> tab{};
  constexpr int L = CrtTable<S>::L;
  constexpr int W = CrtTable<S>::kW;
  Big M = modulus_product(S);
  double md = 0.0;
  for (int k = kBigLimbs - 1; k >= 0; --k) md = md * 0x1p32 + static_cast<double>(M.w[k]);
  for (int k = 0; k < L; ++k) tab.m[k] = static_cast<double>(big_bits(M, W * k, W));
  for (int t = 0; t < S; ++t) {
    uint32_t mt = static_cast<uint32_t>(modulus(t));
    Big rest = product_except(S, t);
    uint32_t inv = inv_mod(big_mod_small(rest, mt), mt);
    Big w = big_mul_small(rest, inv);
    for (int k = 0; k < L; ++k) tab.w[t][k] = static_cast<double>(big_bits(w, W * k, W));
  }
  double p1 = 1.0;
  for (int k = 0; k < W * (L - 1); ++k) p1 *= 2.0;
  tab.q1 = p1 / md;
  double p0 = 1.0;
  for (int k = 0; k < W * (L - 2); ++k) p0 *= 2.0;
  tab.q0 = L >= 2 ? p0 / md : 0.0;
  return tab;
}

constexpr bool crt_layout_ok() {
  for (int s = kMinS; s <= kMaxS; ++s) {
    const int L = crt_limbs(s), W = crt_width(s);
    if (W > 40 || W * L < crt_bits(s)) return false;      // limbs hold M, sums exact
    if (L >= 2 && crt_bits(s) - 1 < W * (L - 1)) return false;  // M > 2^(W (L-1))
    if (L >= 3 && W < 27) return false;                  // neglected limbs < 4e-5
    if (tau_of(s) - W * (L - 1) > 40) return false;      // top limb below 2^40
    if (L == 1 && crt_bits(s) > 53) return false;
  }
  return true;
}
static_assert(crt_layout_ok(), "CRT limb layout");

template <int S>
inline constexpr CrtTable<S> kCrt = make_crt<S>();

}  // namespace oz2
