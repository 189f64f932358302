// Matrix-core formulation of the TurboQuant logit and value sums (gfx950).
//
// Both sums are contractions of bit planes with real vectors:
//
//  * A symmetric Lloyd-Max codebook (c[L-1-j] = -c[j]) written in the index
//    bits b_p as +-1 variables s_p = 2 b_p - 1 keeps only odd-degree terms:
//        c[idx] = sum_{S odd} beta_S prod_{p in S} s_p,
//    beta_S = (1/L) sum_idx c[idx] prod_{p in S} s_p(idx), and for odd |S|
//        prod_{p in S} s_p = 2 x_S - 1,  x_S = XOR_{p in S} b_p.
//    So sum_i q_i c[idx_i] = 2 sum_S beta_S <q, x_S> - c[L-1] sum_i q_i:
//    one 0/1 plane per odd subset S (1, 2, 4, 8 planes for 1..4 bits).
//  * The QJL term sum_j p_j (2 sigma_j - 1) = 2 <p, sigma> - sum_j p_j.
//
// The 0/1 planes are the B operand of v_mfma_i32_16x16x64_i8. A 32-bit word
// w of a plane expands to int8 operands with one AND per dword:
// w & (0x01010101 << k) holds bits k, 8+k, 16+k, 24+k of w as bytes valued 0
// or 2^k (k = 7 gives 0 or -128). The real operand (queries, or attention
// weights) is turned into a 32-bit fixed-point integer that carries the
// matching 2^(7-k) (negated for k = 7), split into four signed 8-bit digits
// (the 16 rows of the MFMA are 4 heads x 4 digits). Sums are exact in int32;
// the float result is sum_digit 2^(8 digit) C_digit / 2^(7 + e).
//
// Operand layouts of v_mfma_i32_16x16x64_i8 (wave64), lane l:
//   A: row l%16, K slots 16*(l/16) + j, j = 0..15 (byte j of a 16-byte vector)
//   B: column l%16, the same K slots
//   C: rows 4*(l/16) + r, column l%16, r = 0..3
// K slot (kg = l/16, j = 4r + jb) of a 64-coordinate chunk holds coordinate
// 32*word + 8*jb + k with k = 4*(kg%2) + r and word = 2*(kg/2) + half for
// d = 128 (two chunks, half = 0, 1) or word = kg/2 for d = 64.
#pragma once

#include "tq_device.h"

namespace tq {

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4i mfma_i8(const v4i &a, const v4i &b, const v4i &c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Odd subsets of the index bits used as planes, as bit masks over the bits.
template <int W> struct Basis;
template <> struct Basis<1> { static constexpr int N = 1; static constexpr int M[1] = {1}; };
template <> struct Basis<2> { static constexpr int N = 2; static constexpr int M[2] = {1, 2}; };
template <> struct Basis<3> { static constexpr int N = 4; static constexpr int M[4] = {1, 2, 4, 7}; };
template <> struct Basis<4> {
  static constexpr int N = 8;
  static constexpr int M[8] = {1, 2, 4, 8, 7, 11, 13, 14};
};

__host__ __device__ constexpr int basis_size(int w) { return w == 1 ? 1 : w == 2 ? 2 : w == 3 ? 4 : 8; }

// Bytes of one (group, head chunk) record of prepared queries: the MFMA
// operand fragments of up to two row groups of 4 heads ((basis + sign plane)
// x D/64 fragments of 64 lanes x 16 bytes each) and 8 heads' constants.
__host__ __device__ constexpr int64_t prepared_stride(int d, int w) {
  return 2LL * (basis_size(w) + 1) * (d / 64) * 1024 + 128;
}

__device__ __forceinline__ int basis_mask(int w, int s) {
  // same tables as Basis<W>::M, for runtime use
  if (w <= 2) return 1 << s;
  if (w == 3) return s < 3 ? (1 << s) : 7;
  const int m4[8] = {1, 2, 4, 8, 7, 11, 13, 14};
  return m4[s];
}

// beta_S for the planes of a w-bit codebook (L = 2^w centroids).
__device__ __forceinline__ float basis_coeff(const float *cent, int w, int mask) {
  const int L = 1 << w;
  float acc = 0.f;
  for (int idx = 0; idx < L; ++idx) {
    const int par = __popc(static_cast<unsigned>(idx & mask)) ;
    // prod_{p in S} (2 b_p - 1) = (-1)^(|S| - popcount(idx & S))
    const int neg = (__popc(static_cast<unsigned>(mask)) - par) & 1;
    acc += neg ? -cent[idx] : cent[idx];
  }
  return acc / static_cast<float>(L);
}

// Four int8 operands from one plane word: bytes hold bits k0..k0+3 (+8, +16, +24).
__device__ __forceinline__ v4i expand_bits(uint32_t w, const uint32_t (&mask)[4]) {
  v4i b;
  b[0] = static_cast<int>(w & mask[0]);
  b[1] = static_cast<int>(w & mask[1]);
  b[2] = static_cast<int>(w & mask[2]);
  b[3] = static_cast<int>(w & mask[3]);
  return b;
}

// Signed base-256 digits of v (|v| <= 2^30) packed as bytes: digit s is byte s.
__device__ __forceinline__ uint32_t signed_digits(int32_t v) {
  return (static_cast<uint32_t>(v) + 0x00808080u) ^ 0x00808080u;
}

// sum_s 2^(8 s) C_s for the 4 digit rows a lane holds. A K slot's product is
// digit (|d| <= 128) x 2^k, and the 64 slots of one MFMA hold each bit k
// 0..7 eight times (sum of 2^k: 2040), so a row accumulated over at most 16
// MFMAs (the planes of a 4-bit key, or the value tiles of a split) keeps
// |C_s| < 128 * 2040 * 16 < 2^22: the digit pairs C_0 + 256 C_1 and
// C_2 + 256 C_3 stay below 2^31 in int32, and one fma joins them.
__device__ __forceinline__ float combine_digits(const v4i &c) {
  const int lo = c[0] + (c[1] << 8);
  const int hi = c[2] + (c[3] << 8);
  return fmaf(static_cast<float>(hi), 65536.f, static_cast<float>(lo));
}

// K-slot -> coordinate within the 64-coordinate chunk `half`.
__device__ __forceinline__ int slot_coord(int D, int kg, int j, int half) {
  const int r = j >> 2, jb = j & 3;
  const int k = 4 * (kg & 1) + r;
  const int word = (D == 128) ? (2 * (kg >> 1) + half) : (kg >> 1);
  return 32 * word + 8 * jb + k;
}

// Exponent e with max_abs * 2^(e + 7) < 2^30 (0 when max_abs is 0).
__device__ __forceinline__ int fixed_exponent(float max_abs) {
  if (!(max_abs > 0.f)) return 0;
  int E;
  frexpf(max_abs, &E);          // max_abs = f 2^E, f in [0.5, 1)
  return 23 - E;
}

}  // namespace tq
