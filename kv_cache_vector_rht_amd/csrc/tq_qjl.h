// QJL projection of key residuals on the matrix cores:
//   sigma_j = [ (S r)_j >= 0 ],  j < D,
// the 1-bit sign of a Johnson-Lindenstrauss projection of the residual
// ("TurboQuantとは？仕組み・実測精度・2026年7月時点の実装状況", 第2段).
//
// Z^T = S R^T is computed with v_mfma_f32_32x32x16_f16: A = a 32x16 tile
// of S (fp16, exact as stored), B = a 16x32 tile of R^T (one column per
// token). Each residual is pre-scaled by 2^10
// (exact) and split as r = hi + lo in fp16 (22 significant bits; the scaling
// keeps lo out of the fp16 subnormal range), so two MFMAs with fp32
// accumulation give the projection to about 2^-22 relative, far inside the
// 1e-6 decision margin. The residual arrives already scaled by 2^10. The
// signs come back per token: the C tile holds, in
// lane l, column l%32 (a token) and 16 of the 32 rows (projection indices);
// a lane swap merges the two halves into the token's 32-bit word.
#pragma once

#include "tq_device.h"

namespace tq {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ v16f mfma_f16_32x32x16(const v8h &a, const v8h &b, const v16f &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

union V8H {
  v8h h;
  uint32_t u[4];
};

// Two residual coordinates (already scaled by 2^10) as fp16 hi and lo parts,
// each pair packed in one dword: hi = fp16(a) rounded toward zero, lo =
// fp16(a - hi) likewise (a - hi is exact in fp32), so hi + lo carries 22
// significant bits of a.
__device__ __forceinline__ void split_pair(float a0, float a1, uint32_t &hi, uint32_t &lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a0, a1));
  // a - fp32(hi half) in one mixed-precision fma (the fp16 operand is
  // widened inside the instruction; the difference is exact)
  float d0, d1;
  asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(d0) : "v"(hi), "v"(a0));
  asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d1) : "v"(hi), "v"(a1));
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(d0, d1));
}

// Bit 8 (q / 4) + q % 4 set where c[q] >= 0, q < 16 (the C tile rows one
// lane half holds). The sums start from +0, so no entry is -0 and c >= 0
// exactly when the sign bit is clear; byte permutes gather the sign bytes
// of c[b], c[b + 4], c[b + 8], c[b + 12] into one word per b.
__device__ __forceinline__ uint32_t nonneg_bits(const v16f &c) {
  uint32_t neg = 0u;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t t1 = __builtin_amdgcn_perm(__float_as_uint(c[b + 4]), __float_as_uint(c[b]), 0x0c0c0703u);
    const uint32_t t2 = __builtin_amdgcn_perm(__float_as_uint(c[b + 12]), __float_as_uint(c[b + 8]), 0x0c0c0703u);
    const uint32_t sb = __builtin_amdgcn_perm(t2, t1, 0x05040100u);
    neg |= (sb >> (7 - b)) & (0x01010101u << b);
  }
  return ~neg & 0x0f0f0f0fu;
}

// Stage the fp16 sketch [D][D] in LDS with rows padded by 8 halves. The
// block has THREADS threads; all loads are issued before the first store.
template <int D, int THREADS>
__device__ __forceinline__ void stage_sketch(const uint16_t *__restrict__ sketch, uint16_t *s_sk) {
  constexpr int RP = D + 8;
  constexpr int N = D * D / 8 / THREADS;     // 16-byte pieces per thread
  static_assert(N * THREADS == D * D / 8, "sketch pieces per thread");
  uint4 v[N];
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] = reinterpret_cast<const uint4 *>(sketch)[k * THREADS + threadIdx.x];
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const int e = k * THREADS + threadIdx.x;
    const int row = e / (D / 8), c8 = e % (D / 8);
    // column unit 4 a + 2 h + b (coordinates 32 a + 16 h + 8 b ..) goes to
    // position (D / 16) h + 2 a + b, the K order of the encoder's lanes
    const int pos = (D / 16) * ((c8 >> 1) & 1) + 2 * (c8 >> 2) + (c8 & 1);
    *reinterpret_cast<uint4 *>(s_sk + row * RP + pos * 8) = v[k];
  }
}

// Sign words of one 32-token tile: lane half h of token t holds the tile's
// residual coordinates 32 b + 16 h + i (times 2^10) in r[16 b + i], b < D/32.
// K slot (ks, h, e) of the projection is coordinate
// 32 (ks / 2) + 16 h + 8 (ks % 2) + e = r[8 ks + e] of lane half h (the
// staged sketch's columns are in this order), so every lane feeds its own
// coordinates. sig[jt] is the token's sign word of projections
// 32 jt .. 32 jt + 31.
template <int D>
__device__ __forceinline__ void qjl_tile(const uint16_t *s_sk, const float *r, uint32_t (&sig)[D / 32]) {
  constexpr int RP = D + 8;
  constexpr int KS = D / 16;
  const int lane = lane_id();
  const int hw = lane / 32;
  V8H bh[KS], bl[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) split_pair(r[8 * ks + e], r[8 * ks + e + 1], bh[ks].u[e / 2], bl[ks].u[e / 2]);
  }
#pragma unroll
  for (int jt = 0; jt < D / 32; ++jt) {
    v16f c = {};
    const uint16_t *arow = s_sk + (jt * 32 + (lane % 32)) * RP + (D / 2) * hw;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      V8H a;
      const uint4 u = *reinterpret_cast<const uint4 *>(arow + 8 * ks);
      a.u[0] = u.x; a.u[1] = u.y; a.u[2] = u.z; a.u[3] = u.w;
      c = mfma_f16_32x32x16(a.h, bh[ks].h, c);
      c = mfma_f16_32x32x16(a.h, bl[ks].h, c);
    }
    // lane l holds rows 8(q/4) + 4 hw + q%4 of column l%32
    uint32_t pw = nonneg_bits(c);
    pw <<= 4 * hw;
    auto m = __builtin_amdgcn_permlane32_swap(pw, pw, false, false);
    sig[jt] = pw | (hw ? m[0] : m[1]);
  }
}

}  // namespace tq
