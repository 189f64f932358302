#pragma once
// Encode kernels: norm -> random-sign Walsh-Hadamard rotation -> Lloyd-Max
// threshold decisions -> (keys) residual, residual norm, QJL sign bits ->
// bit-packed codes and fp16 scalars.
//
// The method's steps follow "TurboQuant と RotorQuant を DGX Spark で試して
// みた" (section "PolarQuant + QJL の 2 段階圧縮": rotate, quantize without
// per-block scales, correct the error with one bit) and "TurboQuantとは？仕組
// み・実測精度・2026年7月時点の実装状況" (第1段: randomized Hadamard rotation +
// per-coordinate Lloyd-Max; 第2段: 1-bit JL projection of the residual).
//
// Mapping: every lane holds 64 coordinates of one token. For d = 64 a wave
// encodes 64 tokens (one lane each); for d = 128 it encodes 32 tokens, token
// t in lanes t and t + 32 (coordinates [0, 64) and [64, 128)). The first six
// butterfly stages of the rotation run in registers, the seventh (d = 128)
// pairs lane t with lane t + 32. A ballot over the wave of one coordinate's
// index bit yields 64 token bits: one 32-bit value-code word per 32-token
// block (d = 64: two blocks of the same coordinate; d = 128: coordinates c
// and c + 64 of one block). Key records are assembled per lane (each lane
// writes its half of every plane). The QJL projection of the wave's
// residuals runs on the matrix cores (tq_qjl.h).
#include "tq_device.h"
#include "tq_kernels.h"
#include "tq_qjl.h"

namespace tq {

// dst[lane LANE] = value (wave-uniform): v_writelane_b32.
template <int LANE>
__device__ __forceinline__ void write_lane(uint32_t &dst, uint32_t value) {
  const uint32_t v = __builtin_amdgcn_readfirstlane(value);
  asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(dst) : "s"(v), "i"(LANE));
}

// Lloyd-Max decisions by binary search over the sorted thresholds, most
// significant bit first: bit l of idx = [y >= t[((P << 1) | 1) << l) - 1]],
// P the bits above l. This gives idx = #{j : t_j <= y} (ties go up). The
// candidate thresholds sit in registers; pick() selects among them with the
// bits already decided (a tree of selects, no memory access).
template <int NB, int OFF, int N>
__device__ __forceinline__ float pick(const float (&cand)[N], const bool *dec) {
  if constexpr (NB == 0) {
    return cand[OFF];
  } else {
    const float hi = pick<NB - 1, OFF + (1 << (NB - 1))>(cand, dec + 1);
    const float lo = pick<NB - 1, OFF>(cand, dec + 1);
    return dec[0] ? hi : lo;
  }
}

// Thresholds grouped by level: lvl[l] holds the 2^(W-1-l) candidates of
// level l, indexed by the higher bits.
template <int W>
struct Levels {
  float t[(1 << W) - 1];
  __device__ __forceinline__ void load(const float *th) {
    int at = 0;
#pragma unroll
    for (int l = W - 1; l >= 0; --l)
#pragma unroll
      for (int P = 0; P < (1 << (W - 1 - l)); ++P) t[at++] = th[(((P << 1) | 1) << l) - 1];
  }
};

// dec[0] is the most significant bit (W - 1), dec[W-1] bit 0.
template <int W>
__device__ __forceinline__ void decide(float y, const Levels<W> &lv, bool (&dec)[W]) {
  static_for<0, W>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    dec[k] = y >= pick<k, (1 << k) - 1>(lv.t, dec);
  });
}

// c[idx] of a symmetric codebook (c[L-1-i] = -c[i]) from the decided bits:
// the upper half holds c_up[k], k = the lower bits; the lower half mirrors
// it with the lower bits inverted and the sign flipped.
template <int W>
__device__ __forceinline__ float centroid(const float (&c_up)[(1 << W) / 2], const bool (&dec)[W]) {
  if constexpr (W == 1) {
    return dec[0] ? c_up[0] : -c_up[0];
  } else {
    bool k[W - 1];
#pragma unroll
    for (int i = 0; i < W - 1; ++i) k[i] = dec[i + 1] == dec[0];
    const float cp = pick<W - 1, 0>(c_up, k);
    return dec[0] ? cp : -cp;
  }
}

// The other half-wave's copy of x (lane l <-> lane l ^ 32).
__device__ __forceinline__ float swap_half_f(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float((lane_id() < 32) ? r[1] : r[0]);
}

template <int D, int W, bool KEY>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 8))) void encode_kernel(EncodeParams p) {
  constexpr int L = 1 << W;
  constexpr int C = 64;                      // coordinates per lane
  constexpr int LPT = D / C;                 // lanes per token (1 or 2)
  constexpr int TPW = kWave / LPT;           // tokens per wave (64 or 32)
  constexpr int NWL = C / 32;                // plane words per lane (2)
  __shared__ float s_cent[L];
  __shared__ float s_th[L];
  __shared__ float s_sign[D];
  __shared__ __attribute__((aligned(16))) uint16_t s_sk[KEY ? D * (D + 8) : 8];
  if (threadIdx.x < L) s_cent[threadIdx.x] = p.centroids[threadIdx.x];
  if (threadIdx.x < L - 1) s_th[threadIdx.x] = p.thresholds[threadIdx.x];
  for (int i = threadIdx.x; i < D; i += blockDim.x) s_sign[i] = p.signs[i];
  if (KEY) stage_sketch<D>(p.sketch, s_sk);
  __syncthreads();

  const int lane = lane_id();
  const int tok = lane % TPW;                // token within the wave
  const int hv = lane / TPW;                 // which 64 coordinates (d = 128)
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (wave >= p.n_waves) return;             // whole wave exits together
  const int64_t seq = wave / p.groups_per_seq;
  const int64_t g = p.g0 + wave % p.groups_per_seq;
  const int64_t pos = g * TPW + tok;         // cache slot
  const int64_t t = pos - p.t0;              // input token
  const bool active = (t >= 0) && (t < p.n_tok);

  float v[C];
  if (active) {
    const int64_t off = seq * p.x_seq_stride + t * p.x_tok_stride + C * hv;
    if (p.xt == 0) load_row_vec_f32<C>(static_cast<const float *>(p.x) + off, v);
    else if (p.xt == 1) load_row_vec_16<C, true>(static_cast<const uint16_t *>(p.x) + off, v);
    else load_row_vec_16<C, false>(static_cast<const uint16_t *>(p.x) + off, v);
  } else {
#pragma unroll
    for (int i = 0; i < C; ++i) v[i] = 0.f;
  }

  // (a1) norm, accumulated in fp32 in coordinate order (then the two halves)
  float n2 = 0.f;
#pragma unroll
  for (int i = 0; i < C; ++i) n2 = fmaf(v[i], v[i], n2);
  if (LPT == 2) {
    const float o = swap_half_f(n2);
    n2 = hv ? (o + n2) : (n2 + o);
  }
  const float n = sqrtf(n2);

  // (a2) y = H diag(s) x / (n sqrt(D)); the zero vector maps to y = 0
#pragma unroll
  for (int i = 0; i < C; ++i) v[i] *= s_sign[C * hv + i];
  fwht_regs<C>(v);
  if (LPT == 2) {
    // stage 7: y_i = v_i + v_{i+64} (lane t), y_{i+64} = v_i - v_{i+64} (lane t + 32).
    // Swapping a value with itself across half-waves leaves the lower
    // half's copy (v_i) in the first register and the upper half's
    // (v_{i+64}) in the second, in every lane.
    const float sgn = hv ? -1.f : 1.f;
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const uint32_t u = __float_as_uint(v[i]);
      auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      v[i] = fmaf(sgn, __uint_as_float(r[1]), __uint_as_float(r[0]));
    }
  }
  const float inv = (n > 0.f) ? 1.0f / (n * sqrtf(static_cast<float>(D))) : 0.f;
#pragma unroll
  for (int i = 0; i < C; ++i) v[i] *= inv;

  Levels<W> lv;
  lv.load(s_th);

  if (KEY) {
    // (a3) indices -> this lane's half of every plane: each decision's lane
    // mask is added in as the carry of plane + plane, coordinate 31 first,
    // so coordinate i lands on bit i % 32;
    // (a4) residual, kept as r' = 2^10 r = fma(y, 2^10, -2^10 c) (exactly
    // 2^10 times the rounded y - c), the scale the QJL projection wants
    float c_up[L / 2];
#pragma unroll
    for (int j = 0; j < L / 2; ++j) c_up[j] = 1024.0f * s_cent[L / 2 + j];
    uint32_t planes[W][NWL];
#pragma unroll
    for (int q = 0; q < W; ++q)
#pragma unroll
      for (int k = 0; k < NWL; ++k) planes[q][k] = 0u;
    float g2 = 0.f;
#pragma unroll
    for (int i = C - 1; i >= 0; --i) {
      bool dec[W];
      decide<W>(v[i], lv, dec);
#pragma unroll
      for (int q = 0; q < W; ++q) {
        const uint64_t m = __ballot(dec[W - 1 - q]);
        uint64_t carry;
        asm("v_addc_co_u32_e64 %0, %1, %0, %0, %2" : "+v"(planes[q][i / 32]), "=s"(carry) : "s"(m));
      }
      v[i] = fmaf(v[i], 1024.0f, -centroid<W>(c_up, dec));
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < C; ++i) g2 = fmaf(v[i], v[i], g2);
    if (LPT == 2) {
      const float o = swap_half_f(g2);
      g2 = hv ? (o + g2) : (g2 + o);
    }
    const float gamma = sqrtf(g2) * (1.0f / 1024.0f);

    // (a5) QJL sign bits sigma_j = [ (S r)_j >= 0 ], on the matrix cores
    uint32_t sig[D / 32];
    qjl_signs_mfma<D>(s_sk, v, sig);

    if (active) {
      // (a6) record: W index planes then the sign plane, D/8 bytes each;
      // this lane writes bytes [8 hv, 8 hv + 8) of every plane
      constexpr int REC = (W + 1) * D / 8;
      constexpr int PB = D / 8;
      uint8_t *rec = static_cast<uint8_t *>(p.codes) + (seq * p.cap + pos) * REC + 8 * hv;
#pragma unroll
      for (int q = 0; q < W; ++q)
        *reinterpret_cast<uint2 *>(rec + q * PB) = make_uint2(planes[q][0], planes[q][1]);
      *reinterpret_cast<uint2 *>(rec + W * PB) = make_uint2(sig[2 * hv], sig[2 * hv + 1]);
      if (hv == 0) {
        const uint32_t sc = static_cast<uint32_t>(float_to_f16_bits(n)) |
                            (static_cast<uint32_t>(float_to_f16_bits(gamma)) << 16);
        reinterpret_cast<uint32_t *>(p.scalars)[seq * p.cap + pos] = sc;
      }
    }
  } else {
    // values: the ballot of coordinate slot c gives 64 token bits; lane c
    // keeps them (lo: bits 0-31, hi: bits 32-63)
    uint32_t lo[W], hi[W];
#pragma unroll
    for (int q = 0; q < W; ++q) { lo[q] = 0u; hi[q] = 0u; }
    static_for<0, C>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      bool dec[W];
      decide<W>(v[i], lv, dec);
#pragma unroll
      for (int q = 0; q < W; ++q) {
        const uint64_t m = __ballot(active && dec[W - 1 - q]);
        write_lane<i>(lo[q], static_cast<uint32_t>(m));
        write_lane<i>(hi[q], static_cast<uint32_t>(m >> 32));
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    const uint64_t valid = __ballot(active);
    const int64_t nblk = p.cap / kValueBlock;
    uint32_t *words = static_cast<uint32_t *>(p.codes);
    // d = 64: lo -> block 2g, hi -> block 2g + 1 (coordinate = lane)
    // d = 128: both -> block g; lo -> coordinate lane, hi -> coordinate 64 + lane
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const uint32_t vm = LPT == 2 ? static_cast<uint32_t>(valid) : static_cast<uint32_t>(valid >> (32 * half));
      if (vm == 0u) continue;
      const int64_t blk = LPT == 2 ? g : 2 * g + half;
      const int coord = LPT == 2 ? 64 * half + lane : lane;
      uint32_t *base = words + (seq * nblk + blk) * W * D + coord;
#pragma unroll
      for (int q = 0; q < W; ++q) {
        uint32_t w = half ? hi[q] : lo[q];
        uint32_t *dst = base + q * D;
        if (vm != 0xffffffffu) w = (*dst & ~vm) | (w & vm);
        *dst = w;
      }
    }
    if (active && hv == 0) p.scalars[seq * p.cap + pos] = float_to_f16_bits(n);
  }
}

// ---------------------------------------------------------------- dispatch

template <int D, int W, bool KEY>
static hipError_t launch_encode_dw(const EncodeParams &p, hipStream_t st) {
  const int64_t blocks = (p.n_waves + 3) / 4;
  hipLaunchKernelGGL((encode_kernel<D, W, KEY>), dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_encode_d(const EncodeParams &p, int w, bool key, hipStream_t st) {
  if (key) {
    switch (w) {
      case 1: return launch_encode_dw<D, 1, true>(p, st);
      case 2: return launch_encode_dw<D, 2, true>(p, st);
      case 3: return launch_encode_dw<D, 3, true>(p, st);
      default: return launch_encode_dw<D, 4, true>(p, st);
    }
  }
  switch (w) {
    case 1: return launch_encode_dw<D, 1, false>(p, st);
    case 2: return launch_encode_dw<D, 2, false>(p, st);
    case 3: return launch_encode_dw<D, 3, false>(p, st);
    default: return launch_encode_dw<D, 4, false>(p, st);
  }
}

}  // namespace tq
