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
// Mapping: one wave encodes 64 consecutive cache slots of one sequence, one
// lane per token. The whole vector stays in the lane's registers, so the
// rotation is a register-only butterfly network (no shuffles, no LDS), and
// the threshold compares of a coordinate across the 64 lanes are exactly the
// 64 token bits of a value-code word (one ballot per plane and coordinate).
// Key records are assembled per lane. The QJL projection of a 64-token tile
// is in tq_qjl.h.
#include "tq_device.h"
#include "tq_kernels.h"
#include "tq_qjl.h"

namespace tq {

template <int D, int W, bool KEY>
__global__ __launch_bounds__(256) void encode_kernel(EncodeParams p) {
  constexpr int L = 1 << W;
  constexpr int NW = D / 32;                 // 32-bit words per plane
  __shared__ float s_cent[L];
  __shared__ float s_sign[D];
  if (threadIdx.x < L) s_cent[threadIdx.x] = p.centroids[threadIdx.x];
  for (int i = threadIdx.x; i < D; i += blockDim.x) s_sign[i] = p.signs[i];
  __syncthreads();

  const int lane = lane_id();
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (wave >= p.n_waves) return;             // whole wave exits together
  const int64_t seq = wave / p.groups_per_seq;
  const int64_t g = p.g0 + wave % p.groups_per_seq;
  const int64_t pos = g * kWave + lane;      // cache slot
  const int64_t t = pos - p.t0;              // input token
  const bool active = (t >= 0) && (t < p.n_tok);

  float v[D];
  if (active) {
    if (p.xt == 0) {
      load_row_vec_f32<D>(static_cast<const float *>(p.x) + seq * p.x_seq_stride + t * p.x_tok_stride, v);
    } else {
      const uint16_t *row = static_cast<const uint16_t *>(p.x) + seq * p.x_seq_stride + t * p.x_tok_stride;
      if (p.xt == 1) load_row_vec_16<D, true>(row, v);
      else load_row_vec_16<D, false>(row, v);
    }
  } else {
#pragma unroll
    for (int i = 0; i < D; ++i) v[i] = 0.f;
  }

  // (a1) norm, accumulated in fp32 in coordinate order
  float n2 = 0.f;
#pragma unroll
  for (int i = 0; i < D; ++i) n2 = fmaf(v[i], v[i], n2);
  const float n = sqrtf(n2);

  // (a2) y = H diag(s) x / (n sqrt(D)); the zero vector maps to y = 0
#pragma unroll
  for (int i = 0; i < D; ++i) v[i] *= s_sign[i];
  fwht_regs<D>(v);
  const float inv = (n > 0.f) ? 1.0f / (n * sqrtf(static_cast<float>(D))) : 0.f;
#pragma unroll
  for (int i = 0; i < D; ++i) v[i] *= inv;

  // (a3) idx = #{j : y >= t_j}; thresholds are wave-uniform
  float th[L - 1];
#pragma unroll
  for (int j = 0; j < L - 1; ++j) th[j] = p.thresholds[j];

  if (KEY) {
    uint32_t planes[W][NW];
#pragma unroll
    for (int q = 0; q < W; ++q)
#pragma unroll
      for (int k = 0; k < NW; ++k) planes[q][k] = 0u;
    float g2 = 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) {
      int idx = 0;
#pragma unroll
      for (int j = 0; j < L - 1; ++j) idx += (v[i] >= th[j]) ? 1 : 0;
#pragma unroll
      for (int q = 0; q < W; ++q) planes[q][i / 32] |= static_cast<uint32_t>((idx >> q) & 1) << (i % 32);
      // (a4) residual in the rotated unit domain
      v[i] = v[i] - s_cent[idx];
      g2 = fmaf(v[i], v[i], g2);
    }
    const float gamma = sqrtf(g2);

    // (a5) QJL sign bits sigma_j = [ (S r)_j >= 0 ]
    uint32_t sig[NW];
    qjl_signs<D>(p.sketch, v, sig);

    if (active) {
      // (a6) record: W index planes then the sign plane, D/8 bytes each
      constexpr int REC = (W + 1) * D / 8;
      uint8_t *rec = static_cast<uint8_t *>(p.codes) + (seq * p.cap + pos) * REC;
      if (NW == 4) {
#pragma unroll
        for (int q = 0; q < W; ++q)
          *reinterpret_cast<uint4 *>(rec + q * 16) = make_uint4(planes[q][0], planes[q][1], planes[q][2], planes[q][3]);
        *reinterpret_cast<uint4 *>(rec + W * 16) = make_uint4(sig[0], sig[1], sig[2], sig[3]);
      } else {
#pragma unroll
        for (int q = 0; q < W; ++q)
          *reinterpret_cast<uint2 *>(rec + q * 8) = make_uint2(planes[q][0], planes[q][1]);
        *reinterpret_cast<uint2 *>(rec + W * 8) = make_uint2(sig[0], sig[1]);
      }
      const uint32_t sc = static_cast<uint32_t>(float_to_f16_bits(n)) |
                          (static_cast<uint32_t>(float_to_f16_bits(gamma)) << 16);
      reinterpret_cast<uint32_t *>(p.scalars)[seq * p.cap + pos] = sc;
    }
  } else {
    // values: one ballot per (plane, coordinate) gives the 64 token bits
    constexpr int CPL = (D + kWave - 1) / kWave;   // coordinates owned per lane
    uint32_t lo[W][CPL], hi[W][CPL];
#pragma unroll
    for (int q = 0; q < W; ++q)
#pragma unroll
      for (int c = 0; c < CPL; ++c) { lo[q][c] = 0u; hi[q][c] = 0u; }
#pragma unroll
    for (int i = 0; i < D; ++i) {
      int idx = 0;
#pragma unroll
      for (int j = 0; j < L - 1; ++j) idx += (v[i] >= th[j]) ? 1 : 0;
#pragma unroll
      for (int q = 0; q < W; ++q) {
        const uint64_t m = __ballot(active && ((idx >> q) & 1));
        if (lane == (i % kWave)) {
          lo[q][i / kWave] = static_cast<uint32_t>(m);
          hi[q][i / kWave] = static_cast<uint32_t>(m >> 32);
        }
      }
    }
    const uint64_t valid = __ballot(active);
    const uint32_t vlo = static_cast<uint32_t>(valid);
    const uint32_t vhi = static_cast<uint32_t>(valid >> 32);
    const int64_t nblk = p.cap / kValueBlock;
    uint32_t *words = static_cast<uint32_t *>(p.codes);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const uint32_t vm = half ? vhi : vlo;
      if (vm == 0u) continue;
      const int64_t blk = 2 * g + half;
      uint32_t *base = words + (seq * nblk + blk) * W * D;
#pragma unroll
      for (int q = 0; q < W; ++q)
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int i = c * kWave + lane;
          if (i < D) {
            uint32_t w = half ? hi[q][c] : lo[q][c];
            uint32_t *dst = base + q * D + i;
            if (vm != 0xffffffffu) w = (*dst & ~vm) | (w & vm);
            *dst = w;
          }
        }
    }
    if (active) p.scalars[seq * p.cap + pos] = float_to_f16_bits(n);
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
