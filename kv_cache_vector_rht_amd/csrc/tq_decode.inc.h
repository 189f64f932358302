// Query preparation, logit scan over packed keys, and split-context fused
// decode attention over packed keys and values, on the matrix cores.
//
// Estimator (pages: "TurboQuantとは？仕組み・実測精度・2026年7月時点の実装状況",
// 第2段: the QJL residual bit makes the inner-product estimate unbiased; its
// まとめ names the attention-logit computation as the accelerated operation):
//   logit(q, k) = n ( sum_i q'_i c[idx_i]
//                     + sqrt(pi/2)/D * gamma * sum_j p_j (2 sigma_j - 1) ),
// q' = R q, p = S q'. Both sums are bit-plane contractions (tq_mfma.h); the
// query side is prepared once per (batch, kv-head) group, then every key
// record is read once for all heads of its group.
#pragma once

#include "tq_device.h"
#include "tq_kernels.h"
#include "tq_mfma.h"

namespace tq {

constexpr float kSqrtHalfPi = 1.2533141373155002f;   // sqrt(pi / 2)

// ------------------------------------------------------------------ query prep

// One block (256 threads) per query head. The block stages the sketch in
// LDS (coalesced), rotates its query, projects it, and writes the four
// digit rows of its head into the group's MFMA operands.
template <int D>
__global__ __launch_bounds__(256) void query_prep_kernel(QueryPrepParams p) {
  __shared__ uint32_t s_sk[D * D / 2];       // the sketch, fp16 pairs
  __shared__ float sq[D], sp[D], sb[9], sred[8];
  const int G = p.group;
  const int n_q = p.n_kv * G;
  const int64_t hq = blockIdx.x;             // global query-head index b * n_q + h
  const int64_t b = hq / n_q;
  const int hh = static_cast<int>(hq % n_q);
  const int64_t grp = b * p.n_kv + hh / G;
  const int h = hh % G;                      // head within the group
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = lane_id();

  // issue the sketch and query loads first
  const uint4 *src = reinterpret_cast<const uint4 *>(p.sketch);
  for (int e = tid; e < D * D / 8; e += blockDim.x) reinterpret_cast<uint4 *>(s_sk)[e] = src[e];
  if (tid < D) {
    float v;
    if (p.xt == 0) v = static_cast<const float *>(p.q)[hq * D + tid];
    else if (p.xt == 1) v = bf16_bits_to_float(static_cast<const uint16_t *>(p.q)[hq * D + tid]);
    else v = f16_bits_to_float(static_cast<const uint16_t *>(p.q)[hq * D + tid]);
    sq[tid] = v * p.signs[tid];
  }
  const int NB = basis_size(p.kw);
  if (tid < NB) sb[tid] = basis_coeff(p.centroids, p.kw, basis_mask(p.kw, tid));
  __syncthreads();
  for (int hs = 1; hs < D; hs <<= 1) {
    float a = 0.f, c = 0.f;
    int i = 0;
    if (tid < D / 2) {
      i = (tid / hs) * 2 * hs + (tid % hs);
      a = sq[i];
      c = sq[i + hs];
    }
    __syncthreads();
    if (tid < D / 2) {
      sq[i] = a + c;
      sq[i + hs] = a - c;
    }
    __syncthreads();
  }
  if (tid < D) sq[tid] *= (1.0f / sqrtf(static_cast<float>(D)));
  __syncthreads();
  // p_j = sum_k S[j][k] q'_k, two threads per output
  {
    const int j = tid % D, part = tid / D;   // D = 128: part 0/1; D = 64: part 0..3
    constexpr int PARTS = 256 / D;
    constexpr int PW = D / PARTS / 2;         // sketch dwords per part (32 or 8)
    float acc = 0.f;
    // rotated start so that neighbouring threads hit different LDS banks
#pragma unroll 8
    for (int m = 0; m < PW; ++m) {
      const int k = part * (D / PARTS) + 2 * ((m + j) % PW);
      const uint32_t two = s_sk[(j * D + k) / 2];
      acc = fmaf(f16_bits_to_float(static_cast<uint16_t>(two & 0xffffu)), sq[k], acc);
      acc = fmaf(f16_bits_to_float(static_cast<uint16_t>(two >> 16)), sq[k + 1], acc);
    }
    __syncthreads();                          // the sketch is no longer read below
    float *red = reinterpret_cast<float *>(s_sk);
    red[tid] = acc;
    __syncthreads();
    if (tid < D) {
      float v = 0.f;
      for (int q = 0; q < PARTS; ++q) v += red[q * D + tid];
      sp[tid] = v;
    }
    __syncthreads();
  }
  // statistics: wave 0 -> q', wave 1 -> p
  if (wave < 2) {
    const float *x = wave == 0 ? sq : sp;
    float mx = 0.f, sm = 0.f;
    for (int i = lane; i < D; i += kWave) { mx = fmaxf(mx, fabsf(x[i])); sm += x[i]; }
    mx = wave_max(mx);
    sm = wave_sum(sm);
    if (lane == 0) { sred[2 * wave] = mx; sred[2 * wave + 1] = sm; }
  }
  if (tid == 0) {
    float mb = 0.f;
    for (int s = 0; s < NB; ++s) mb = fmaxf(mb, fabsf(sb[s]));
    sb[8] = mb;
  }
  __syncthreads();

  const int NH = D / 64;
  const int NMF = (NB + 1) * NH;
  const int rg = h / 4, hl = h % 4;
  const int el = fixed_exponent(2.0f * sb[8] * sred[0]);
  const int eq = fixed_exponent(2.0f * sred[2]);
  uint8_t *dst = p.out + grp * p.group_bytes;
  // the 16 lanes of this head in each operand: rows 4 hl + s, k-groups kg
  for (int item = tid; item < NMF * 16; item += blockDim.x) {
    const int mf = item / 16;
    const int s = (item % 16) % 4, kg = (item % 16) / 4;
    const int l = 16 * kg + 4 * hl + s;
    const bool qjl = mf >= NB * NH;
    const int plane = qjl ? 0 : mf / NH;
    const int half = mf % NH;
    const float coef = qjl ? 2.0f : 2.0f * sb[plane];
    const int e = qjl ? eq : el;
    const float *x = qjl ? sp : sq;
    uint32_t dw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int coord = slot_coord(D, kg, j, half);
      const int k = 4 * (kg & 1) + (j >> 2);
      float v = ldexpf(coef * x[coord], 7 - k + e);
      if (k == 7) v = -v;
      const uint32_t dig = signed_digits(__float2int_rn(v));
      dw[j >> 2] |= ((dig >> (8 * s)) & 0xffu) << (8 * (j & 3));
    }
    *reinterpret_cast<uint4 *>(dst + (static_cast<size_t>(rg * NMF + mf) * kWave + l) * 16) =
        make_uint4(dw[0], dw[1], dw[2], dw[3]);
  }
  // rows of absent heads in this head's last row group stay zero: the
  // group's first head of a row group clears them
  const int RG = (G + 3) / 4;
  if (hl == 0 && rg == RG - 1 && G % 4 != 0) {
    for (int item = tid; item < NMF * 64; item += blockDim.x) {
      const int mf = item / 64, l = item % 64;
      if ((l % 16) / 4 >= G % 4)
        *reinterpret_cast<uint4 *>(dst + (static_cast<size_t>(rg * NMF + mf) * kWave + l) * 16) = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  if (tid == 0) {
    float *fl = reinterpret_cast<float *>(dst + qprep_frag_bytes(D, p.kw, G)) + 4 * h;
    fl[0] = ldexpf(1.0f, -7 - el);
    fl[1] = p.centroids[(1 << p.kw) - 1] * sred[1];
    fl[2] = ldexpf(1.0f, -7 - eq);
    fl[3] = sred[3];
  }
}

template <int D>
hipError_t launch_query_prep_d(const QueryPrepParams &p, hipStream_t st) {
  const uint32_t heads = static_cast<uint32_t>(p.batch) * p.n_kv * p.group;
  if (heads == 0) return hipSuccess;
  hipLaunchKernelGGL((query_prep_kernel<D>), dim3(heads), dim3(256), 0, st, p);
  return hipGetLastError();
}

// ------------------------------------------------------------ key tiles

// One 16-key tile of a wave: lane (kg = l/16, n = l%16) holds the plane words
// of key n that its K slots need, and the key's fp16 scalars.
template <int D, int KW>
struct KeyTile {
  static constexpr int NH = D / 64;
  uint32_t w[KW + 1][NH];
  float n, g;
};

template <int D, int KW>
__device__ __forceinline__ void load_key_tile(const uint8_t *kcodes, const uint16_t *kscalars, int64_t slot0,
                                              int64_t t, int64_t n_keys, KeyTile<D, KW> &kt) {
  constexpr int REC = (KW + 1) * D / 8;
  const int lane = lane_id();
  const int wh = (lane / 16) >> 1;
  if (t < n_keys) {
    const uint8_t *rec = kcodes + (slot0 + t) * REC;
#pragma unroll
    for (int q = 0; q <= KW; ++q) {
      if (D == 128) {
        const uint2 u = *reinterpret_cast<const uint2 *>(rec + q * 16 + wh * 8);
        kt.w[q][0] = u.x;
        kt.w[q][D == 128 ? 1 : 0] = u.y;
      } else {
        kt.w[q][0] = *reinterpret_cast<const uint32_t *>(rec + q * 8 + wh * 4);
      }
    }
    const uint32_t sc = reinterpret_cast<const uint32_t *>(kscalars)[slot0 + t];
    kt.n = f16_bits_to_float(static_cast<uint16_t>(sc & 0xffffu));
    kt.g = f16_bits_to_float(static_cast<uint16_t>(sc >> 16));
  } else {
#pragma unroll
    for (int q = 0; q <= KW; ++q)
#pragma unroll
      for (int hf = 0; hf < KeyTile<D, KW>::NH; ++hf) kt.w[q][hf] = 0u;
    kt.n = 0.f;
    kt.g = 0.f;
  }
}

// Accumulate the key planes and the sign plane of one tile for NRG row groups.
template <int D, int KW, int NRG>
__device__ __forceinline__ void key_tile_mfma(const KeyTile<D, KW> &kt, const v4i (&a)[NRG][(Basis<KW>::N + 1) * (D / 64)],
                                              const uint32_t (&mask)[4], int nrg, v4i (&clm)[NRG], v4i (&cqj)[NRG]) {
  constexpr int NB = Basis<KW>::N;
  constexpr int NH = D / 64;
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg) { clm[rg] = v4i{0, 0, 0, 0}; cqj[rg] = v4i{0, 0, 0, 0}; }
#pragma unroll
  for (int s = 0; s < NB; ++s) {
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      uint32_t w = 0u;
#pragma unroll
      for (int q = 0; q < KW; ++q)
        if ((Basis<KW>::M[s] >> q) & 1) w ^= kt.w[q][hf];
      const v4i bv = expand_bits(w, mask);
#pragma unroll
      for (int rg = 0; rg < NRG; ++rg)
        if (rg < nrg) clm[rg] = mfma_i8(a[rg][s * NH + hf], bv, clm[rg]);
    }
  }
#pragma unroll
  for (int hf = 0; hf < NH; ++hf) {
    const v4i bv = expand_bits(kt.w[KW][hf], mask);
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg)
      if (rg < nrg) cqj[rg] = mfma_i8(a[rg][NB * NH + hf], bv, cqj[rg]);
  }
}

__device__ __forceinline__ float tile_logit(const v4i &clm, const v4i &cqj, const float *fl, float n, float g,
                                            float kappa) {
  const float lm = fmaf(combine_digits(clm), fl[0], -fl[1]);
  const float qj = fmaf(combine_digits(cqj), fl[2], -fl[3]);
  return n * fmaf(kappa * g, qj, lm);
}

template <int D, int KW, int NRG>
__device__ __forceinline__ void load_afrags(const uint8_t *frag, int rg0, int nrg, v4i (&a)[NRG][(Basis<KW>::N + 1) * (D / 64)]) {
  constexpr int NMF = (Basis<KW>::N + 1) * (D / 64);
  const int lane = lane_id();
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
    for (int mf = 0; mf < NMF; ++mf) {
      if (rg < nrg) {
        const uint4 u = *reinterpret_cast<const uint4 *>(frag + ((static_cast<size_t>(rg0 + rg) * NMF + mf) * kWave + lane) * 16);
        a[rg][mf] = v4i{static_cast<int>(u.x), static_cast<int>(u.y), static_cast<int>(u.z), static_cast<int>(u.w)};
      } else {
        a[rg][mf] = v4i{0, 0, 0, 0};
      }
    }
}

__device__ __forceinline__ void lane_masks(uint32_t (&mask)[4]) {
  const int kk = 4 * ((lane_id() / 16) & 1);
#pragma unroll
  for (int r = 0; r < 4; ++r) mask[r] = 0x01010101u << (kk + r);
}

// ------------------------------------------------------------------ logits

constexpr int kLogitTilesPerWave = 4;

template <int D, int KW, int NRG>
__global__ __launch_bounds__(256) void logits_kernel(LogitsParams p) {
  constexpr int NMF = (Basis<KW>::N + 1) * (D / 64);
  const int G = p.group;
  const int n_q = p.n_kv * G;
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / p.n_kv;
  const int64_t kvh = bh % p.n_kv;
  const uint8_t *prep = p.qprep + bh * p.group_bytes;
  const float *fl = reinterpret_cast<const float *>(prep + p.frag_bytes);
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int kg = lane / 16;
  uint32_t mask[4];
  lane_masks(mask);
  const int64_t slot0 = bh * p.cap;
  const float kappa = kSqrtHalfPi / static_cast<float>(D);
  const int64_t tile0 = (static_cast<int64_t>(blockIdx.x) * 4 + wave) * kLogitTilesPerWave;
  const int RG = (G + 3) / 4;
  for (int rg0 = 0; rg0 < RG; rg0 += NRG) {
    const int nrg = min(NRG, RG - rg0);
    v4i a[NRG][NMF];
    load_afrags<D, KW, NRG>(prep, rg0, nrg, a);
    KeyTile<D, KW> kt[kLogitTilesPerWave];
#pragma unroll
    for (int it = 0; it < kLogitTilesPerWave; ++it)
      load_key_tile<D, KW>(p.kcodes, p.kscalars, slot0, (tile0 + it) * 16 + (lane % 16), p.n_keys, kt[it]);
#pragma unroll
    for (int it = 0; it < kLogitTilesPerWave; ++it) {
      const int64_t t = (tile0 + it) * 16 + (lane % 16);
      if ((tile0 + it) * 16 >= p.n_keys) break;
      v4i clm[NRG], cqj[NRG];
      key_tile_mfma<D, KW, NRG>(kt[it], a, mask, nrg, clm, cqj);
#pragma unroll
      for (int rg = 0; rg < NRG; ++rg) {
        const int h = 4 * (rg0 + rg) + kg;
        if (rg < nrg && h < G && t < p.n_keys)
          p.logits[(b * n_q + kvh * G + h) * p.n_keys + t] = tile_logit(clm[rg], cqj[rg], fl + 4 * h, kt[it].n, kt[it].g, kappa);
      }
    }
  }
}

template <int D>
hipError_t launch_logits_d(const LogitsParams &p, int w, hipStream_t st) {
  if (p.n_keys == 0 || p.batch == 0 || p.n_kv == 0) return hipSuccess;
  const int64_t keys_per_block = 4 * kLogitTilesPerWave * 16;
  dim3 grid(static_cast<uint32_t>((p.n_keys + keys_per_block - 1) / keys_per_block),
            static_cast<uint32_t>(p.batch) * p.n_kv);
  const bool two = p.group > 4 && w <= 3;
#define TQ_LG(WW)                                                                          \
  if (two) hipLaunchKernelGGL((logits_kernel<D, WW, 2>), grid, dim3(256), 0, st, p);      \
  else hipLaunchKernelGGL((logits_kernel<D, WW, 1>), grid, dim3(256), 0, st, p);
  switch (w) {
    case 1: TQ_LG(1); break;
    case 2: TQ_LG(2); break;
    case 3: TQ_LG(3); break;
    default: TQ_LG(4);
  }
#undef TQ_LG
  return hipGetLastError();
}

// ------------------------------------------------------------ decode attend

// One block (4 waves) per (batch*kv-head, context split of SPLIT tokens):
//  1. scaled logits of the split's tokens for all G heads (key MFMA) -> LDS
//  2. per head: m = max, l = sum exp(logit - m); weights exp(logit - m) * n_v
//  3. weights -> fixed-point int8 digit operands in LDS (one shared
//     exponent per block, from the largest value norm)
//  4. value planes x weights on the matrix cores, int32 over the split
//  5. partials {m, l, acc[D]} per head, acc in the rotated domain
template <int D, int KW, int VW, int NRG>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeParams p) {
  constexpr int NMF = (Basis<KW>::N + 1) * (D / 64);
  constexpr int NBV = Basis<VW>::N;
  constexpr int NT = D / 64;                 // value N-tiles (16 coords) per wave
  extern __shared__ float smem[];
  const int G = p.group;
  const int SPLIT = p.split;
  const int RG = (G + 3) / 4;
  float *sl = smem;                                        // [G][SPLIT]
  float *snv = sl + G * SPLIT;                             // [SPLIT]
  uint8_t *fragv = reinterpret_cast<uint8_t *>(snv + SPLIT);   // [RG][SPLIT/64][64][16]
  float *sstat = reinterpret_cast<float *>(fragv + static_cast<size_t>(RG) * (SPLIT / 64) * 1024);  // [G][4]
  double *ssw = reinterpret_cast<double *>(sstat + 4 * G);   // [G]
  float *sred = reinterpret_cast<float *>(ssw + G);          // [8]

  const int64_t bh = blockIdx.y;
  const int64_t b = bh / p.n_kv;
  const int split = blockIdx.x;
  int64_t ctx = p.ctx_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > p.max_ctx ? p.max_ctx : ctx);
  const int64_t t_beg = static_cast<int64_t>(split) * SPLIT;
  const int n_t = static_cast<int>(min(static_cast<int64_t>(SPLIT), ctx - t_beg));
  float *part = p.partials + (bh * p.n_splits + split) * G * (D + 2);
  const int tid = threadIdx.x;
  if (n_t <= 0) {
    for (int i = tid; i < G * (D + 2); i += blockDim.x) part[i] = ((i % (D + 2)) == 0) ? -INFINITY : 0.f;
    return;
  }
  const uint8_t *prep = p.qprep + bh * p.group_bytes;
  const float *fl = reinterpret_cast<const float *>(prep + p.frag_bytes);
  const int wave = tid / kWave;
  const int lane = lane_id();
  const int kg = lane / 16;
  uint32_t mask[4];
  lane_masks(mask);
  const int64_t slot0 = bh * p.cap + t_beg;
  const float kappa = kSqrtHalfPi / static_cast<float>(D);
  const int n_tiles16 = (n_t + 15) / 16;

  // 1. logits
  for (int rg0 = 0; rg0 < RG; rg0 += NRG) {
    const int nrg = min(NRG, RG - rg0);
    v4i a[NRG][NMF];
    load_afrags<D, KW, NRG>(prep, rg0, nrg, a);
    for (int tile = wave; tile < n_tiles16; tile += 4) {
      const int tt = tile * 16 + (lane % 16);
      KeyTile<D, KW> kt;
      load_key_tile<D, KW>(p.kcodes, p.kscalars, slot0, tt, n_t, kt);
      v4i clm[NRG], cqj[NRG];
      key_tile_mfma<D, KW, NRG>(kt, a, mask, nrg, clm, cqj);
#pragma unroll
      for (int rg = 0; rg < NRG; ++rg) {
        const int h = 4 * (rg0 + rg) + kg;
        if (rg < nrg && h < G && tt < n_t)
          sl[h * SPLIT + tt] = tile_logit(clm[rg], cqj[rg], fl + 4 * h, kt.n, kt.g, kappa) * p.sm_scale;
      }
    }
  }
  for (int tt = tid; tt < n_t; tt += blockDim.x) snv[tt] = f16_bits_to_float(p.vscalars[slot0 + tt]);
  __syncthreads();

  // 2. softmax statistics and weights; the largest value norm fixes the exponent
  float nvm = 0.f;
  for (int tt = lane; tt < n_t; tt += kWave) nvm = fmaxf(nvm, snv[tt]);
  nvm = wave_max(nvm);
  const int ew = fixed_exponent(nvm);
  for (int h = wave; h < G; h += 4) {
    float m = -INFINITY;
    for (int tt = lane; tt < n_t; tt += kWave) m = fmaxf(m, sl[h * SPLIT + tt]);
    m = wave_max(m);
    float l = 0.f;
    for (int tt = lane; tt < n_t; tt += kWave) {
      const float e = __expf(sl[h * SPLIT + tt] - m);
      l += e;
      sl[h * SPLIT + tt] = e * snv[tt];
    }
    l = wave_sum(l);
    if (lane == 0) { sstat[4 * h] = m; sstat[4 * h + 1] = l; }
  }
  __syncthreads();

  // 3. weight operands: row (local head, digit), K slot -> token of a 64-token tile
  const int n_tiles64 = (n_t + 63) / 64;
  for (int row = tid; row < RG * n_tiles64 * kWave; row += blockDim.x) {
    const int l = row % kWave;
    const int tile = (row / kWave) % n_tiles64;
    const int rg = row / (kWave * n_tiles64);
    const int m = l % 16, kgl = l / 16;
    const int h = 4 * rg + m / 4, s = m % 4;
    uint32_t dw[4] = {0u, 0u, 0u, 0u};
    if (h < G) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int tok = tile * 64 + slot_coord(64, kgl, j, 0);
        const int k = 4 * (kgl & 1) + (j >> 2);
        if (tok < n_t) {
          float v = ldexpf(sl[h * SPLIT + tok], 7 - k + ew);
          if (k == 7) v = -v;
          const uint32_t dig = signed_digits(__float2int_rn(v));
          dw[j >> 2] |= ((dig >> (8 * s)) & 0xffu) << (8 * (j & 3));
        }
      }
    }
    *reinterpret_cast<uint4 *>(fragv + (static_cast<size_t>(rg) * (SPLIT / 64) + tile) * 1024 + l * 16) =
        make_uint4(dw[0], dw[1], dw[2], dw[3]);
  }
  // exact sum of the effective weights: sum_t int(w_t 2^(7-k+ew)) 2^k, per head
  for (int h = wave; h < G; h += 4) {
    double acc = 0.0;
    for (int tt = lane; tt < n_t; tt += kWave) {
      const int k = tt & 7;   // token 8*jb + k of a 32-token word carries weight 2^k
      float v = ldexpf(sl[h * SPLIT + tt], 7 - k + ew);
      acc += static_cast<double>(__float2int_rn(v)) * static_cast<double>(1 << k);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, kWave);
    if (lane == 0) ssw[h] = acc;
  }
  __syncthreads();

  // 4. value planes on the matrix cores; wave w owns coordinates [16*NT*w, 16*NT*(w+1))
  const int64_t nblk = p.cap / kValueBlock;
  const int64_t blk0 = t_beg / kValueBlock;
  float vb[NBV];
  for (int s = 0; s < NBV; ++s) vb[s] = basis_coeff(p.vcent, VW, Basis<VW>::M[s]);
  const float cvmax = p.vcent[(1 << VW) - 1];
  for (int rg0 = 0; rg0 < RG; rg0 += NRG) {
    const int nrg = min(NRG, RG - rg0);
    v4i acc[NRG][NBV][NT];
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
      for (int s = 0; s < NBV; ++s)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[rg][s][nt] = v4i{0, 0, 0, 0};
    for (int tile = 0; tile < n_tiles64; ++tile) {
      v4i av[NRG];
#pragma unroll
      for (int rg = 0; rg < NRG; ++rg) {
        if (rg < nrg) {
          const uint4 u = *reinterpret_cast<const uint4 *>(fragv + (static_cast<size_t>(rg0 + rg) * (SPLIT / 64) + tile) * 1024 + lane * 16);
          av[rg] = v4i{static_cast<int>(u.x), static_cast<int>(u.y), static_cast<int>(u.z), static_cast<int>(u.w)};
        }
      }
      const int64_t blk = blk0 + 2 * tile + (kg >> 1);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int coord = (wave * NT + nt) * 16 + (lane % 16);
        uint32_t pw[VW];
        if (2 * tile + (kg >> 1) < (n_t + kValueBlock - 1) / kValueBlock) {
          const uint32_t *src = p.vcodes + ((bh * nblk + blk) * VW) * D + coord;
#pragma unroll
          for (int q = 0; q < VW; ++q) pw[q] = src[q * D];
        } else {
#pragma unroll
          for (int q = 0; q < VW; ++q) pw[q] = 0u;
        }
#pragma unroll
        for (int s = 0; s < NBV; ++s) {
          uint32_t w = 0u;
#pragma unroll
          for (int q = 0; q < VW; ++q)
            if ((Basis<VW>::M[s] >> q) & 1) w ^= pw[q];
          const v4i bv = expand_bits(w, mask);
#pragma unroll
          for (int rg = 0; rg < NRG; ++rg)
            if (rg < nrg) acc[rg][s][nt] = mfma_i8(av[rg], bv, acc[rg][s][nt]);
        }
      }
    }
    // 5. epilogue: acc = (2 sum_S beta_S X_S - c_max SW) / 2^(7+ew)
    const float inv = ldexpf(1.0f, -7 - ew);
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) {
      const int h = 4 * (rg0 + rg) + kg;
      if (rg < nrg && h < G) {
        const float sw = static_cast<float>(ssw[h]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          float x = 0.f;
#pragma unroll
          for (int s = 0; s < NBV; ++s) x = fmaf(vb[s], combine_digits(acc[rg][s][nt]), x);
          const int coord = (wave * NT + nt) * 16 + (lane % 16);
          part[h * (D + 2) + 2 + coord] = fmaf(2.0f, x, -cvmax * sw) * inv;
        }
      }
    }
  }
  for (int h = tid; h < G; h += blockDim.x) {
    part[h * (D + 2)] = sstat[4 * h];
    part[h * (D + 2) + 1] = sstat[4 * h + 1];
  }
}

// Merge the splits of one (batch, query head) with log-sum-exp weights, then
// rotate back: out = diag(s_v) H acc / sqrt(D).
template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecodeParams p) {
  __shared__ float s[D];
  const int G = p.group;
  const int n_q = p.n_kv * G;
  const int64_t bq = blockIdx.x;             // b * n_q + h
  const int64_t b = bq / n_q;
  const int h = static_cast<int>(bq % n_q);
  const int64_t bh = b * p.n_kv + h / G;
  const int g = h % G;
  const int i = threadIdx.x;
  const float *base = p.partials + bh * p.n_splits * G * (D + 2) + g * (D + 2);
  const int64_t stride = static_cast<int64_t>(G) * (D + 2);
  float M = -INFINITY;
  for (int sp = 0; sp < p.n_splits; ++sp) M = fmaxf(M, base[sp * stride]);
  float lt = 0.f, acc = 0.f;
  if (M > -INFINITY) {
    for (int sp = 0; sp < p.n_splits; ++sp) {
      const float m = base[sp * stride];
      if (m == -INFINITY) continue;
      const float e = __expf(m - M);
      lt = fmaf(base[sp * stride + 1], e, lt);
      acc = fmaf(base[sp * stride + 2 + i], e, acc);
    }
  }
  s[i] = (lt > 0.f) ? acc / lt : 0.f;
  __syncthreads();
#pragma unroll
  for (int hs = 1; hs < D; hs <<= 1) {
    const float a = s[i];
    const float c = s[i ^ hs];
    __syncthreads();
    s[i] = (i & hs) ? (c - a) : (a + c);
    __syncthreads();
  }
  const float o = s[i] * p.vsigns[i] * (1.0f / sqrtf(static_cast<float>(D)));
  if (p.out_t == 0) static_cast<float *>(p.out)[bq * D + i] = o;
  else static_cast<uint16_t *>(p.out)[bq * D + i] = float_to_bf16_bits(o);
}

template <int D, int KW, int VW>
static void launch_decode_kv(const DecodeParams &p, dim3 grid, size_t shm, hipStream_t st) {
  if (p.group > 4) hipLaunchKernelGGL((decode_split_kernel<D, KW, VW, 2>), grid, dim3(256), shm, st, p);
  else hipLaunchKernelGGL((decode_split_kernel<D, KW, VW, 1>), grid, dim3(256), shm, st, p);
}

template <int D>
hipError_t launch_decode_d(const DecodeParams &p, int kw, int vw, hipStream_t st) {
  if (p.batch == 0 || p.n_kv == 0) return hipSuccess;
  dim3 grid(static_cast<uint32_t>(p.n_splits), static_cast<uint32_t>(p.batch) * p.n_kv);
  const size_t shm = decode_split_smem(D, p.group, p.split);
#define TQ_DS_V(KK)                                            \
  switch (vw) {                                                \
    case 1: launch_decode_kv<D, KK, 1>(p, grid, shm, st); break; \
    case 2: launch_decode_kv<D, KK, 2>(p, grid, shm, st); break; \
    case 3: launch_decode_kv<D, KK, 3>(p, grid, shm, st); break; \
    default: launch_decode_kv<D, KK, 4>(p, grid, shm, st);     \
  }
  switch (kw) {
    case 1: TQ_DS_V(1); break;
    case 2: TQ_DS_V(2); break;
    case 3: TQ_DS_V(3); break;
    default: TQ_DS_V(4);
  }
#undef TQ_DS_V
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint32_t rows = static_cast<uint32_t>(p.batch) * p.n_kv * p.group;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(rows), dim3(D), 0, st, p);
  return hipGetLastError();
}

}  // namespace tq
