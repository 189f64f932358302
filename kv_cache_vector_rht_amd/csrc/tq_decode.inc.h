#pragma once
// Query preparation, logit scan over packed keys, and split-context fused
// decode attention over packed keys and values.
//
// Estimator (pages: "TurboQuantとは？仕組み・実測精度・2026年7月時点の実装状況",
// 第2段, the QJL residual bit makes the inner-product estimate unbiased; the
// logit computation is the operation behind the 8x figure in its まとめ):
//   logit(q, k) = n ( sum_i q'_i c[idx_i]
//                     + sqrt(pi/2)/D * gamma * sum_j p_j (2 sigma_j - 1) )
// with q' = R q and p = S q'. The rotated query and its projection are
// computed once per query head; the scan then reads each key record once for
// all heads of its group.
#include "tq_device.h"
#include "tq_kernels.h"

namespace tq {

constexpr float kSqrtHalfPi = 1.2533141373155002f;   // sqrt(pi / 2)

// ------------------------------------------------------------------ query prep

template <int D>
__global__ __launch_bounds__(D) void query_prep_kernel(QueryPrepParams p) {
  __shared__ float s[D];
  const int64_t h = blockIdx.x;
  const int i = threadIdx.x;
  float v;
  if (p.xt == 0) v = static_cast<const float *>(p.q)[h * D + i];
  else if (p.xt == 1) v = bf16_bits_to_float(static_cast<const uint16_t *>(p.q)[h * D + i]);
  else v = f16_bits_to_float(static_cast<const uint16_t *>(p.q)[h * D + i]);
  s[i] = v * p.signs[i];
  __syncthreads();
#pragma unroll
  for (int hs = 1; hs < D; hs <<= 1) {
    const float a = s[i];
    const float b = s[i ^ hs];
    __syncthreads();
    s[i] = (i & hs) ? (b - a) : (a + b);
    __syncthreads();
  }
  const float qr = s[i] * (1.0f / sqrtf(static_cast<float>(D)));
  __syncthreads();
  s[i] = qr;
  p.out[(h * 2 + 0) * D + i] = qr;
  __syncthreads();
  const uint32_t *row = reinterpret_cast<const uint32_t *>(p.sketch + static_cast<int64_t>(i) * D);
  float acc = 0.f;
#pragma unroll 8
  for (int k = 0; k < D; k += 2) {
    const uint32_t two = row[k / 2];
    acc = fmaf(f16_bits_to_float(static_cast<uint16_t>(two & 0xffffu)), s[k], acc);
    acc = fmaf(f16_bits_to_float(static_cast<uint16_t>(two >> 16)), s[k + 1], acc);
  }
  p.out[(h * 2 + 1) * D + i] = acc;
}

template <int D>
hipError_t launch_query_prep_d(const QueryPrepParams &p, hipStream_t st) {
  if (p.n_heads == 0) return hipSuccess;
  hipLaunchKernelGGL((query_prep_kernel<D>), dim3(static_cast<uint32_t>(p.n_heads)), dim3(D), 0, st, p);
  return hipGetLastError();
}

// ------------------------------------------------------------ per-key logits

// Logits of one key against heads [h0, h0 + nh) (nh <= 4) of the group whose
// prepared queries sit in LDS as sq[g][0][D] = q', sq[g][1][D] = p.
template <int D, int W>
__device__ __forceinline__ void key_logits4(const uint32_t (&rec)[(W + 1) * D / 32], float n, float gamma,
                                            const float *sq, const float *cent, int h0, int nh,
                                            float (&out)[4]) {
  constexpr int NW = D / 32;
  float lm[4] = {0.f, 0.f, 0.f, 0.f};
  float qj[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int jw = 0; jw < NW; ++jw) {
    const uint32_t sw = rec[W * NW + jw];
#pragma unroll
    for (int jb = 0; jb < 32; ++jb) {
      const int i = jw * 32 + jb;
      int idx = 0;
#pragma unroll
      for (int q = 0; q < W; ++q) idx |= static_cast<int>((rec[q * NW + jw] >> jb) & 1u) << q;
      const float c = cent[idx];
      const bool pos = (sw >> jb) & 1u;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (g < nh) {
          const float *qg = sq + (h0 + g) * 2 * D;
          lm[g] = fmaf(qg[i], c, lm[g]);
          const float pj = qg[D + i];
          qj[g] += pos ? pj : -pj;
        }
      }
    }
  }
  const float kg = kSqrtHalfPi / static_cast<float>(D) * gamma;
#pragma unroll
  for (int g = 0; g < 4; ++g) out[g] = n * fmaf(kg, qj[g], lm[g]);
}

template <int D, int W>
__device__ __forceinline__ void load_key(const uint8_t *kcodes, const uint16_t *kscalars, int64_t slot,
                                         uint32_t (&rec)[(W + 1) * D / 32], float &n, float &gamma) {
  constexpr int REC = (W + 1) * D / 8;
  const uint8_t *r = kcodes + slot * REC;
  if (D == 128) {
#pragma unroll
    for (int q = 0; q <= W; ++q) {
      const uint4 u = *reinterpret_cast<const uint4 *>(r + q * 16);
      rec[q * 4 + 0] = u.x; rec[q * 4 + 1] = u.y; rec[q * 4 + 2] = u.z; rec[q * 4 + 3] = u.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q <= W; ++q) {
      const uint2 u = *reinterpret_cast<const uint2 *>(r + q * 8);
      rec[q * 2 + 0] = u.x; rec[q * 2 + 1] = u.y;
    }
  }
  const uint32_t sc = reinterpret_cast<const uint32_t *>(kscalars)[slot];
  n = f16_bits_to_float(static_cast<uint16_t>(sc & 0xffffu));
  gamma = f16_bits_to_float(static_cast<uint16_t>(sc >> 16));
}

// ------------------------------------------------------------------ logits

template <int D, int W>
__global__ __launch_bounds__(256) void logits_kernel(LogitsParams p) {
  extern __shared__ float smem[];
  const int G = p.group;
  const int n_q = p.n_kv * G;
  float *sq = smem;                          // [G][2][D]
  float *cent = smem + G * 2 * D;            // [2^W]
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / p.n_kv;
  const int64_t kvh = bh % p.n_kv;
  const float *qsrc = p.qprep + (b * n_q + kvh * G) * 2 * D;
  for (int i = threadIdx.x; i < G * 2 * D; i += blockDim.x) sq[i] = qsrc[i];
  if (threadIdx.x < (1 << W)) cent[threadIdx.x] = p.centroids[threadIdx.x];
  __syncthreads();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= p.n_keys) return;
  uint32_t rec[(W + 1) * D / 32];
  float n, gamma;
  load_key<D, W>(p.kcodes, p.kscalars, bh * p.cap + t, rec, n, gamma);
  float *dst = p.logits + (b * n_q + kvh * G) * p.n_keys + t;
  for (int h0 = 0; h0 < G; h0 += 4) {
    const int nh = min(4, G - h0);
    float out[4];
    key_logits4<D, W>(rec, n, gamma, sq, cent, h0, nh, out);
#pragma unroll
    for (int g = 0; g < 4; ++g)
      if (g < nh) dst[(h0 + g) * p.n_keys] = out[g];
  }
}

template <int D>
hipError_t launch_logits_d(const LogitsParams &p, int w, hipStream_t st) {
  if (p.n_keys == 0 || p.batch == 0 || p.n_kv == 0) return hipSuccess;
  dim3 grid(static_cast<uint32_t>((p.n_keys + 255) / 256), static_cast<uint32_t>(p.batch) * p.n_kv);
  const size_t shm = (static_cast<size_t>(p.group) * 2 * D + 16) * sizeof(float);
  switch (w) {
    case 1: hipLaunchKernelGGL((logits_kernel<D, 1>), grid, dim3(256), shm, st, p); break;
    case 2: hipLaunchKernelGGL((logits_kernel<D, 2>), grid, dim3(256), shm, st, p); break;
    case 3: hipLaunchKernelGGL((logits_kernel<D, 3>), grid, dim3(256), shm, st, p); break;
    default: hipLaunchKernelGGL((logits_kernel<D, 4>), grid, dim3(256), shm, st, p);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------ decode attend

// One block per (batch*kv-head, context split): logits for the split's tokens,
// per-head softmax statistics (max m, sum l of exp(scaled logit - m)), and the
// weighted sum of decoded values in the rotated domain. Partials are written
// as [G][D+2] = {m, l, acc[D]}.
template <int D, int KW, int VW>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeParams p) {
  extern __shared__ float smem[];
  const int G = p.group;
  const int n_q = p.n_kv * G;
  const int SPLIT = p.split;
  float *sq = smem;                          // [G][2][D]
  float *sl = sq + G * 2 * D;                // [G][SPLIT]
  float *snv = sl + G * SPLIT;               // [SPLIT]
  float *skc = snv + SPLIT;                  // [16]
  float *svc = skc + 16;                     // [16]
  float *sml = svc + 16;                     // [G][2]

  const int64_t bh = blockIdx.y;
  const int64_t b = bh / p.n_kv;
  const int64_t kvh = bh % p.n_kv;
  const int split = blockIdx.x;
  int64_t ctx = p.ctx_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > p.max_ctx ? p.max_ctx : ctx);
  const int64_t t_beg = static_cast<int64_t>(split) * SPLIT;
  const int64_t t_end = min(t_beg + SPLIT, ctx);
  const int n_t = static_cast<int>(t_end - t_beg);
  float *part = p.partials + (bh * p.n_splits + split) * G * (D + 2);

  if (n_t <= 0) {
    for (int i = threadIdx.x; i < G * (D + 2); i += blockDim.x) {
      const int c = i % (D + 2);
      part[i] = (c == 0) ? -INFINITY : 0.f;
    }
    return;
  }

  const float *qsrc = p.qprep + (b * n_q + kvh * G) * 2 * D;
  for (int i = threadIdx.x; i < G * 2 * D; i += blockDim.x) sq[i] = qsrc[i];
  if (threadIdx.x < (1 << KW)) skc[threadIdx.x] = p.kcent[threadIdx.x];
  if (threadIdx.x < (1 << VW)) svc[threadIdx.x] = p.vcent[threadIdx.x];
  __syncthreads();

  // phase 1: scaled logits and value norms
  for (int tt = threadIdx.x; tt < n_t; tt += blockDim.x) {
    const int64_t slot = bh * p.cap + t_beg + tt;
    uint32_t rec[(KW + 1) * D / 32];
    float n, gamma;
    load_key<D, KW>(p.kcodes, p.kscalars, slot, rec, n, gamma);
    for (int h0 = 0; h0 < G; h0 += 4) {
      const int nh = min(4, G - h0);
      float out[4];
      key_logits4<D, KW>(rec, n, gamma, sq, skc, h0, nh, out);
#pragma unroll
      for (int g = 0; g < 4; ++g)
        if (g < nh) sl[(h0 + g) * SPLIT + tt] = out[g] * p.sm_scale;
    }
    snv[tt] = f16_bits_to_float(p.vscalars[slot]);
  }
  __syncthreads();

  // phase 2: softmax statistics, one wave per head
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int n_waves = blockDim.x / kWave;
  for (int g = wave; g < G; g += n_waves) {
    float m = -INFINITY;
    for (int tt = lane; tt < n_t; tt += kWave) m = fmaxf(m, sl[g * SPLIT + tt]);
    m = wave_max(m);
    float l = 0.f;
    for (int tt = lane; tt < n_t; tt += kWave) {
      const float e = __expf(sl[g * SPLIT + tt] - m);
      sl[g * SPLIT + tt] = e;
      l += e;
    }
    l = wave_sum(l);
    if (lane == 0) { sml[2 * g] = m; sml[2 * g + 1] = l; }
  }
  __syncthreads();

  // phase 3: acc[g][i] = sum_t w[g][t] * n_t * c_v[idx_t,i]
  constexpr int NP = 256 / D;                // threads per coordinate
  constexpr int MAXH = 32 / NP;              // heads per thread (G <= 32)
  const int i = threadIdx.x % D;
  const int hp = threadIdx.x / D;
  float acc[MAXH];
#pragma unroll
  for (int s = 0; s < MAXH; ++s) acc[s] = 0.f;
  const int64_t nblk = p.cap / kValueBlock;
  const int64_t blk0 = t_beg / kValueBlock;
  const int nb = (n_t + kValueBlock - 1) / kValueBlock;
  for (int kb = 0; kb < nb; ++kb) {
    uint32_t wv[VW];
    const uint32_t *src = p.vcodes + ((bh * nblk + blk0 + kb) * VW) * D + i;
#pragma unroll
    for (int q = 0; q < VW; ++q) wv[q] = src[q * D];
    const int jn = min(kValueBlock, n_t - kb * kValueBlock);
    for (int j = 0; j < jn; ++j) {
      int idx = 0;
#pragma unroll
      for (int q = 0; q < VW; ++q) idx |= static_cast<int>((wv[q] >> j) & 1u) << q;
      const int tt = kb * kValueBlock + j;
      const float val = svc[idx] * snv[tt];
#pragma unroll
      for (int s = 0; s < MAXH; ++s) {
        const int g = hp + s * NP;
        if (g < G) acc[s] = fmaf(sl[g * SPLIT + tt], val, acc[s]);
      }
    }
  }
#pragma unroll
  for (int s = 0; s < MAXH; ++s) {
    const int g = hp + s * NP;
    if (g < G) {
      part[g * (D + 2) + 2 + i] = acc[s];
      if (i == 0) { part[g * (D + 2)] = sml[2 * g]; part[g * (D + 2) + 1] = sml[2 * g + 1]; }
    }
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

template <int D>
hipError_t launch_decode_d(const DecodeParams &p, int kw, int vw, hipStream_t st) {
  if (p.batch == 0 || p.n_kv == 0) return hipSuccess;
  dim3 grid(static_cast<uint32_t>(p.n_splits), static_cast<uint32_t>(p.batch) * p.n_kv);
  const size_t shm = decode_split_smem(D, p.group, p.split);
#define TQ_DS(KK, VV) hipLaunchKernelGGL((decode_split_kernel<D, KK, VV>), grid, dim3(256), shm, st, p)
#define TQ_DS_V(KK)                                       \
  switch (vw) {                                           \
    case 1: TQ_DS(KK, 1); break;                          \
    case 2: TQ_DS(KK, 2); break;                          \
    case 3: TQ_DS(KK, 3); break;                          \
    default: TQ_DS(KK, 4);                                \
  }
  switch (kw) {
    case 1: TQ_DS_V(1); break;
    case 2: TQ_DS_V(2); break;
    case 3: TQ_DS_V(3); break;
    default: TQ_DS_V(4);
  }
#undef TQ_DS_V
#undef TQ_DS
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint32_t rows = static_cast<uint32_t>(p.batch) * p.n_kv * p.group;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(rows), dim3(D), 0, st, p);
  return hipGetLastError();
}

}  // namespace tq
