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
  {
    constexpr int N = D * D / 8 / 256;
    const uint4 *src = reinterpret_cast<const uint4 *>(p.sketch);
    uint4 v[N];
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = src[k * 256 + tid];
#pragma unroll
    for (int k = 0; k < N; ++k) reinterpret_cast<uint4 *>(s_sk)[k * 256 + tid] = v[k];
  }
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
// of key n that its K slots need, and the key's raw fp16 scalar pair.
template <int D, int KW>
struct KeyTile {
  static constexpr int NH = D / 64;
  uint32_t w[KW + 1][NH];
  uint32_t sc;
  __device__ __forceinline__ float norm() const { return f16_bits_to_float(static_cast<uint16_t>(sc & 0xffffu)); }
  __device__ __forceinline__ float gamma() const { return f16_bits_to_float(static_cast<uint16_t>(sc >> 16)); }
};

// Loads are issued unconditionally (past the end the slot is clamped to the
// first one): a key's words only feed its own MFMA column, and columns past
// the end are never stored, so no branch holds the loads back.
template <int D, int KW>
__device__ __forceinline__ void load_key_tile(const uint8_t *kcodes, const uint16_t *kscalars, int64_t slot0,
                                              int64_t t, int64_t n_keys, KeyTile<D, KW> &kt) {
  constexpr int REC = (KW + 1) * D / 8;
  const int lane = lane_id();
  const int wh = (lane / 16) >> 1;
  const int64_t tc = (t < n_keys) ? t : 0;
  const uint8_t *rec = kcodes + (slot0 + tc) * REC;
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
  kt.sc = reinterpret_cast<const uint32_t *>(kscalars)[slot0 + tc];
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

// fl = {inv_lm, cst_lm, inv_qj, cst_qj} of the lane's head (held in
// registers: a global load here would make the wait for it also wait for
// every prefetched tile issued before it).
__device__ __forceinline__ float tile_logit(const v4i &clm, const v4i &cqj, const float4 &fl, float n, float g,
                                            float kappa) {
  const float lm = fmaf(combine_digits(clm), fl.x, -fl.y);
  const float qj = fmaf(combine_digits(cqj), fl.z, -fl.w);
  return n * fmaf(kappa * g, qj, lm);
}

// Per-head constants of the NRG row groups this lane's C rows belong to.
template <int NRG>
__device__ __forceinline__ void load_head_consts(const float *fl, int h_base, int n_heads, float4 (&fh)[NRG]) {
  const int kg = lane_id() / 16;
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg) {
    const int h = h_base + 4 * rg + kg;
    fh[rg] = (h < n_heads) ? *reinterpret_cast<const float4 *>(fl + 4 * h) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
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
    float4 fh[NRG];
    load_head_consts<NRG>(fl, 4 * rg0, G, fh);
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
          p.logits[(b * n_q + kvh * G + h) * p.n_keys + t] = tile_logit(clm[rg], cqj[rg], fh[rg], kt[it].norm(), kt[it].gamma(), kappa);
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

// Pipeline stages of the decode kernel: while the block computes on one
// split, the direct-to-LDS loads of the next two are in flight.
constexpr int kStages = 3;

// Block layout: D/16 waves. Wave w owns the 16-key tiles w, w + NW, ... of
// every split (their logits and attention weights) and the value
// coordinates [16 w, 16 w + 16). Its share of a split is staged in a region
// of LDS that only it reads, so no barrier guards the staging:
//   [0, OFF_S)         key tiles, 16 x REC bytes each; for d = 128 plane-major
//                      (the 16 keys' words of plane 0, then of plane 1, ...)
//   [OFF_S, OFF_V)     the tiles' key scalar pairs (64 B per tile), then their
//                      value norms (32 B per tile)
//   [OFF_V, ...)       value words: [32-token block][plane][16 coordinates]
template <int D, int KW, int VW>
struct DecodeShape {
  static constexpr int S = kDecodeSplit;
  static constexpr int NW = D / 16;
  static constexpr int THREADS = NW * kWave;
  static constexpr int KT = S / 16 / NW;             // key tiles per wave
  static constexpr int VT = S / 64;                  // 64-token value tiles
  static constexpr int REC = (KW + 1) * D / 8;       // record bytes = 16-byte units per key tile
  static constexpr int KI = (REC + 63) / 64;         // loads per key tile
  static constexpr int SU = 6 * KT;                  // scalar units
  static constexpr int VU = (S / 32) * VW * 4;       // value units
  static constexpr int VI = (VU + 63) / 64;
  static constexpr int P = KT * KI + 1 + VI;         // loads per wave per split
  static constexpr int OFF_S = KT * REC * 16;
  static constexpr int OFF_V = OFF_S + (SU * 16 + 255) / 256 * 256;
  static constexpr int WAVE_BYTES = OFF_V + VU * 16;
  static constexpr int STAGE_BYTES = NW * WAVE_BYTES;
};

typedef __attribute__((address_space(3))) void lds_void_t;

// The staging loads and the waits for them are written as inline assembly:
// the compiler then neither counts these loads nor adds waits for them of
// its own (it would otherwise make LDS reads wait for every staging load in
// flight). Its own waits for its own memory operations stay correct: loads
// it does not know about only make them wait longer.

// 16 bytes per lane from global memory straight into LDS at lds + 16 * lane
// (lds is the same for the whole wave and goes to M0). dma16 reads at
// base + off (base the same for the whole wave, off this lane's 32-bit byte
// offset); dma16_at at this lane's own address.
__device__ __forceinline__ uint32_t lds_m0(uint8_t *lds) {
  return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t *)lds)));
}
__device__ __forceinline__ void dma16(const void *base, uint32_t off, uint8_t *lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds_m0(lds)) : "memory");
}
__device__ __forceinline__ void dma16_at(const void *src, uint8_t *lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds_m0(lds)) : "memory");
}

// Wait until at most N vector memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Workgroup barrier over LDS data only: earlier LDS writes complete, the
// staging loads in flight are not waited for.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Issue this wave's share of split sp into its region of a stage buffer.
// Every wave issues exactly P loads. Tiles past the cache capacity load the
// sequence's first tile instead (their keys are past the context and get
// zero weight), so every address stays inside the caller's arrays.
// The sequence's arrays: wave-uniform base addresses (lane offsets from
// them stay below 4 GiB).
struct SeqArrays {
  const uint8_t *kcodes, *kscal, *vcodes, *vscal;
  int32_t cap, nblk;
};

template <int D, int KW, int VW>
__device__ __forceinline__ void issue_split(const SeqArrays &sa, int sp, uint8_t *stage, int wave) {
  using SH = DecodeShape<D, KW, VW>;
  constexpr int REC = SH::REC;
  const int lane = lane_id();
  uint8_t *wb = stage + wave * SH::WAVE_BYTES;
  const int t_beg = sp * SH::S;
  uint32_t tile0[SH::KT];
#pragma unroll
  for (int u = 0; u < SH::KT; ++u) {
    const int t = t_beg + 16 * (wave + SH::NW * u);
    tile0[u] = static_cast<uint32_t>((t < sa.cap) ? t : 0);
  }
#pragma unroll
  for (int u = 0; u < SH::KT; ++u) {
#pragma unroll
    for (int ki = 0; ki < SH::KI; ++ki) {
      const int unit = ki * 64 + lane;
      if (unit < REC) {
        // d = 128: LDS unit 16 q + i <- plane q of key i; d = 64: a plain copy
        const uint32_t lo = (D == 128) ? (unit % 16) * REC + (unit / 16) * 16 : unit * 16;
        dma16(sa.kcodes, tile0[u] * REC + lo, wb + u * REC * 16 + ki * 1024);
      }
    }
  }
  if (lane < SH::SU) {
    // lanes [0, 4 KT): key scalar pairs of tile lane/4; then value norms
    const bool key = lane < 4 * SH::KT;
    const int u = key ? lane / 4 : (lane - 4 * SH::KT) / 2;
    const int m = key ? lane % 4 : (lane - 4 * SH::KT) % 2;
    uint32_t t0 = 0;
#pragma unroll
    for (int v = 0; v < SH::KT; ++v) t0 = (u == v) ? tile0[v] : t0;
    dma16_at(key ? sa.kscal + (t0 + 4 * m) * 4 : sa.vscal + (t0 + 8 * m) * 2, wb + SH::OFF_S);
  }
#pragma unroll
  for (int vi = 0; vi < SH::VI; ++vi) {
    const int unit = vi * 64 + lane;
    if (unit < SH::VU) {
      const int blk = unit / (4 * VW), q = (unit / 4) % VW, m = unit % 4;
      int bg = t_beg / kValueBlock + blk;
      bg = (bg < sa.nblk) ? bg : 0;
      const uint32_t off = ((static_cast<uint32_t>(bg) * VW + q) * D + 16 * wave + 4 * m) * 4;
      dma16(sa.vcodes, off, wb + SH::OFF_V + vi * 1024);
    }
  }
}

// One block per (batch*kv-head, block index within the group) and the heads
// [h0, h0 + GE) of the group, GE <= 4 NRG. The block walks the splits
// blockIdx.x, blockIdx.x + gridDim.x, ... (kDecodeSplit tokens each)
// through a ring of kStages LDS buffers. Per split, each wave:
//  1. computes the logits of its key tiles for every head (key MFMA),
//     scaled by sm_scale; publishes its per-head maxima and largest value
//     norm                                                     -- barrier
//  2. merges the split maximum into the running (m, l) (online softmax,
//     m' = max(m, m_split), alpha = exp(m - m')), forms its tokens' weights
//     exp(logit - m') n_v as fixed-point int8 digits (one exponent per
//     split, from its largest value norm) written into the shared MFMA
//     operand tiles, and publishes their exact per-head sums   -- barrier
//  3. contracts the weights with its value coordinates' planes on the
//     matrix cores (int32 over the split) and folds the result into its
//     fp32 accumulators: acc = alpha acc + split sum
//  4. refills the stage buffer with the split kStages ahead.
// The block's partial {m, l, acc} goes to the workspace; merge_kernel
// combines them.
template <int D, int KW, int VW, int NRG>
__global__ __launch_bounds__(4 * D) void decode_kernel(DecodeParams p) {   // 4 D = (D / 16) waves
  using SH = DecodeShape<D, KW, VW>;
  constexpr int S = SH::S, NW = SH::NW, KT = SH::KT, VT = SH::VT, REC = SH::REC, P = SH::P;
  constexpr int NMF = (Basis<KW>::N + 1) * (D / 64);
  constexpr int NBV = Basis<VW>::N;
  constexpr int GMAX = 4 * NRG;
  constexpr int NBG = (NRG == 2 && NBV == 8) ? 4 : NBV;
  __shared__ __attribute__((aligned(1024))) uint8_t st0[SH::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[SH::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[SH::STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t sfrag[NRG * VT * 1024];
  __shared__ float spm[NW][GMAX];
  __shared__ float spnv[NW];
  __shared__ double spsw[NW][GMAX];
  __shared__ float svb[NBV];

  const int G = p.group;
  const int n_q = p.n_kv * G;
  const int GE = min(GMAX, G - p.h0);
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / p.n_kv;
  const int64_t kvh = bh % p.n_kv;
  int64_t ctx64 = p.ctx_lens[b];
  ctx64 = ctx64 < 0 ? 0 : (ctx64 > p.max_ctx ? p.max_ctx : ctx64);
  const int ctx = static_cast<int>(ctx64);
  const int n_splits = (ctx + S - 1) / S;
  const int nb = gridDim.x;
  const int bx = blockIdx.x;
  const int ns = (n_splits > bx) ? (n_splits - bx + nb - 1) / nb : 0;   // splits of this block
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = lane_id();
  const int kg = lane / 16;
  const int col = lane % 16;
  uint32_t mask[4];
  lane_masks(mask);
  const float kappa = kSqrtHalfPi / static_cast<float>(D);
  const uint8_t *prep = p.qprep + bh * p.group_bytes;
  const float *fl = reinterpret_cast<const float *>(prep + p.frag_bytes);

  if (tid < NBV) svb[tid] = basis_coeff(p.vcent, VW, basis_mask(VW, tid));
  const float cvmax = p.vcent[(1 << VW) - 1];

  float m_run[NRG], l_run[NRG], accf[NRG];
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg) { m_run[rg] = -INFINITY; l_run[rg] = 0.f; accf[rg] = 0.f; }

  SeqArrays sa;
  sa.cap = static_cast<int32_t>(p.cap);
  sa.nblk = static_cast<int32_t>(p.cap / kValueBlock);
  sa.kcodes = p.kcodes + bh * p.cap * REC;
  sa.kscal = reinterpret_cast<const uint8_t *>(p.kscalars) + bh * p.cap * 4;
  sa.vcodes = reinterpret_cast<const uint8_t *>(p.vcodes + bh * sa.nblk * VW * D);
  sa.vscal = reinterpret_cast<const uint8_t *>(p.vscalars) + bh * p.cap * 2;
  v4i a[NRG][NMF];
  float4 fh[NRG];
  if (ns > 0) {
    // split 0 and the query operands travel together; both are waited for
    // here, so no wait for the operands is left inside the split loop
    issue_split<D, KW, VW>(sa, bx, st0, wave);
    load_afrags<D, KW, NRG>(prep, p.h0 / 4, NRG, a);
    load_head_consts<NRG>(fl, p.h0, p.h0 + GE, fh);
    wait_vm<0>();
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) {
#pragma unroll
      for (int mf = 0; mf < NMF; ++mf) asm volatile("" ::"v"(a[rg][mf]));
      asm volatile("" ::"v"(fh[rg].x), "v"(fh[rg].y), "v"(fh[rg].z), "v"(fh[rg].w));
    }
    if (ns > 1) issue_split<D, KW, VW>(sa, bx + nb, st1, wave);
    if (ns > 2) issue_split<D, KW, VW>(sa, bx + 2 * nb, st2, wave);
  }

  auto step = [&](uint8_t *buf, int it) __attribute__((always_inline)) {
    const int sp = bx + it * nb;
    const int n = min(S, ctx - sp * S);
    const int ahead = min(kStages - 1, ns - 1 - it);
    if (ahead >= 2) wait_vm<2 * P>();
    else if (ahead == 1) wait_vm<P>();
    else wait_vm<0>();
    const uint8_t *wb = buf + wave * SH::WAVE_BYTES;

    // 1. logits of this wave's key tiles
    float lg[KT][NRG], nvv[KT];
    float mx[NRG];
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) mx[rg] = -INFINITY;
    float nvm = 0.f;
#pragma unroll
    for (int u = 0; u < KT; ++u) {
      const int tl = 16 * (wave + NW * u) + col;
      const uint8_t *kb = wb + u * REC * 16;
      KeyTile<D, KW> kt;
#pragma unroll
      for (int q = 0; q <= KW; ++q) {
        if constexpr (D == 128) {
          const uint2 v = *reinterpret_cast<const uint2 *>(kb + (16 * q + col) * 16 + 8 * (kg >> 1));
          kt.w[q][0] = v.x;
          kt.w[q][D == 128 ? 1 : 0] = v.y;
        } else {
          kt.w[q][0] = *reinterpret_cast<const uint32_t *>(kb + col * REC + q * 8 + 4 * (kg >> 1));
        }
      }
      kt.sc = *reinterpret_cast<const uint32_t *>(wb + SH::OFF_S + 64 * u + 4 * col);
      const uint16_t nvb = *reinterpret_cast<const uint16_t *>(wb + SH::OFF_S + 64 * KT + 32 * u + 2 * col);
      v4i clm[NRG], cqj[NRG];
      key_tile_mfma<D, KW, NRG>(kt, a, mask, NRG, clm, cqj);
      const bool valid = tl < n;
      const float kn = kt.norm(), kgm = kt.gamma();
#pragma unroll
      for (int rg = 0; rg < NRG; ++rg) {
        const float l = tile_logit(clm[rg], cqj[rg], fh[rg], kn, kgm, kappa) * p.sm_scale;
        lg[u][rg] = valid ? l : -INFINITY;
        mx[rg] = fmaxf(mx[rg], lg[u][rg]);
      }
      const float nvf = f16_bits_to_float(nvb);
      nvv[u] = valid ? nvf : 0.f;
      nvm = fmaxf(nvm, nvv[u]);
    }
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) mx[rg] = row_max16(mx[rg]);
    nvm = wave_max(nvm);
    if (col == 0) {
#pragma unroll
      for (int rg = 0; rg < NRG; ++rg) spm[wave][4 * rg + kg] = mx[rg];
    }
    if (lane == 0) spnv[wave] = nvm;
    lds_barrier();

    // 2. running statistics, weights -> operand digits, their sums
    float nvmax = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) nvmax = fmaxf(nvmax, spnv[w]);
    const int ew = fixed_exponent(nvmax);
    float alpha[NRG];
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) {
      float ms = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) ms = fmaxf(ms, spm[w][4 * rg + kg]);
      const float mn = fmaxf(m_run[rg], ms);
      alpha[rg] = (m_run[rg] == -INFINITY) ? 0.f : __expf(m_run[rg] - mn);
      m_run[rg] = mn;
      l_run[rg] *= alpha[rg];
    }
    double sw[NRG];
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) sw[rg] = 0.0;
#pragma unroll
    for (int u = 0; u < KT; ++u) {
      const int tl = 16 * (wave + NW * u) + col;
      const int vt = tl / 64, t64 = tl % 64;
      const int k = t64 & 7;
      const int kga = 2 * (t64 >> 5) + ((t64 >> 2) & 1);
      const int jb = (t64 >> 3) & 3, r = t64 & 3;
#pragma unroll
      for (int rg = 0; rg < NRG; ++rg) {
        const float e = __expf(lg[u][rg] - m_run[rg]);
        l_run[rg] += e;
        const int fx = __float2int_rn(ldexpf(e * nvv[u], 7 - k + ew));
        sw[rg] += static_cast<double>(fx) * static_cast<double>(1 << k);
        const uint32_t dig = signed_digits(k == 7 ? -fx : fx);
        uint8_t *dst = sfrag + (rg * VT + vt) * 1024 + (16 * kga + 4 * kg) * 16 + 4 * r + jb;
#pragma unroll
        for (int s = 0; s < 4; ++s) dst[16 * s] = static_cast<uint8_t>(dig >> (8 * s));
      }
    }
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) {
      const double t = row_sum16d(sw[rg]);
      if (col == 0) spsw[wave][4 * rg + kg] = t;
    }
    lds_barrier();

    // 3. value planes x weights on the matrix cores, NBG planes at a time
    //    (with 8 heads and 8 planes, two passes keep the int32 sums in registers)
    float x[NRG];
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) x[rg] = 0.f;
#pragma unroll
    for (int s0 = 0; s0 < NBV; s0 += NBG) {
      v4i acc[NRG][NBG];
#pragma unroll
      for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
        for (int s = 0; s < NBG; ++s) acc[rg][s] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int vt = 0; vt < VT; ++vt) {
        if (vt * 64 < n) {
          v4i av[NRG];
#pragma unroll
          for (int rg = 0; rg < NRG; ++rg) {
            const uint4 q4 = *reinterpret_cast<const uint4 *>(sfrag + (rg * VT + vt) * 1024 + lane * 16);
            av[rg] = v4i{static_cast<int>(q4.x), static_cast<int>(q4.y), static_cast<int>(q4.z), static_cast<int>(q4.w)};
          }
          uint32_t pw[VW];
#pragma unroll
          for (int q = 0; q < VW; ++q)
            pw[q] = *reinterpret_cast<const uint32_t *>(wb + SH::OFF_V + ((2 * vt + (kg >> 1)) * VW + q) * 64 + 4 * col);
#pragma unroll
          for (int s = 0; s < NBG; ++s) {
            uint32_t w = 0u;
#pragma unroll
            for (int q = 0; q < VW; ++q)
              if ((Basis<VW>::M[s0 + s] >> q) & 1) w ^= pw[q];
            const v4i bv = expand_bits(w, mask);
#pragma unroll
            for (int rg = 0; rg < NRG; ++rg) acc[rg][s] = mfma_i8(av[rg], bv, acc[rg][s]);
          }
        }
      }
#pragma unroll
      for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
        for (int s = 0; s < NBG; ++s) x[rg] = fmaf(svb[s0 + s], combine_digits(acc[rg][s]), x[rg]);
    }
    const float inv = ldexpf(1.0f, -7 - ew);
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) {
      double swt = 0.0;
#pragma unroll
      for (int w = 0; w < NW; ++w) swt += spsw[w][4 * rg + kg];
      const float ssum = fmaf(2.0f, x[rg], -cvmax * static_cast<float>(swt)) * inv;
      accf[rg] = fmaf(accf[rg], alpha[rg], ssum);
    }

    // 4. refill this stage (this wave's region only; its reads are done)
    if (it + kStages < ns) {
      wait_lds();
      issue_split<D, KW, VW>(sa, sp + kStages * nb, buf, wave);
    }
  };

  for (int it = 0; it < ns;) {
    step(st0, it);
    if (++it >= ns) break;
    step(st1, it);
    if (++it >= ns) break;
    step(st2, it);
    ++it;
  }

  // partial of this block: {m, l, acc[D]} per head of the chunk
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg) {
    const float l = row_sum16(l_run[rg]);
    if (col == 0) spm[wave][4 * rg + kg] = l;
  }
  __syncthreads();
  float *part = p.partials + (bh * nb + bx) * G * (D + 2);
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg) {
    const int hl = 4 * rg + kg;
    if (hl < GE) part[(p.h0 + hl) * (D + 2) + 2 + 16 * wave + col] = accf[rg];
  }
  if (wave == 0 && col == 0) {
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) {
      const int hl = 4 * rg + kg;
      if (hl < GE) {
        float l = 0.f;
        for (int w = 0; w < NW; ++w) l += spm[w][hl];
        part[(p.h0 + hl) * (D + 2)] = m_run[rg];
        part[(p.h0 + hl) * (D + 2) + 1] = l;
      }
    }
  }
}

// Merge of the split partials of one (batch, kv-head) group and head chunk
// (8 heads): log-sum-exp weights over the blocks, division by the softmax
// sum, inverse rotation out = diag(s_v) H acc / sqrt(D), store. A kernel of
// its own: the partials are visible to it without any device-wide fence.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(DecodeParams p) {
  __shared__ float ob[8][D];
  __shared__ float se[8][kDecodeMaxBlocks];
  __shared__ float sL[8];
  const int G = p.group;
  const int n_q = p.n_kv * G;
  const int h0 = 8 * blockIdx.x;
  const int GE = min(8, G - h0);
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / p.n_kv;
  const int64_t kvh = bh % p.n_kv;
  const int nb = p.n_splits;
  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  const float *pbase = p.partials + bh * nb * G * (D + 2);
  const int64_t pstride = static_cast<int64_t>(G) * (D + 2);
  for (int hl = wave; hl < GE; hl += 4) {
    float M = -INFINITY;
    for (int j = lane; j < nb; j += kWave) M = fmaxf(M, pbase[j * pstride + (h0 + hl) * (D + 2)]);
    M = wave_max(M);
    float L = 0.f;
    for (int j = lane; j < nb; j += kWave) {
      const float m = pbase[j * pstride + (h0 + hl) * (D + 2)];
      const float e = (m == -INFINITY) ? 0.f : __expf(m - M);
      se[hl][j] = e;
      L = fmaf(pbase[j * pstride + (h0 + hl) * (D + 2) + 1], e, L);
    }
    L = wave_sum(L);
    if (lane == 0) sL[hl] = L;
  }
  __syncthreads();
  for (int e = tid; e < GE * D; e += 256) {
    const int hl = e / D, i = e % D;
    const float *src = pbase + (h0 + hl) * (D + 2) + 2 + i;
    float acc = 0.f;
    int j = 0;
    for (; j + 8 <= nb; j += 8) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = src[(j + k) * pstride];
#pragma unroll
      for (int k = 0; k < 8; ++k) acc = fmaf(v[k], se[hl][j + k], acc);
    }
    for (; j < nb; ++j) acc = fmaf(src[j * pstride], se[hl][j], acc);
    ob[hl][i] = (sL[hl] > 0.f) ? acc / sL[hl] : 0.f;
  }
  __syncthreads();
  for (int hs = 1; hs < D; hs <<= 1) {
    for (int e = tid; e < GE * D / 2; e += 256) {
      const int hl = e / (D / 2);
      const int r = e % (D / 2);
      const int j = (r / hs) * 2 * hs + (r % hs);
      const float x = ob[hl][j];
      const float y = ob[hl][j + hs];
      ob[hl][j] = x + y;
      ob[hl][j + hs] = x - y;
    }
    __syncthreads();
  }
  for (int e = tid; e < GE * D; e += 256) {
    const int hl = e / D, j = e % D;
    const float o = ob[hl][j] * p.vsigns[j] * (1.0f / sqrtf(static_cast<float>(D)));
    const int64_t row = b * n_q + kvh * G + h0 + hl;
    if (p.out_t == 0) static_cast<float *>(p.out)[row * D + j] = o;
    else static_cast<uint16_t *>(p.out)[row * D + j] = float_to_bf16_bits(o);
  }
}

template <int D, int KW, int VW>
static void launch_decode_kv(const DecodeParams &p, dim3 grid, hipStream_t st) {
  dim3 block(DecodeShape<D, KW, VW>::THREADS);
  if (p.group - p.h0 > 4) hipLaunchKernelGGL((decode_kernel<D, KW, VW, 2>), grid, block, 0, st, p);
  else hipLaunchKernelGGL((decode_kernel<D, KW, VW, 1>), grid, block, 0, st, p);
}

template <int D>
hipError_t launch_decode_d(const DecodeParams &p0, int kw, int vw, hipStream_t st) {
  if (p0.batch == 0 || p0.n_kv == 0) return hipSuccess;
  // n_splits here is the number of blocks per (batch, kv-head) group
  dim3 grid(static_cast<uint32_t>(p0.n_splits), static_cast<uint32_t>(p0.batch) * p0.n_kv);
  for (int hc = 0; hc < p0.n_hchunks; ++hc) {
    DecodeParams p = p0;
    p.h0 = 8 * hc;
#define TQ_DS_V(KK)                                          \
    switch (vw) {                                            \
      case 1: launch_decode_kv<D, KK, 1>(p, grid, st); break; \
      case 2: launch_decode_kv<D, KK, 2>(p, grid, st); break; \
      case 3: launch_decode_kv<D, KK, 3>(p, grid, st); break; \
      default: launch_decode_kv<D, KK, 4>(p, grid, st);      \
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
  }
  hipLaunchKernelGGL((merge_kernel<D>), dim3(static_cast<uint32_t>(p0.n_hchunks), grid.y), dim3(256), 0, st, p0);
  return hipGetLastError();
}

}  // namespace tq
