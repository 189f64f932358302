// Single-pass prefill attention over the coded cache: one block holds up to
// 64 (position, head) pairs of a KV head and reads each split of the context
// once for all of them (long prefills sit at the high end of the throughput
// range the pages measure: "TurboQuantとは？仕組み・実測精度・2026年7月時点の
// 実装状況", section 「精度劣化ゼロ」の出所と、マージ後に判明した実測値).
//
// Per split of kPrefillSplit tokens, staged in LDS by direct-to-LDS loads:
//  1. key logits: wave w holds the query operands of the row groups
//     [RGW w, RGW w + RGW) (4 pairs each; prepared by prep_kernel) and
//     contracts every key tile of the split with them on the matrix cores
//     (the int8 bit-plane formulation of the logit scan);
//  2. online softmax per pair (the wave owns its pairs), the weights
//     exp(logit - m) n_v scaled by 2^sc and split into fp16 hi + lo, written
//     in the A layout of v_mfma_f32_16x16x32_f16, with every pair's rescale
//     factor alpha;
//  3. values: wave w owns the coordinates [16 w, 16 w + 16) and decodes
//     them for every token of the split (index bits -> centroid from a
//     table, fp16 hi + lo), then weights x values on the matrix cores for
//     all 64 pairs (hi hi + hi lo + lo hi: fp32-grade products), folded
//     into acc = alpha acc + split sum.
// With 64 pairs the value contraction is cheaper as a real-valued product
// than as bit planes: the planes' cost grows with pairs x basis planes,
// the decoding here once per value. The block's partial {m, l, acc} goes
// to the workspace; merge_kernel combines the blocks of a group.
#pragma once

#include "tq_decode.inc.h"

namespace tq {

typedef _Float16 v8f16 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v4f mfma_f16_16x16x32(const v8f16 &a, const v8f16 &b, const v4f &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

union H8 {
  v8f16 h;
  uint4 q;
  uint32_t u[4];
};

constexpr int kPrefillPairs = kPrefillBlockPairs;   // pairs per block: 16 row groups of 4
constexpr int kPrefillSplit = kPrefillSplitTokens;  // tokens per split
constexpr int kPrefillStages = 2;

// Stage layout (16-byte units, in this order; chunks of 64 units are
// issued round-robin over the waves, each wave the same number of loads):
//   key records  KTL tiles x REC units (d = 128: plane-major within a tile,
//                as the scan kernels stage them; d = 64: a plain copy)
//   key scalars  S x KSB bytes
//   value words  [S / 32 blocks][VW planes][D coordinates] uint32
//   value norms  S x 2 bytes
template <int D, int KW, int VW>
struct PrefillShape {
  static constexpr int NW = D / 16;                 // waves: one per 16 value coordinates
  static constexpr int RGW = 16 / NW;               // key row groups per wave
  static constexpr int S = kPrefillSplit;
  static constexpr int KTL = S / 16;
  static constexpr int REC = key_planes(KW) * D / 8;
  static constexpr int KSB = key_scalar_bytes(KW);
  static constexpr int KU = KTL * REC;
  static constexpr int SU = S * KSB / 16;
  static constexpr int VU = (S / kValueBlock) * VW * D / 4;
  static constexpr int NU = S * 2 / 16;
  static constexpr int U = KU + SU + VU + NU;
  static constexpr int CHUNKS0 = (U + kWave - 1) / kWave;
  static constexpr int P = (CHUNKS0 + NW - 1) / NW;  // loads per wave per split
  static constexpr int CHUNKS = P * NW;
  static constexpr int STAGE = CHUNKS * 1024;
  static constexpr int OFF_KS = KU * 16;
  static constexpr int OFF_V = (KU + SU) * 16;
  static constexpr int OFF_VN = (KU + SU + VU) * 16;
  static constexpr int KS = S / 32;                  // 32-token K steps of the value product
  static constexpr int WBYTES = 4 * KS * 2 * 1024;   // weights: [row tile][K step][hi, lo][64 lanes][16 B]
};

// Issue this wave's share of split sp into a stage: chunk c (64 units) is
// issued by wave c % NW. Units past the cache capacity (or the padding past
// the stage's content) read the sequence's first bytes instead, so that
// every address stays inside the caller's arrays; those tokens lie past
// every context and get zero weight.
template <int D, int KW, int VW>
__device__ __forceinline__ void prefill_issue(const SeqArrays &sa, int sp, uint8_t *stage, int wave) {
  using PS = PrefillShape<D, KW, VW>;
  const int lane = lane_id();
  const int t_beg = sp * PS::S;
#pragma unroll
  for (int k = 0; k < PS::P; ++k) {
    const int c = wave + PS::NW * k;
    const int u = c * kWave + lane;
    const uint8_t *src = sa.kcodes;
    uint32_t off = 0;
    if (u < PS::KU) {
      const int tile = u / PS::REC, i = u % PS::REC;
      const int t = t_beg + 16 * tile;
      const uint32_t t0 = static_cast<uint32_t>(t < sa.cap ? t : 0);
      const uint32_t lo = (D == 128) ? (i % 16) * PS::REC + (i / 16) * 16 : i * 16;
      off = t0 * PS::REC + lo;
    } else if (u < PS::KU + PS::SU) {
      const int m = u - PS::KU;
      const int t = t_beg + m * (16 / PS::KSB);
      src = sa.kscal;
      off = static_cast<uint32_t>(t < sa.cap ? t : 0) * PS::KSB;
    } else if (u < PS::KU + PS::SU + PS::VU) {
      const int m = u - PS::KU - PS::SU;
      const int per_blk = VW * D / 4;                     // units per 32-token block
      int bg = t_beg / kValueBlock + m / per_blk;
      bg = bg < sa.nblk ? bg : 0;
      src = sa.vcodes;
      off = (static_cast<uint32_t>(bg) * per_blk + m % per_blk) * 16;
    } else if (u < PS::U) {
      const int m = u - PS::KU - PS::SU - PS::VU;
      const int t = t_beg + 8 * m;
      src = sa.vscal;
      off = static_cast<uint32_t>(t < sa.cap ? t : 0) * 2;
    }
    dma16_at(src + off, stage + c * 1024);
  }
}

// Entry b of the value-decoding table: bit j of byte b moved to bit
// 8 (j % 4) + 2 of word j / 4, so that OR-ing in plane q's entry shifted by q
// builds, in byte j % 4 of word j / 4, 4 x the index of token j.
__device__ __forceinline__ uint2 spread_entry(uint32_t b) {
  uint2 e = make_uint2(0u, 0u);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    e.x |= ((b >> j) & 1u) << (8 * j + 2);
    e.y |= ((b >> (j + 4)) & 1u) << (8 * j + 2);
  }
  return e;
}

template <int D, int KW, int VW>
__global__ __launch_bounds__(4 * D) void prefill_kernel(ScanParams p) {
  using PS = PrefillShape<D, KW, VW>;
  constexpr int NW = PS::NW, RGW = PS::RGW, S = PS::S, KTL = PS::KTL, KS = PS::KS;
  constexpr int NMF = key_frags(D, KW);
  constexpr int NST = kPrefillStages;
  constexpr int L = 1 << VW;
  constexpr float kCentScale = 256.f;                 // centroids x 2^8 in the fp16 operands
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NST * PS::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t wts[PS::WBYTES];
  __shared__ uint32_t ctab[L];                        // centroid x 2^8 as fp16 hi | lo << 16
  __shared__ uint2 spread[256];
  __shared__ float salpha[kPrefillPairs];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = lane_id();
  const int kg = lane / 16, col = lane % 16;
  const int G = p.group;                               // pairs of the group (chunk x qgroup)
  const int z0 = kPrefillPairs * static_cast<int>(blockIdx.z);
  const int PE = min(kPrefillPairs, G - z0);           // live pairs of this block
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / p.n_kv;
  const int nb = static_cast<int>(gridDim.x), bx = static_cast<int>(blockIdx.x);
  const int pos0 = p.pos0[b];
  // context of the block: through the last live pair's position
  int64_t ctx64 = static_cast<int64_t>(pos0) + (z0 + PE - 1) / p.qgroup + 1;
  ctx64 = ctx64 < 0 ? 0 : (ctx64 > p.max_ctx ? p.max_ctx : ctx64);
  const int ctx = static_cast<int>(ctx64);
  const int n_splits = (ctx + S - 1) / S;
  const int ns = (n_splits > bx) ? (n_splits - bx + nb - 1) / nb : 0;

  if (tid < L) {
    const float c = p.vcent[tid] * kCentScale;
    uint32_t hi, lo;
    split_pair(c, 0.f, hi, lo);
    ctab[tid] = (hi & 0xffffu) | (lo << 16);
  }
  if (tid < 256) spread[tid] = spread_entry(static_cast<uint32_t>(tid));

  SeqArrays sa;
  sa.cap = static_cast<int32_t>(p.cap);
  sa.nblk = static_cast<int32_t>(p.cap / kValueBlock);
  sa.kcodes = p.kcodes + bh * p.cap * PS::REC;
  sa.kscal = reinterpret_cast<const uint8_t *>(p.kscalars) + bh * p.cap * PS::KSB;
  sa.vcodes = reinterpret_cast<const uint8_t *>(p.vcodes + bh * sa.nblk * VW * D);
  sa.vscal = reinterpret_cast<const uint8_t *>(p.vscalars) + bh * p.cap * 2;

  // the wave's query operands (row groups g = RGW wave + r of the block)
  // and head constants, from the prepared records (8 pairs per record)
  v4i a[RGW][NMF];
  float4 fh[RGW];
  int lim[RGW];
  const int64_t pstride = prepared_stride(D, key_lm(KW));
#pragma unroll
  for (int r = 0; r < RGW; ++r) {
    const int g = RGW * wave + r;
    const int pr = z0 + 4 * g;                        // first pair of the row group
    const int pair = pr + kg;                         // this lane's pair in the logit layout
    int64_t l = static_cast<int64_t>(pos0) + pair / p.qgroup + 1;
    l = l > ctx64 ? ctx64 : l;
    lim[r] = (4 * g + kg < PE && l > 0) ? static_cast<int>(l) : 0;
    if (4 * g < PE) {
      const uint8_t *rec = p.prepared + (bh * p.n_hchunks + pr / 8) * pstride;
      const int rgi = (pr / 4) % 2;
#pragma unroll
      for (int mf = 0; mf < NMF; ++mf) {
        const uint4 v = *reinterpret_cast<const uint4 *>(rec + ((rgi * NMF + mf) * kWave + lane) * 16);
        a[r][mf] = v4i{static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z), static_cast<int>(v.w)};
      }
      fh[r] = *reinterpret_cast<const float4 *>(rec + pstride - 128 + 16 * (4 * rgi + kg));
    } else {
#pragma unroll
      for (int mf = 0; mf < NMF; ++mf) a[r][mf] = v4i{0, 0, 0, 0};
      fh[r] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  for (int k = 0; k < min(ns, NST); ++k) prefill_issue<D, KW, VW>(sa, bx + k * nb, ring + k * PS::STAGE, wave);

  uint32_t mask[4];
  lane_masks(mask);
  const float kappa = key_qjl(KW) ? kSqrtHalfPi / static_cast<float>(D) : 0.f;
  // logits and the running maxima in log2 units (exp2 in the softmax); the
  // partial's m goes out in natural-log units
  const float sl = p.sm_scale * 1.4426950408889634f;
  float m_run[RGW], l_run[RGW];
#pragma unroll
  for (int r = 0; r < RGW; ++r) { m_run[r] = -INFINITY; l_run[r] = 0.f; }
  v4f acc[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) acc[rt] = v4f{0.f, 0.f, 0.f, 0.f};
  const int coord = 16 * wave + col;                  // value coordinate of this lane (value phase)

  int issued = min(ns, NST);
  for (int it = 0; it < ns; ++it) {
    const int sp = bx + it * nb;
    uint8_t *buf = ring + (it % NST) * PS::STAGE;
    wait_splits<PS::P>(max(0, issued - it - 1));
    __syncthreads();                                  // the stage, and every wave done with split it - 1
    if (it >= 1 && it - 1 + NST < ns) {
      prefill_issue<D, KW, VW>(sa, bx + (it - 1 + NST) * nb, ring + ((it - 1) % NST) * PS::STAGE, wave);
      ++issued;
    }
    const int t0 = sp * S;

    // 1. logits of the wave's pairs for every key tile of the split,
    //    software-pipelined: tile u + 1's products are issued before tile u's
    //    epilogue, so that the epilogue's VALU work runs beside them
    float lg[KTL][RGW];
    float mx[RGW];
#pragma unroll
    for (int r = 0; r < RGW; ++r) mx[r] = -INFINITY;
    auto tile_products = [&](int u, v4i (&clm)[RGW], v4i (&cqj)[RGW], uint32_t &sc) {
      const uint8_t *kb = buf + u * PS::REC * 16;
      KeyTile<D, KW> kt;
#pragma unroll
      for (int q = 0; q < key_planes(KW); ++q) {
        if constexpr (D == 128) {
          const uint2 v = *reinterpret_cast<const uint2 *>(kb + (16 * q + col) * 16 + 8 * (kg >> 1));
          kt.w[q][0] = v.x;
          kt.w[q][D == 128 ? 1 : 0] = v.y;
        } else {
          kt.w[q][0] = *reinterpret_cast<const uint32_t *>(kb + col * PS::REC + q * 8 + 4 * (kg >> 1));
        }
      }
      const int tok = 16 * u + col;
      if constexpr (key_qjl(KW)) kt.sc = *reinterpret_cast<const uint32_t *>(buf + PS::OFF_KS + 4 * tok);
      else kt.sc = *reinterpret_cast<const uint16_t *>(buf + PS::OFF_KS + 2 * tok);
      key_tile_mfma<D, KW, RGW>(kt, a, mask, RGW, clm, cqj);
      sc = kt.sc;
    };
    v4i clm[2][RGW], cqj[2][RGW];
    uint32_t ksc[2];
    tile_products(0, clm[0], cqj[0], ksc[0]);
#pragma unroll
    for (int u = 0; u < KTL; ++u) {
      const int cur = u & 1;
      if (u + 1 < KTL) tile_products(u + 1, clm[cur ^ 1], cqj[cur ^ 1], ksc[cur ^ 1]);
      const int tok = 16 * u + col;
      const float kn = f16_bits_to_float(static_cast<uint16_t>(ksc[cur] & 0xffffu));
      const float kgm = f16_bits_to_float(static_cast<uint16_t>(ksc[cur] >> 16));
#pragma unroll
      for (int r = 0; r < RGW; ++r) {
        const float l = tile_logit<key_qjl(KW)>(clm[cur][r], cqj[cur][r], fh[r], kn, kgm, kappa) * sl;
        lg[u][r] = (t0 + tok < lim[r]) ? l : -INFINITY;
        asm volatile("" : "+v"(lg[u][r]));       // formed here, not at its later uses
        mx[r] = fmaxf(mx[r], lg[u][r]);
      }
      // at most two tiles' operands and accumulators live at a time
      __builtin_amdgcn_sched_barrier(0);
    }

    // 2. softmax statistics of the wave's pairs; weights into the A layout
    float nvm = 0.f;
    for (int t = lane; t < S; t += kWave) {
      const float nv = f16_bits_to_float(*reinterpret_cast<const uint16_t *>(buf + PS::OFF_VN + 2 * t));
      if (t0 + t < ctx) nvm = fmaxf(nvm, nv);
    }
    nvm = wave_max(nvm);
    int ex = 0;
    (void)frexpf(nvm, &ex);
    const int sc = (nvm > 0.f) ? 14 - ex : 0;         // weights below 2^14
    const float up = ldexpf(1.0f, sc);
    float nvu[KTL];                                    // value norm x 2^sc of token 16 u + col
#pragma unroll
    for (int u = 0; u < KTL; ++u) {
      const int tok = 16 * u + col;
      const float nv = f16_bits_to_float(*reinterpret_cast<const uint16_t *>(buf + PS::OFF_VN + 2 * tok));
      nvu[u] = (t0 + tok < ctx) ? nv * up : 0.f;       // (slots past the context are not read as data)
    }
#pragma unroll
    for (int r = 0; r < RGW; ++r) {
      const float ms = row_max16(mx[r]);
      const float mn = fmaxf(m_run[r], ms);
      const float alpha = (m_run[r] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run[r] - mn);
      m_run[r] = mn;
      l_run[r] *= alpha;
      const int pl = 4 * (RGW * wave + r) + kg;      // pair within the block
      if (col == 0) salpha[pl] = alpha;
      const float msub = (mn == -INFINITY) ? 0.f : mn;
      const int rt = pl / 16, r16 = pl % 16;
      const bool odd = col & 1;
#pragma unroll
      for (int u = 0; u < KTL; ++u) {
        const int tok = 16 * u + col;
        const float e = __builtin_amdgcn_exp2f(lg[u][r] - msub);   // 0 for masked tokens (-inf)
        l_run[r] += e;
        const float wv = e * nvu[u];
        // tokens 2 m, 2 m + 1 (lanes col, col ^ 1) share a dword of the A
        // layout: both lanes split the pair into fp16 hi + lo, the even lane
        // stores the hi halves, the odd lane the lo halves
        const float w_even = dpp_f<0xA0>(wv);           // quad_perm [0, 0, 2, 2]
        const float w_odd = dpp_f<0xF5>(wv);            // quad_perm [1, 1, 3, 3]
        uint32_t hi, lo;
        split_pair(w_even, w_odd, hi, lo);
        const uint32_t word = odd ? lo : hi;
        const int ks = tok / 32, kq = (tok % 32) / 8, j = tok % 8;
        uint8_t *dst = wts + ((rt * KS + ks) * 2 + (odd ? 1 : 0)) * 1024 + ((kq * 16 + r16) * 16 + 2 * (j & ~1));
        *reinterpret_cast<uint32_t *>(dst) = word;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();                                  // weights and alphas

    // 3. values: this wave's coordinates for every token of the split. Per
    //    K step of 32 tokens: B = the decoded centroids of the lane's
    //    coordinate for tokens 32 ks + 8 kg + j (j < 8), A = the weights of
    //    the 4 row tiles. The next step's B is decoded after this step's
    //    products are issued.
    auto decode_b = [&](int ks, H8 &bh, H8 &bl) {
      // 4 x the tokens' indices as the bytes of two words, then the
      // centroid hi / lo parts from the table
      uint32_t ix[2] = {0u, 0u};
#pragma unroll
      for (int q = 0; q < VW; ++q) {
        const uint32_t w = *reinterpret_cast<const uint32_t *>(buf + PS::OFF_V + ((ks * VW + q) * D + coord) * 4);
        const uint2 e = spread[(w >> (8 * kg)) & 0xffu];
        ix[0] |= e.x << q;
        ix[1] |= e.y << q;
      }
      const uint8_t *ct = reinterpret_cast<const uint8_t *>(ctab);
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const uint32_t e0 = *reinterpret_cast<const uint32_t *>(ct + ((ix[j / 4] >> (8 * (j % 4))) & 0xffu));
        const uint32_t e1 = *reinterpret_cast<const uint32_t *>(ct + ((ix[j / 4] >> (8 * (j % 4) + 8)) & 0xffu));
        bh.u[j / 2] = __builtin_amdgcn_perm(e1, e0, 0x05040100u);   // hi halves of e0, e1
        bl.u[j / 2] = __builtin_amdgcn_perm(e1, e0, 0x07060302u);   // lo halves
      }
    };
    v4f cs[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) cs[rt] = v4f{0.f, 0.f, 0.f, 0.f};
    H8 bh[2], bl[2];
    decode_b(0, bh[0], bl[0]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cur = ks & 1;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        H8 ah[1], al[1];
        const uint8_t *src = wts + ((rt * KS + ks) * 2) * 1024 + lane * 16;
        ah[0].q = *reinterpret_cast<const uint4 *>(src);
        al[0].q = *reinterpret_cast<const uint4 *>(src + 1024);
        cs[rt] = mfma_f16_16x16x32(ah[0].h, bh[cur].h, cs[rt]);
        cs[rt] = mfma_f16_16x16x32(ah[0].h, bl[cur].h, cs[rt]);
        cs[rt] = mfma_f16_16x16x32(al[0].h, bh[cur].h, cs[rt]);
      }
      if (ks + 1 < KS) decode_b(ks + 1, bh[cur ^ 1], bl[cur ^ 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    const float down = ldexpf(1.0f, -sc) * (1.0f / kCentScale);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[rt][i] = fmaf(acc[rt][i], salpha[16 * rt + 4 * kg + i], cs[rt][i] * down);
  }

  // the block's partial {m, l, acc} per live pair
  float *part = p.partials + (bh * nb + bx) * static_cast<int64_t>(G) * (D + 2);
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pl = 16 * rt + 4 * kg + i;
      if (pl < PE) part[(z0 + pl) * (D + 2) + 2 + coord] = acc[rt][i];
    }
#pragma unroll
  for (int r = 0; r < RGW; ++r) {
    const float l = row_sum16(l_run[r]);
    const int pl = 4 * (RGW * wave + r) + kg;
    if (col == 0 && pl < PE) {
      part[(z0 + pl) * (D + 2)] = m_run[r] * 0.6931471805599453f;
      part[(z0 + pl) * (D + 2) + 1] = l;
    }
  }
}

template <int D, int KW>
static void launch_prefill_v(const ScanParams &p, int vw, dim3 grid, hipStream_t st) {
  const dim3 block(4 * D);
  switch (vw) {
    case 1: hipLaunchKernelGGL((prefill_kernel<D, KW, 1>), grid, block, 0, st, p); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<D, KW, 2>), grid, block, 0, st, p); break;
    case 3: hipLaunchKernelGGL((prefill_kernel<D, KW, 3>), grid, block, 0, st, p); break;
    default: hipLaunchKernelGGL((prefill_kernel<D, KW, 4>), grid, block, 0, st, p);
  }
}

// The single-pass prefill: the query preparation of every 8 pairs into
// p.prepared_w (== p.prepared), the scan (grid: p.nb blocks per group,
// groups, chunks of 64 pairs), then the merge of the blocks' partials.
template <int D>
hipError_t launch_prefill_d(const ScanParams &p, int kw, int vw, hipStream_t st) {
  if (p.batch == 0 || p.n_kv == 0) return hipSuccess;
  hipError_t e = launch_prepare_d<D>(p, kw, st);
  if (e != hipSuccess) return e;
  const uint32_t groups = static_cast<uint32_t>(p.batch) * p.n_kv;
  const dim3 grid(static_cast<uint32_t>(p.nb), groups,
                  static_cast<uint32_t>((p.group + kPrefillPairs - 1) / kPrefillPairs));
  switch (kw) {
    case 1: launch_prefill_v<D, 1>(p, vw, grid, st); break;
    case 2: launch_prefill_v<D, 2>(p, vw, grid, st); break;
    case 3: launch_prefill_v<D, 3>(p, vw, grid, st); break;
    case 4: launch_prefill_v<D, 4>(p, vw, grid, st); break;
    case kKeyMse + 1: launch_prefill_v<D, kKeyMse + 1>(p, vw, grid, st); break;
    case kKeyMse + 2: launch_prefill_v<D, kKeyMse + 2>(p, vw, grid, st); break;
    case kKeyMse + 3: launch_prefill_v<D, kKeyMse + 3>(p, vw, grid, st); break;
    default: launch_prefill_v<D, kKeyMse + 4>(p, vw, grid, st);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((merge_kernel<D>), dim3(static_cast<uint32_t>(p.n_hchunks), groups), dim3(kMergeThreads), 0,
                     st, p);
  return hipGetLastError();
}

}  // namespace tq
