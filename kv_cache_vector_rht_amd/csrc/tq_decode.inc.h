// Logit scan over packed keys and split-context fused decode attention over
// packed keys and values, on the matrix cores, with the query preparation
// done by each block in its prologue.
//
// Estimator (pages: "TurboQuantとは？仕組み・実測精度・2026年7月時点の実装状況",
// 第2段: the QJL residual bit makes the inner-product estimate unbiased; its
// まとめ names the attention-logit computation as the accelerated operation):
//   logit(q, k) = n ( sum_i q'_i c[idx_i]
//                     + sqrt(pi/2)/D * gamma * sum_j p_j (2 sigma_j - 1) ),
// q' = R q, p = S q'. Both sums are bit-plane contractions (tq_mfma.h); the
// query side of a (batch, kv-head) group is prepared by every block that
// scans its keys, and every key record is read once for all heads of a
// chunk of up to 8 heads.
#pragma once

#include "tq_device.h"
#include "tq_kernels.h"
#include "tq_mfma.h"
#include "tq_qjl.h"

namespace tq {

constexpr float kSqrtHalfPi = 1.2533141373155002f;   // sqrt(pi / 2)

// ------------------------------------------------------------ key tiles

// MFMA operand fragments of the query side per row group: one per key basis
// plane (and the sign plane of full records) and 64-coordinate chunk.
__host__ __device__ constexpr int key_frags(int d, int kw) {
  return (basis_size(key_lm(kw)) + (key_qjl(kw) ? 1 : 0)) * (d / 64);
}

// One 16-key tile of a wave: lane (kg = l/16, n = l%16) holds the plane words
// of key n that its K slots need, and the key's raw fp16 scalars (norm in the
// low half, residual norm in the high half; MSE-only records: the norm alone).
template <int D, int KW>
struct KeyTile {
  static constexpr int NH = D / 64;
  uint32_t w[key_planes(KW)][NH];
  uint32_t sc;
  __device__ __forceinline__ float norm() const { return f16_bits_to_float(static_cast<uint16_t>(sc & 0xffffu)); }
  __device__ __forceinline__ float gamma() const { return f16_bits_to_float(static_cast<uint16_t>(sc >> 16)); }
};

// Accumulate the key planes and (full records) the sign plane of one tile for
// NRG row groups.
template <int D, int KW, int NRG>
__device__ __forceinline__ void key_tile_mfma(const KeyTile<D, KW> &kt, const v4i (&a)[NRG][key_frags(D, KW)],
                                              const uint32_t (&mask)[4], int nrg, v4i (&clm)[NRG], v4i (&cqj)[NRG]) {
  constexpr int KL = key_lm(KW);
  constexpr int NB = Basis<KL>::N;
  constexpr int NH = D / 64;
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg) { clm[rg] = v4i{0, 0, 0, 0}; cqj[rg] = v4i{0, 0, 0, 0}; }
#pragma unroll
  for (int s = 0; s < NB; ++s) {
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      uint32_t w = 0u;
#pragma unroll
      for (int q = 0; q < KL; ++q)
        if ((Basis<KL>::M[s] >> q) & 1) w ^= kt.w[q][hf];
      const v4i bv = expand_bits(w, mask);
#pragma unroll
      for (int rg = 0; rg < NRG; ++rg)
        if (rg < nrg) clm[rg] = mfma_i8(a[rg][s * NH + hf], bv, clm[rg]);
    }
  }
  if constexpr (key_qjl(KW)) {
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      const v4i bv = expand_bits(kt.w[KL][hf], mask);
#pragma unroll
      for (int rg = 0; rg < NRG; ++rg)
        if (rg < nrg) cqj[rg] = mfma_i8(a[rg][NB * NH + hf], bv, cqj[rg]);
    }
  }
}

// fl = {inv_lm, cst_lm, inv_qj, cst_qj} of the lane's head. QJ: the full
// estimator; else its first term alone (MSE-only records).
template <bool QJ>
__device__ __forceinline__ float tile_logit(const v4i &clm, const v4i &cqj, const float4 &fl, float n, float g,
                                            float kappa) {
  const float lm = fmaf(combine_digits(clm), fl.x, -fl.y);
  if constexpr (!QJ) return n * lm;
  const float qj = fmaf(combine_digits(cqj), fl.z, -fl.w);
  return n * fmaf(kappa * g, qj, lm);
}

__device__ __forceinline__ void lane_masks(uint32_t (&mask)[4]) {
  const int kk = 4 * ((lane_id() / 16) & 1);
#pragma unroll
  for (int r = 0; r < 4; ++r) mask[r] = 0x01010101u << (kk + r);
}

// ------------------------------------------------------------------ staging

// Every scan block walks splits of one (batch, kv-head) sequence through a
// ring of LDS stage buffers; while it computes on one split, the loads of the
// next ones are in flight. The logit scan takes 256-token splits; decode
// attention 512-token splits in two stages where they fit in LDS (fewer
// barriers and per-split steps per token), else 256 tokens in kStages.
constexpr int kStages = 3;

// Block layout: NW waves (D/16 for decode; the logit scan may take more).
// Wave w owns the 16-key tiles w, w + NW, ... of
// every split and (decode) the value coordinates [16 w, 16 w + 16). Its
// share of a split is staged in a region of LDS that only it reads, so no
// barrier guards the staging:
//   [0, OFF_S)         key tiles, 16 x REC bytes each; for d = 128 plane-major
//                      (the 16 keys' words of plane 0, then of plane 1, ...),
//                      for fp8 keys chunk-major (16-byte chunk q of key i at
//                      16-byte unit 16 q + i)
//   [OFF_S, OFF_V)     the tiles' key scalars (64 B per tile, 32 B for
//                      MSE-only records, none for fp8 keys), then (decode)
//                      their value norms (32 B per tile)
//   [OFF_V, ...)       (decode) value words: [32-token block][plane][16 coords]
template <int D, int KW, int VW, bool LOGITS, int SPLIT, int NWAVE = D / 16>
struct ScanShape {
  static constexpr bool K8 = KW == kKeyFp8;          // fp8 key records
  static constexpr int S = SPLIT;
  static constexpr int NW = NWAVE;
  static constexpr int THREADS = NW * kWave;
  static constexpr int KT = S / 16 / NW;             // key tiles per wave
  static constexpr int VT = S / 64;                  // 64-token value tiles
  static constexpr int REC = K8 ? D : key_planes(KW) * D / 8;   // record bytes = 16-byte units per key tile
  static constexpr int KI = (REC + 63) / 64;         // loads per key tile
  static constexpr int KSU = K8 ? 0 : key_scalar_bytes(KW);   // key scalar units per tile (16 keys' scalars)
  static constexpr int SU = (KSU + (LOGITS ? 0 : 2)) * KT;   // scalar units
  static constexpr int VU = LOGITS ? 0 : (S / 32) * VW * 4;   // value units
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
// 4 bytes per lane from this lane's address into LDS at lds + 4 * lane.
__device__ __forceinline__ void dma4_at(const void *src, uint8_t *lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "{m0}"(lds_m0(lds)) : "memory");
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

// Issue this wave's share of split sp into its region of a stage buffer.
// Every wave issues exactly P loads. Tiles past the cache capacity load the
// sequence's first tile instead (their keys are past the context and are
// never used), so every address stays inside the caller's arrays.
template <int D, int KW, int VW, bool LOGITS, int SPLIT, int NWAVE = D / 16>
__device__ __forceinline__ void issue_split(const SeqArrays &sa, int sp, uint8_t *stage, int wave) {
  using SH = ScanShape<D, KW, VW, LOGITS, SPLIT, NWAVE>;
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
        // d = 128 and fp8 keys: LDS unit 16 q + i <- 16-byte unit q (a plane,
        // or 16 fp8 coordinates) of key i; d = 64: a plain copy
        const uint32_t lo = (D == 128 || SH::K8) ? (unit % 16) * REC + (unit / 16) * 16 : unit * 16;
        dma16(sa.kcodes, tile0[u] * REC + lo, wb + u * REC * 16 + ki * 1024);
      }
    }
  }
  if (lane < SH::SU) {
    // lanes [0, KSU KT): unit m of the key scalars of tile lane / KSU (KSU
    // units of 16 bytes per tile: 16 / KSU keys each; none for fp8 keys);
    // then value norms
    constexpr int KSD = SH::KSU > 0 ? SH::KSU : 1;
    const bool key = lane < SH::KSU * SH::KT;
    const int u = key ? lane / KSD : (lane - SH::KSU * SH::KT) / 2;
    const int m = key ? lane % KSD : (lane - SH::KSU * SH::KT) % 2;
    uint32_t t0 = 0;
#pragma unroll
    for (int v = 0; v < SH::KT; ++v) t0 = (u == v) ? tile0[v] : t0;
    dma16_at(key ? sa.kscal + (t0 + (16 / KSD) * m) * KSD : sa.vscal + (t0 + 8 * m) * 2, wb + SH::OFF_S);
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

// ------------------------------------------------------------------ query prep

// Walsh-Hadamard butterflies over the 64 lanes of a wave, lane bit b being
// index bit b: stage b pairs lane l with l ^ 2^b, the lower lane keeping the
// sum and the upper one the difference (lower - upper). The exchanges stay
// in the vector ALU: quad permutes (bits 0, 1), row rotates (bits 2, 3:
// rotating a 16-lane row right by n hands lane l the value of lane l - n),
// lane-row and half-wave swaps (bits 4, 5).
__device__ __forceinline__ float wave_fwht(float x, int lane) {
  auto bfly = [lane](float own, float other, int bit) { return ((lane >> bit) & 1) ? other - own : own + other; };
  x = bfly(x, dpp_f<0xB1>(x), 0);
  x = bfly(x, dpp_f<0x4E>(x), 1);
  {
    // both rotations by every lane before the select: a lane-exchange in a
    // divergent branch would read lanes that are switched off
    const float from_below = dpp_f<0x124>(x), from_above = dpp_f<0x12C>(x);
    x = bfly(x, (lane & 4) ? from_below : from_above, 2);
  }
  x = bfly(x, dpp_f<0x128>(x), 3);
  {
    // a lane-row swap of x with itself leaves the even row's copy in the
    // first register and the odd row's in the second
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = fmaf((lane & 16) ? -1.f : 1.f, __uint_as_float(r[1]), __uint_as_float(r[0]));
  }
  {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    x = fmaf((lane & 32) ? -1.f : 1.f, __uint_as_float(r[1]), __uint_as_float(r[0]));
  }
  return x;
}

// Scratch of the in-block query preparation (byte offsets):
//   SQ, SP  q' and p, [8][D] float
//   SQH,SQL q' of each head scaled by a power of two (its max |q'| below
//           2^14) and split into fp16 hi + lo, [8][D] halves each: the B
//           operands of the sketch product
//   SST     per head: max |q'| and sum q' [8][4]; SCON per-head constants [8][4]
//   SB      key basis coefficients [8]
//   SPS     per 32-row tile of S and head: max |p| and sum p over the tile
//   CENT    the centroids [2^w] float, staged by a direct-to-LDS load
//   FRAG    the operand bytes in the MFMA A layout, [NRG][NMF][64 lanes][16]
// Prepared-query records (tq_prepare_queries) hold the operand fragments
// [NRG][NMF][64 lanes][16 bytes] (REC_FRAG bytes), then the 8 heads'
// constants (128 bytes); a scan block copies one to the start of its
// scratch.
template <int D, int KW, int NRG>
struct PrepShape {
  static constexpr int NB = Basis<key_lm(KW)>::N;
  static constexpr int NMF = key_frags(D, KW);
  static constexpr int SQ = 0;
  static constexpr int SP = SQ + 8 * D * 4;
  static constexpr int SQH = SP + 8 * D * 4;
  static constexpr int SQL = SQH + 8 * D * 2;
  static constexpr int SST = SQL + 8 * D * 2;
  static constexpr int SCON = SST + 8 * 4 * 4;
  static constexpr int SB = SCON + 8 * 4 * 4;
  static constexpr int SPS = SB + 64;                 // per row tile and head: max |p|, sum p
  static constexpr int CENT = SPS + (D / 32) * 8 * 2 * 4;
  static constexpr int FRAG = (CENT + 64 + 1023) / 1024 * 1024;
  static constexpr int REC_FRAG = NRG * NMF * 1024;
  static constexpr int BYTES = FRAG + REC_FRAG;
  static_assert(REC_FRAG + 128 <= BYTES, "a prepared record fits in the scratch");
};

// Inputs of the query preparation, loaded straight into the registers of the
// waves that use them: the query rows of the heads a wave rotates (head
// wave + NW k, lane l holding elements E l .. E l + E - 1, E = D / 64) with
// their signs, and for the waves of the sketch product their 32-row tile of
// the sketch as MFMA A operands, 16 bytes per K step.
template <int D, int NW>
struct PrepIn {
  static constexpr int E = D / kWave;
  static constexpr int HPW = (8 + NW - 1) / NW;        // heads per wave (at most 8 heads)
  float q[HPW][E];
  float s[E];
  uint4 sk[D / 16];
};

// Tokens per decode split: 512 (two stages) if those stages, the query
// preparation's scratch and the weight operands fit in LDS, else 256.
template <int D, int KW, int VW, int NRG>
constexpr int attend_split() {
  using S5 = ScanShape<D, KW, VW, false, 512>;
  using PS = PrepShape<D, KW == kKeyFp8 ? 1 : KW, NRG>;
  constexpr int PSB = KW == kKeyFp8 ? 4096 : PS::BYTES;
  constexpr int ring = S5::STAGE_BYTES + (S5::STAGE_BYTES > PSB ? S5::STAGE_BYTES : PSB);
  return ring + NRG * (512 / 64) * 1024 <= 160 * 1024 - 4096 ? 512 : 256;
}

// A block's place in a group: its block index bx in [0, nb) and its chunk
// of 8 heads. The chunks are the launch grid's z dimension, or (p.zin > 0,
// nb a multiple of 8) interleaved into x: x = 8 (zin u + c) + r stands for
// block 8 u + r of chunk c. Consecutive block ids go to the XCDs in turn,
// so the zin blocks that scan the same splits for different chunks then
// start together on the same XCD and its L2 serves their repeated reads.
__device__ __forceinline__ int head_chunk0(const ScanParams &p) {
  return 8 * (p.zin ? static_cast<int>((blockIdx.x >> 3) % static_cast<uint32_t>(p.zin)) : static_cast<int>(blockIdx.z));
}
__device__ __forceinline__ int scan_block_index(const ScanParams &p) {
  return p.zin ? static_cast<int>((blockIdx.x & 7u) + 8u * (blockIdx.x / (8u * static_cast<uint32_t>(p.zin))))
               : static_cast<int>(blockIdx.x);
}
__device__ __forceinline__ int scan_blocks(const ScanParams &p) {
  return p.zin ? static_cast<int>(gridDim.x / static_cast<uint32_t>(p.zin)) : static_cast<int>(gridDim.x);
}

// Row of q holding head v of the group of (b, kv-head kvh).
__device__ __forceinline__ int64_t query_row(const ScanParams &p, int64_t b, int64_t kvh, int v) {
  const int gq = p.qgroup;
  return (b * p.chunk + v / gq) * (static_cast<int64_t>(p.n_kv) * gq) + kvh * gq + v % gq;
}

// Load the preparation's inputs (a block of NW waves): the query rows and
// signs into the registers of the waves that rotate them, the sketch tiles
// into those of the waves of the sketch product (ordinary loads: these waves
// issue no direct-to-LDS load before they have consumed them), and the
// centroids into the scratch by one direct-to-LDS load of the last wave.
template <int D, int KW, int NRG, int NW = D / 16>
__device__ __forceinline__ void issue_prep(const ScanParams &p, int64_t bh, int GE, uint8_t *scratch, int wave,
                                           PrepIn<D, NW> &in) {
  using PS = PrepShape<D, KW, NRG>;
  using PI = PrepIn<D, NW>;
  constexpr int E = PI::E;
  const int lane = lane_id();
  if (wave < GE) {
#pragma unroll
    for (int e = 0; e < E; ++e) in.s[e] = p.ksigns[E * lane + e];
#pragma unroll
    for (int k = 0; k < PI::HPW; ++k) {
      const int h = wave + NW * k;
      if (h < GE) {
        const int64_t row = query_row(p, bh / p.n_kv, bh % p.n_kv, head_chunk0(p) + h);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int64_t i = row * D + E * lane + e;
          in.q[k][e] = (p.xt == 0) ? static_cast<const float *>(p.q)[i]
                       : (p.xt == 1) ? bf16_bits_to_float(static_cast<const uint16_t *>(p.q)[i])
                                     : f16_bits_to_float(static_cast<const uint16_t *>(p.q)[i]);
        }
      }
    }
  }
  if (key_qjl(KW) && wave < D / 32) {
    const int r = 32 * wave + lane % 32, half = lane / 32;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      in.sk[ks] = *reinterpret_cast<const uint4 *>(p.sketch + static_cast<int64_t>(r) * D + 16 * ks + 8 * half);
  }
  if (wave == NW - 1 && lane < (1 << key_lm(KW))) dma4_at(p.kcent + lane, scratch + PS::CENT);
}

// Query preparation of the heads [h0, h0 + GE) (GE <= 4 NRG) of group bh by
// one block of NW waves, from the staged inputs: q' = R q, p = S q', the
// digit operands of the key planes (2 beta_s q') and of the sign plane
// (2 p), one fixed-point exponent per head for each, and the per-head
// constants {2^-(7+e_lm), c[L-1] sum q', 2^-(7+e_qj), sum p}. (MSE-only
// key records: no p, no sign-plane operand, the last two constants 0.) Every wave
// ends holding all operand fragments of the chunk in a[][] and its heads'
// constants in fh[] (rows of absent heads zero).
// Phases, each closed by a block barrier: (1) one wave per head rotates it
// (q' = H diag(s) q / sqrt(D) in registers) and writes q', its statistics
// and its scaled fp16 hi + lo split; (2) the waves of the sketch's 32-row
// tiles form p = S q' on the matrix cores; (3) every thread writes the
// digits of one (head, coordinate) for every operand, straight into the
// fragment layout; (4) every wave loads the fragments. late_loads(): the
// waves of phase 2 call it right after their products, the other waves at
// the start of phase 2 (the caller issues there the first key loads of the
// waves that had preparation work to do first).
template <int D, int KW, int NRG, int NW = D / 16, class LateLoads>
__device__ __forceinline__ void group_prep(const ScanParams &p, int GE, uint8_t *scratch, const PrepIn<D, NW> &in,
                                           LateLoads late_loads, v4i (&a)[NRG][PrepShape<D, KW, NRG>::NMF],
                                           float4 (&fh)[NRG]) {
  using PS = PrepShape<D, KW, NRG>;
  constexpr bool QJ = key_qjl(KW);
  constexpr int KL = key_lm(KW);
  constexpr int NB = PS::NB, NMF = PS::NMF, NH = D / 64, NK = NB + (QJ ? 1 : 0);
  constexpr int E = D / kWave;
  constexpr int L = 1 << KL;
  float *sq = reinterpret_cast<float *>(scratch + PS::SQ);      // [8][D]
  float *sp = reinterpret_cast<float *>(scratch + PS::SP);      // [8][D]
  uint16_t *sqh = reinterpret_cast<uint16_t *>(scratch + PS::SQH);   // [8][D]
  uint16_t *sql = reinterpret_cast<uint16_t *>(scratch + PS::SQL);   // [8][D]
  float *sst = reinterpret_cast<float *>(scratch + PS::SST);    // [8][4]
  float *scon = reinterpret_cast<float *>(scratch + PS::SCON);  // [8][4]
  float *sb = reinterpret_cast<float *>(scratch + PS::SB);      // [8]
  float *sps = reinterpret_cast<float *>(scratch + PS::SPS);    // [D/32][8][2]
  const float *cent = reinterpret_cast<const float *>(scratch + PS::CENT);
  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();

  // (1) q' = H (s q) / sqrt(D): one wave per head, lane l holding elements
  //     E l .. E l + E - 1 (index bit 0 in registers for D = 128, the others
  //     across the lanes)
#pragma unroll
  for (int kh = 0; kh < PrepIn<D, NW>::HPW; ++kh) {
    const int h = wave + NW * kh;
    if (h >= GE) break;
    float x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = in.q[kh][e] * in.s[e];
    if constexpr (E == 2) {
      const float a0 = x[0] + x[1], a1 = x[0] - x[1];
      x[0] = a0;
      x[1] = a1;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = wave_fwht(x[e], lane) * (1.0f / sqrtf(static_cast<float>(D)));
    float mq = 0.f, s1 = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      mq = fmaxf(mq, fabsf(x[e]));
      s1 += x[e];
    }
    mq = wave_max(mq);
    s1 = wave_sum(s1);
    if (lane == 0) { sst[4 * h] = mq; sst[4 * h + 1] = s1; }
    if constexpr (!QJ) {
#pragma unroll
      for (int e = 0; e < E; ++e) sq[h * D + E * lane + e] = x[e];
      continue;
    }
    // the GEMV's B operand: q' times 2^sexp (max |q'| below 2^14), as fp16
    // hi + lo (22 significant bits)
    int ex = 0;
    (void)frexpf(mq, &ex);
    const float up = ldexpf(1.0f, min(14 - ex, 100));
    if constexpr (E == 2) {
      *reinterpret_cast<float2 *>(sq + h * D + 2 * lane) = make_float2(x[0], x[1]);
      uint32_t hi, lo;
      split_pair(x[0] * up, x[1] * up, hi, lo);
      reinterpret_cast<uint32_t *>(sqh + h * D)[lane] = hi;
      reinterpret_cast<uint32_t *>(sql + h * D)[lane] = lo;
    } else {
      sq[h * D + lane] = x[0];
      const float nb = __shfl_xor(x[0], 1);     // the pair (2 m, 2 m + 1) in the even lane
      uint32_t hi, lo;
      split_pair(x[0] * up, nb * up, hi, lo);
      if ((lane & 1) == 0) {
        reinterpret_cast<uint32_t *>(sqh + h * D)[lane / 2] = hi;
        reinterpret_cast<uint32_t *>(sql + h * D)[lane / 2] = lo;
      }
    }
  }
  lds_barrier();

  // (2) p = S q' on the matrix cores (v_mfma_f32_32x32x16_f16), one 32-row
  //     tile of S per wave: A = 32 sketch rows x 16 columns (fp16, exact),
  //     B = 16 entries of q' for the columns = heads (lanes of absent heads
  //     zero) as fp16 hi + lo, two MFMAs per K step: fp32-grade sums. The
  //     epilogue also leaves the tile's max |p| and sum p per head. The
  //     other waves compute the basis coefficients. (The centroids are in
  //     the scratch from here on.)
  if (QJ && wave < D / 32) {
    const int h = lane % 32, half = lane / 32;
    const bool live = h < GE;
    v16f c = {};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const uint4 au = in.sk[ks];                         // sketch row 32 wave + h, columns 16 ks + 8 half ..
      V8H av, bh, bl;
      av.u[0] = au.x; av.u[1] = au.y; av.u[2] = au.z; av.u[3] = au.w;
      const uint4 uh = live ? *reinterpret_cast<const uint4 *>(sqh + h * D + 16 * ks + 8 * half) : make_uint4(0u, 0u, 0u, 0u);
      const uint4 ul = live ? *reinterpret_cast<const uint4 *>(sql + h * D + 16 * ks + 8 * half) : make_uint4(0u, 0u, 0u, 0u);
      bh.u[0] = uh.x; bh.u[1] = uh.y; bh.u[2] = uh.z; bh.u[3] = uh.w;
      bl.u[0] = ul.x; bl.u[1] = ul.y; bl.u[2] = ul.z; bl.u[3] = ul.w;
      c = mfma_f16_32x32x16(av.h, bh.h, c);
      c = mfma_f16_32x32x16(av.h, bl.h, c);
    }
    late_loads();
    int ex = 0;
    if (live) (void)frexpf(sst[4 * h], &ex);
    const int sexp = min(14 - ex, 100);
    // lane holds rows 8 (q / 4) + 4 half + q % 4 of the tile, column h
    float mp = 0.f, s2 = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const float v = ldexpf(c[q], -sexp);
      if (live) sp[h * D + 32 * wave + 8 * (q / 4) + 4 * half + (q % 4)] = v;
      mp = fmaxf(mp, fabsf(v));
      s2 += v;
    }
    mp = fmaxf(mp, swap_half_f(mp));
    s2 += swap_half_f(s2);
    if (live && half == 0) { sps[(wave * 8 + h) * 2] = mp; sps[(wave * 8 + h) * 2 + 1] = s2; }
  } else {
    late_loads();
    const int s = tid - (QJ ? (D / 32) * kWave : 0);
    if (s >= 0 && s < NB) sb[s] = basis_coeff(cent, KL, basis_mask(KL, s));
  }
  lds_barrier();

  // (3) per (head, coordinate): the exponents and the digits of every
  //     operand -- the operand value in fixed point, 2 beta_s q'_c or 2 p_c
  //     times 2^(7 + e - c % 8) (c % 8 is the bit of the plane word whose
  //     expanded byte weighs 2^(c % 8) in the MFMA; the top bit's byte is
  //     negative), as four signed 8-bit digits -- each byte written straight
  //     into the fragment layout (FRAG, over the consumed sketch): lane slot
  //     l = row l%16 (head 4 rg + (l%16)/4, digit l%4), K slots 16 (l/16) +
  //     4 r + jb <-> coordinate 32 word + 8 jb + 4 (kg & 1) + r
  //     (slot_coord); coordinate 0's thread also records the head's
  //     constants
  uint8_t *frag = scratch + PS::FRAG;
  const float cmax = cent[L - 1];
  float mb = 0.f;
#pragma unroll
  for (int s = 0; s < NB; ++s) mb = fmaxf(mb, fabsf(sb[s]));
  for (int e = tid; e < GE * D; e += NW * kWave) {
    const int hl = e / D, coord = e % D;
    float mp = 0.f, s2 = 0.f;
    if constexpr (QJ) {
#pragma unroll
      for (int t = 0; t < D / 32; ++t) { mp = fmaxf(mp, sps[(t * 8 + hl) * 2]); s2 += sps[(t * 8 + hl) * 2 + 1]; }
    }
    const int el = fixed_exponent(2.0f * mb * sst[4 * hl]);
    const int eq = fixed_exponent(2.0f * mp);
    const int k = coord & 7, word = coord >> 5;
    const int half = (D == 128) ? (word & 1) : 0;
    const int kg = 2 * ((D == 128) ? (word >> 1) : word) + (k >> 2);
    const int j = 4 * (k & 3) + ((coord >> 3) & 3);
    const int rg = hl >> 2, u = hl & 3;
#pragma unroll
    for (int m = 0; m < NK; ++m) {
      const bool qjl = m == NB;
      const float coef = qjl ? 2.0f : 2.0f * sb[m];
      float v = ldexpf(coef * (qjl ? sp : sq)[hl * D + coord], 7 - k + (qjl ? eq : el));
      if (k == 7) v = -v;
      const uint32_t dig = signed_digits(__float2int_rn(v));
      uint8_t *dst = frag + (rg * NMF + m * NH + half) * 1024 + (16 * kg + 4 * u) * 16 + j;
#pragma unroll
      for (int sd = 0; sd < 4; ++sd) dst[16 * sd] = static_cast<uint8_t>(dig >> (8 * sd));
    }
    if (coord == 0) {
      scon[4 * hl] = ldexpf(1.0f, -7 - el);
      scon[4 * hl + 1] = cmax * sst[4 * hl + 1];
      scon[4 * hl + 2] = QJ ? ldexpf(1.0f, -7 - eq) : 0.f;
      scon[4 * hl + 3] = s2;
    }
  }
  lds_barrier();

  // (4) every wave loads every fragment; rows of absent heads (never
  //     written above) are zeroed
  const int kgl = lane / 16;
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg) {
    const bool live = 4 * rg + (lane % 16) / 4 < GE;
#pragma unroll
    for (int mf = 0; mf < NMF; ++mf) {
      const uint4 v = *reinterpret_cast<const uint4 *>(frag + ((rg * NMF + mf) * kWave + lane) * 16);
      a[rg][mf] = live ? v4i{static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z), static_cast<int>(v.w)}
                       : v4i{0, 0, 0, 0};
    }
    const int h = 4 * rg + kgl;
    fh[rg] = (h < GE) ? *reinterpret_cast<const float4 *>(scon + 4 * h) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// The lane's operands and head constants from a prepared record copied to
// the start of the scratch (fragments, then the constants).
template <int D, int KW, int NRG>
__device__ __forceinline__ void load_prepared(const uint8_t *scratch, int GE, v4i (&a)[NRG][PrepShape<D, KW, NRG>::NMF],
                                              float4 (&fh)[NRG]) {
  using PS = PrepShape<D, KW, NRG>;
  const int lane = lane_id(), kg = lane / 16;
  const float *scon = reinterpret_cast<const float *>(scratch + PS::REC_FRAG);
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg) {
#pragma unroll
    for (int mf = 0; mf < PS::NMF; ++mf) {
      const uint4 u = *reinterpret_cast<const uint4 *>(scratch + ((rg * PS::NMF + mf) * kWave + lane) * 16);
      a[rg][mf] = v4i{static_cast<int>(u.x), static_cast<int>(u.y), static_cast<int>(u.z), static_cast<int>(u.w)};
    }
    const int h = 4 * rg + kg;
    fh[rg] = (h < GE) ? *reinterpret_cast<const float4 *>(scon + 4 * h) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// Wait until at most n_after * P of this wave's loads are in flight
// (n_after < 8): every load issued before the last n_after splits is done.
template <int P>
__device__ __forceinline__ void wait_splits(int n_after) {
  switch (n_after) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<P>(); break;
    case 2: wait_vm<2 * P>(); break;
    case 3: wait_vm<3 * P>(); break;
    case 4: wait_vm<4 * P < 63 ? 4 * P : 63>(); break;
    case 5: wait_vm<5 * P < 63 ? 5 * P : 63>(); break;
    default: wait_vm<6 * P < 63 ? 6 * P : 63>(); break;
  }
}

// ------------------------------------------------------------------ fp8 keys

typedef __bf16 v8bf16 __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

union BF8 {
  uint4 u;
  v8bf16 v;
};

// Stage the raw query rows of heads [h0, h0 + GE) at scratch (one 16-byte
// load per lane; lanes past the end idle).
template <int D>
__device__ __forceinline__ void issue_q_rows(const ScanParams &p, int64_t bh, int GE, uint8_t *scratch, int wave) {
  const int es = (p.xt == 0) ? 4 : 2;
  const int upr = D * es / 16;
  const int unit = wave * kWave + lane_id();
  if (unit < GE * upr) {
    const int64_t row = query_row(p, bh / p.n_kv, bh % p.n_kv, head_chunk0(p) + unit / upr);
    dma16_at(static_cast<const uint8_t *>(p.q) + row * D * es + (unit % upr) * 16, scratch + unit * 16);
  }
}

// A operands of the fp8-key logits, v_mfma_f32_16x16x32_bf16 over 32
// coordinates per product: row i = 4 u + part of row group rg is head
// 4 rg + u's query split exactly into bf16 parts q = hi + mid + lo (part 3
// zero); lane (i, kg) holds coordinates 32 s + 8 kg .. + 7 of its row.
template <int D, int NRG>
__device__ __forceinline__ void k8_operands(const ScanParams &p, int GE, const uint8_t *qrows,
                                            v8bf16 (&a8)[NRG][D / 32]) {
  const int lane = lane_id(), i = lane % 16, kg = lane / 16;
  const int part = i % 4;
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg) {
    const int hl = 4 * rg + i / 4;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      BF8 o;
      uint32_t w[4] = {0u, 0u, 0u, 0u};
      if (hl < GE && part < 3) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int at = hl * D + 32 * s + 8 * kg + e;
          float x;
          if (p.xt == 0) x = reinterpret_cast<const float *>(qrows)[at];
          else if (p.xt == 1) x = bf16_bits_to_float(reinterpret_cast<const uint16_t *>(qrows)[at]);
          else x = f16_bits_to_float(reinterpret_cast<const uint16_t *>(qrows)[at]);
          uint16_t b = float_to_bf16_bits(x);
          for (int k = 0; k < part; ++k) {             // the remainders are exact in fp32
            x -= bf16_bits_to_float(b);
            b = float_to_bf16_bits(x);
          }
          w[e / 2] |= static_cast<uint32_t>(b) << (16 * (e % 2));
        }
      }
      o.u = make_uint4(w[0], w[1], w[2], w[3]);
      a8[rg][s] = o.v;
    }
  }
}

// Logits of one 16-key tile of fp8 keys (chunk-major in LDS at kb): lane
// (kg, n) converts key n's coordinates 32 s + 8 kg .. + 7 to bf16 (exact)
// as the B operand; the sum of the C rows of the lane's head is q . key.
template <int D, int NRG>
__device__ __forceinline__ void k8_tile_logits(const uint8_t *kb, const v8bf16 (&a8)[NRG][D / 32], int nrg,
                                               float (&dot)[NRG]) {
  const int lane = lane_id(), col = lane % 16, kg = lane / 16;
  v4f c[NRG];
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg) c[rg] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    const uint2 raw = *reinterpret_cast<const uint2 *>(kb + (16 * (2 * s + (kg >> 1)) + col) * 16 + 8 * (kg & 1));
    const auto b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, 1.0f, false);
    const auto b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, 1.0f, true);
    const auto b2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, 1.0f, false);
    const auto b3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, 1.0f, true);
    BF8 bo;
    bo.u = make_uint4(__builtin_bit_cast(uint32_t, b0), __builtin_bit_cast(uint32_t, b1),
                      __builtin_bit_cast(uint32_t, b2), __builtin_bit_cast(uint32_t, b3));
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg)
      if (rg < nrg) c[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8[rg][s], bo.v, c[rg], 0, 0, 0);
  }
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg) dot[rg] = (c[rg][0] + c[rg][1]) + (c[rg][2] + c[rg][3]);
}

// ------------------------------------------------------------------ append

// Element i of a row of dtype xt (0 f32, 1 bf16, 2 f16).
__device__ __forceinline__ float load_elem(const void *base, int64_t i, int xt) {
  if (xt == 0) return static_cast<const float *>(base)[i];
  const uint16_t u = static_cast<const uint16_t *>(base)[i];
  return xt == 1 ? bf16_bits_to_float(u) : f16_bits_to_float(u);
}

// Lloyd-Max decision of one rotated coordinate v against the thresholds
// scaled by ||v|| (th, cent: the codebook in LDS), by the same rule as the
// encode kernels: the sign of v gives the top index bit (v = -0 counts as
// positive) and j = #{k : |v| >= t_{L/2+k} ||v||} over the upper half's
// nonzero thresholds, idx = L/2 + j (v >= 0) or L/2 - 1 - j (v < 0), so that
// a negative v equal to a scaled threshold takes the cell further from zero
// exactly as there; c = cent[idx].
template <int W>
__device__ __forceinline__ void decide_scaled(float v, float vn, const float *th, const float *cent, int &idx,
                                              float &c) {
  constexpr int H = (1 << W) / 2;
  const float a = fabsf(v);
  int j = 0;
#pragma unroll
  for (int k = 0; k < H - 1; ++k) j += (a >= th[H + k] * vn) ? 1 : 0;
  idx = (v >= 0.f) ? H + j : H - 1 - j;
  c = cent[idx];
}

// The new token of group bh, encoded by the one extra block of an append
// launch (4 D threads), which also contributes that token's softmax partial
// for the heads [h0, h0 + GE): the cached context ends one slot earlier for
// the scan blocks, so every head still attends over all ctx_lens[b] tokens.
// Encoding as the encode kernels (store the norm, rotate, Lloyd-Max
// decisions against the thresholds scaled by ||H diag(s) x||; keys: the
// residual, its norm and the signs of its projection S r), written into slot
// t = ctx_lens[b] - 1 of both caches; the value words of slot t's 32-token
// block change in bit t % 32 only. The token's logit takes the same
// estimator from the stored (fp16) norms, in floating point (the queries'
// q' and p = S q' formed here as well); its partial is {m = sm_scale * logit,
// l = 1, acc = n_v c_v[idx]} in the rotated value domain.
// The block shares the CUs with the scan blocks, so it is written for
// latency: every global load it needs is issued first.
// Scratch (over the block's LDS ring): ROT [10][D] floats, the rotated rows
// (q' of each head, the key's residual r, the value's rotation); PZ [9][D]
// their projections (p of each head, z = S r); CK [D] the key's c[idx]; VH
// [D] the decoded value; the key record and stored norms; CB the key and
// value codebooks [4][16] (thresholds, centroids); PART [4][9][D] doubles,
// the projections' partial sums over quarters of the columns of S.
// MSE-only key records: no residual, projections or sign plane; the logit
// is the estimator's first term.
template <int D, int KW, int VW>
__device__ __forceinline__ void append_block(const ScanParams &p, int64_t bh, int GE, int nb, uint8_t *scratch) {
  constexpr bool QJ = key_qjl(KW);
  constexpr int KL = key_lm(KW);
  constexpr int NW = D / 16, E = D / kWave;
  constexpr int RPW = (10 + NW - 1) / NW;                  // rows per wave
  constexpr int REC = key_planes(KW) * D / 8;
  constexpr int KQ = D / 4;                                 // columns of S per thread
  float *rot = reinterpret_cast<float *>(scratch);
  float *pz = rot + 10 * D;
  float *ck = pz + 9 * D;
  float *vh = ck + D;
  uint32_t *rec = reinterpret_cast<uint32_t *>(vh + D);      // REC bytes
  float *shat = reinterpret_cast<float *>(rec + REC / 4);     // stored key norm, gamma
  float *cb = reinterpret_cast<float *>(scratch) + 21 * D + 64;                 // [4][16]
  double *part_s = reinterpret_cast<double *>(scratch + (21 * D + 128) * 4);  // [4][9][D]
  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  const int G = p.group, n_q = p.n_kv * G;
  const int64_t b = bh / p.n_kv, kvh = bh % p.n_kv;
  int64_t ctx = p.ctx_lens ? static_cast<int64_t>(p.ctx_lens[b]) : p.max_ctx;
  ctx = ctx < 0 ? 0 : (ctx > p.max_ctx ? p.max_ctx : ctx);
  float *part = p.partials + (bh * (nb + 1) + nb) * G * (D + 2);
  if (ctx < 1) {                                   // nothing to append: an empty partial
    for (int e = tid; e < GE * (D + 2); e += 4 * D) {
      const int hl = e / (D + 2), i = e % (D + 2);
      part[(head_chunk0(p) + hl) * (D + 2) + i] = (i == 0) ? -INFINITY : 0.f;
    }
    return;
  }
  const int64_t t = ctx - 1;
  const int64_t slot = bh * p.cap + t;
  const int64_t nblk = p.cap / kValueBlock;
  const uint32_t vbit = 1u << (t % kValueBlock);

  // 0. loads: this thread's quarter row of S (row j, columns [KQ kq, KQ kq +
  //    KQ)), the rows of this wave (query heads, key, value; as float) and
  //    their signs, for the value row the words its bits go into, and the
  //    codebooks (into LDS)
  if (tid < 64) {
    const int which = tid / 16, k = tid % 16;
    const int lv = 1 << ((which < 2) ? KL : VW);
    const float *src = (which == 0) ? p.kthr : (which == 1) ? p.kcent : (which == 2) ? p.vthr : p.vcent;
    if (k < lv - ((which & 1) ? 0 : 1)) cb[tid] = src[k];
  }
  const int j = tid % D, kq = tid / D;
  uint4 sk[KQ / 8];
  if constexpr (QJ) {
#pragma unroll
    for (int u = 0; u < KQ / 8; ++u)
      sk[u] = *reinterpret_cast<const uint4 *>(p.sketch + static_cast<int64_t>(j) * D + KQ * kq + 8 * u);
  }
  float x[RPW][E], sgn[RPW][E];
  uint32_t vw_old[E][VW];
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    const int r = wave + NW * k;
    if (r < GE + 2) {
      const bool isq = r < GE;
      const float *sg = (r == GE + 1) ? p.vsigns : p.ksigns;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int i = lane + kWave * e;
        x[k][e] = isq ? load_elem(p.q, (b * n_q + kvh * G + head_chunk0(p) + r) * D + i, p.xt)
                      : load_elem(r == GE ? p.k_new : p.v_new, bh * D + i, p.kv_t);
        sgn[k][e] = sg[i];
      }
      if (r == GE + 1) {
#pragma unroll
        for (int e = 0; e < E; ++e)
#pragma unroll
          for (int q = 0; q < VW; ++q)
            vw_old[e][q] = p.vcodes_w[((bh * nblk + t / kValueBlock) * VW + q) * D + lane + kWave * e];
      }
    }
  }

  __syncthreads();                                 // the codebooks

  // 1. rotations, one wave per row; the key and value rows are encoded
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    const int r = wave + NW * k;
    if (r >= GE + 2) break;
    const bool isq = r < GE, isv = r == GE + 1;
    float y[E];
#pragma unroll
    for (int e = 0; e < E; ++e) y[e] = x[k][e] * sgn[k][e];
    if constexpr (E == 2) {
      const float a0 = y[0] + y[1], a1 = y[0] - y[1];
      y[0] = a0;
      y[1] = a1;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) y[e] = wave_fwht(y[e], lane);
    if (isq) {
#pragma unroll
      for (int e = 0; e < E; ++e) rot[r * D + lane + kWave * e] = y[e] * (1.0f / sqrtf(static_cast<float>(D)));
      continue;
    }
    // v = H diag(s) x: ||v||^2 = D ||x||^2
    float s2 = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) s2 = fmaf(y[e], y[e], s2);
    const float n2 = wave_sum(s2);
    const float nrm = sqrtf(n2 * (1.0f / static_cast<float>(D)));
    const bool nz = n2 > 0.f;
    const float vn = nz ? sqrtf(n2) : 1.0f;
    int idx[E];
    float cq[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (isv) decide_scaled<VW>(y[e], vn, cb + 32, cb + 48, idx[e], cq[e]);
      else decide_scaled<KL>(y[e], vn, cb, cb + 16, idx[e], cq[e]);
    }
    const uint16_t nh = float_to_f16_bits(nrm);
    if (isv) {
      const float nv = f16_bits_to_float(nh);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int i = lane + kWave * e;
        vh[i] = nv * cq[e];
#pragma unroll
        for (int q = 0; q < VW; ++q)
          p.vcodes_w[((bh * nblk + t / kValueBlock) * VW + q) * D + i] =
              ((idx[e] >> q) & 1) ? (vw_old[e][q] | vbit) : (vw_old[e][q] & ~vbit);
      }
      if (lane == 0) p.vscal_w[slot] = nh;
      continue;
    }
    // key: r = y - c[idx] (y = v / ||v||; the zero vector has y = 0), gamma,
    // the index planes of the record
    const float rs = nz ? 1.0f / vn : 0.f;
    float g2 = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = lane + kWave * e;
      const float rr = fmaf(y[e], rs, -cq[e]);
      ck[i] = cq[e];
      rot[GE * D + i] = rr;
      g2 = fmaf(rr, rr, g2);
    }
    const float gamma = sqrtf(wave_sum(g2));
#pragma unroll
    for (int q = 0; q < KL; ++q)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint64_t m = __ballot((idx[e] >> q) & 1);
        if (lane == 0) {
          rec[q * (D / 32) + 2 * e] = static_cast<uint32_t>(m);
          rec[q * (D / 32) + 2 * e + 1] = static_cast<uint32_t>(m >> 32);
        }
      }
    if (lane == 0) {
      shat[0] = f16_bits_to_float(nh);
      if constexpr (QJ) {
        const uint16_t gh = float_to_f16_bits(gamma);
        shat[1] = f16_bits_to_float(gh);
        reinterpret_cast<uint32_t *>(p.kscal_w)[slot] = static_cast<uint32_t>(nh) | (static_cast<uint32_t>(gh) << 16);
      } else {
        shat[1] = 0.f;
        p.kscal_w[slot] = nh;
      }
    }
  }
  __syncthreads();
  if constexpr (!QJ) {
    // MSE-only record: the index planes, by wave 0; each head's logit
    if (wave == 0 && lane < REC / 4) reinterpret_cast<uint32_t *>(p.kcodes_w + slot * REC)[lane] = rec[lane];
    for (int hl = wave; hl < GE; hl += NW) {
      float slm = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) slm = fmaf(rot[hl * D + lane + kWave * e], ck[lane + kWave * e], slm);
      slm = wave_sum(slm);
      float *ph = part + (head_chunk0(p) + hl) * (D + 2);
      if (lane == 0) { ph[0] = shat[0] * slm * p.sm_scale; ph[1] = 1.0f; }
#pragma unroll
      for (int e = 0; e < E; ++e) ph[2 + lane + kWave * e] = vh[lane + kWave * e];
    }
    return;
  }

  // 2. projections PZ[c] = S ROT[c], c <= GE: thread (j, kq) sums its
  //    quarter of row j for every column, then the four quarters are added.
  //    The key's z = S r (c = GE), whose signs are the record's, in fp64;
  //    the heads' p (for the token's logit) in fp32
  {
    double acck = 0.0;
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.f;
#pragma unroll
    for (int u = 0; u < KQ / 8; ++u) {
      const uint32_t wv[4] = {sk[u].x, sk[u].y, sk[u].z, sk[u].w};
      float sv[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        sv[2 * k] = f16_bits_to_float(static_cast<uint16_t>(wv[k] & 0xffffu));
        sv[2 * k + 1] = f16_bits_to_float(static_cast<uint16_t>(wv[k] >> 16));
      }
      const float4 k0 = *reinterpret_cast<const float4 *>(rot + GE * D + KQ * kq + 8 * u);
      const float4 k1 = *reinterpret_cast<const float4 *>(rot + GE * D + KQ * kq + 8 * u + 4);
      const float kv[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) acck = fma(static_cast<double>(sv[k]), static_cast<double>(kv[k]), acck);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        if (c < GE) {
          const float4 r0 = *reinterpret_cast<const float4 *>(rot + c * D + KQ * kq + 8 * u);
          const float4 r1 = *reinterpret_cast<const float4 *>(rot + c * D + KQ * kq + 8 * u + 4);
          const float rv[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
          for (int k = 0; k < 8; ++k) acc[c] = fmaf(sv[k], rv[k], acc[c]);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c)
      if (c < GE) part_s[(kq * 9 + c) * D + j] = static_cast<double>(acc[c]);
    part_s[(kq * 9 + GE) * D + j] = acck;
  }
  __syncthreads();
  for (int e = tid; e < (GE + 1) * D; e += 4 * D) {
    const int c = e / D, jj = e % D;
    const double s = (part_s[c * D + jj] + part_s[(9 + c) * D + jj]) +
                     (part_s[(18 + c) * D + jj] + part_s[(27 + c) * D + jj]);
    pz[c * D + jj] = static_cast<float>(s);
  }
  __syncthreads();

  // 3. the sign plane and the key record, by wave 0 alone (the other waves
  //    go on to the heads' logits, which read the signs from PZ themselves)
  if (wave == 0) {
    uint32_t sw[2 * E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint64_t m = __ballot(pz[GE * D + lane + kWave * e] >= 0.f);
      sw[2 * e] = static_cast<uint32_t>(m);
      sw[2 * e + 1] = static_cast<uint32_t>(m >> 32);
    }
    if (lane < REC / 4) {
      const int k = lane - KL * (D / 32);                // sign-plane word, or < 0: an index-plane word
      uint32_t w = (k < 0) ? rec[lane] : sw[0];
#pragma unroll
      for (int i = 1; i < 2 * E; ++i) w = (k == i) ? sw[i] : w;
      reinterpret_cast<uint32_t *>(p.kcodes_w + slot * REC)[lane] = w;
    }
  }

  // 4. the token's logit for each head and its partial
  const float kappa = kSqrtHalfPi / static_cast<float>(D);
  for (int hl = wave; hl < GE; hl += NW) {
    float slm = 0.f, sqj = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = lane + kWave * e;
      slm = fmaf(rot[hl * D + i], ck[i], slm);
      sqj += (pz[GE * D + i] >= 0.f) ? pz[hl * D + i] : -pz[hl * D + i];
    }
    slm = wave_sum(slm);
    sqj = wave_sum(sqj);
    const float logit = shat[0] * fmaf(kappa * shat[1], sqj, slm);
    float *ph = part + (head_chunk0(p) + hl) * (D + 2);
    if (lane == 0) { ph[0] = logit * p.sm_scale; ph[1] = 1.0f; }
#pragma unroll
    for (int e = 0; e < E; ++e) ph[2 + lane + kWave * e] = vh[lane + kWave * e];
  }
}

// ------------------------------------------------------------------ scan

// One block per (batch*kv-head, block index within the group) and the heads
// [h0, h0 + GE) of the group, GE <= 4 NRG. The block prepares the queries of
// those heads, then walks the splits bx, bx + nb, ... (SH::S tokens each;
// bx and nb from scan_block_index, scan_blocks) through the LDS ring. Per
// split, each wave:
//  1. computes the logits of its key tiles for every head (key MFMA);
//     LOGITS: stores them and moves on; decode: scales them by sm_scale and
//     publishes its per-head maxima and largest value norm   -- barrier
//  2. merges the split maximum into the running (m, l) (online softmax,
//     m' = max(m, m_split), alpha = exp(m - m')), forms its tokens' weights
//     exp(logit - m') n_v as fixed-point int8 digits (one exponent per
//     split, from its largest value norm) written into the shared MFMA
//     operand tiles, and publishes their exact per-head sums  -- barrier
//  3. contracts the weights with its value coordinates' planes on the
//     matrix cores (int32 over the split) and folds the result into its
//     fp32 accumulators: acc = alpha acc + split sum
//  4. refills the stage buffer with the split NST (ring depth) ahead.
// Decode writes the block's partial {m, l, acc} to the workspace;
// merge_kernel combines them.
template <int D, int KW, int VW, int NRG, bool LOGITS, bool APPEND = false, bool PREPARED = false, int NWAVE = D / 16>
__device__ __forceinline__ void scan_block(const ScanParams &p) {
  constexpr int SPLIT = LOGITS ? kLogitSplit : attend_split<D, KW, VW, NRG>();
  static_assert(LOGITS || NWAVE == D / 16, "decode: one wave per 16 value coordinates");
  using SH = ScanShape<D, KW, VW, LOGITS, SPLIT, NWAVE>;
  constexpr bool K8 = SH::K8;
  static_assert(!(K8 && (LOGITS || APPEND)), "fp8 keys: decode attention only");
  using PS = PrepShape<D, K8 ? 1 : KW, NRG>;
  constexpr int PS_BYTES = K8 ? 4096 : PS::BYTES;   // fp8 keys: the raw query rows only
  constexpr int S = SH::S, NW = SH::NW, KT = SH::KT, VT = SH::VT, REC = SH::REC, P = SH::P;
  constexpr int NMF = PS::NMF;
  constexpr int NBV = Basis<VW>::N;
  constexpr int GMAX = 4 * NRG;
  constexpr int NBG = (NRG == 2 && NBV == 8) ? 4 : NBV;
  // (combine_digits: at most 16 MFMAs accumulate into one digit row)
  static_assert(VT <= 16 && key_frags(D, K8 ? 1 : KW) <= 18, "digit sums in range");
  constexpr int SB = SH::STAGE_BYTES;
  // ring depth: 3 stages for decode; the logit scan (small stages, few
  // splits per block) keeps up to 6 in flight, its query preparation in a
  // region of its own so that every stage can be filled before it
  constexpr int LDS_BUDGET = 160 * 1024 - 2048;
  constexpr int NST_L = (LDS_BUDGET - PS_BYTES) / SB < 6 ? (LDS_BUDGET - PS_BYTES) / SB : 6;
  constexpr bool SEP = LOGITS && NST_L >= 3;
  static_assert(!PREPARED || (LOGITS && SEP), "prepared queries: the logit scan with its own preparation region");
  constexpr int NST = SEP ? NST_L : (SPLIT == 512 ? 2 : kStages);
  constexpr int PREP_AT = SEP ? NST * SB : SB;
  constexpr int RING0 = (NST * SB > PREP_AT + PS_BYTES) ? NST * SB : PREP_AT + PS_BYTES;
  // (the append block's scratch overlays the ring)
  constexpr int APPEND_BYTES = APPEND ? (21 * D + 128) * 4 + 4 * 9 * D * 8 : 0;
  constexpr int RING = RING0 > APPEND_BYTES ? RING0 : APPEND_BYTES;
  static_assert(RING <= LDS_BUDGET - (LOGITS ? 0 : NRG * VT * 1024), "LDS budget");
  static_assert(P * (NST - 1) < 64, "vmcnt range");
  // stage k at ring + k * SB; the query preparation uses [PREP_AT,
  // PREP_AT + PS::BYTES), which (decode) stages 1 and 2 reuse once it is done
  __shared__ __attribute__((aligned(1024))) uint8_t ring[RING];
  __shared__ __attribute__((aligned(16))) uint8_t sfrag[LOGITS ? 16 : NRG * VT * 1024];
  __shared__ float spm[NW][GMAX];
  __shared__ float spnv[NW];
  __shared__ float spsw[NW][GMAX];
  __shared__ float svb[NBV];

  const int G = p.group;
  const int n_q = p.n_kv * G;
  const int h0 = head_chunk0(p);
  const int GE = min(GMAX, G - h0);
  // append launches: grid (groups, nb + 1) with the append blocks at y = 0,
  // so that they are dispatched before every scan block (interleaved with
  // the scan blocks, each finishing one would start another scan block late)
  const int64_t bh = APPEND ? blockIdx.x : blockIdx.y;
  const int64_t b = bh / p.n_kv;
  const int64_t kvh = bh % p.n_kv;
  // prefill: the launch's last head sees the most tokens
  int64_t ctx64 = p.pos0 ? static_cast<int64_t>(p.pos0[b]) + (h0 + GE - 1) / p.qgroup + 1
                         : (p.ctx_lens ? static_cast<int64_t>(p.ctx_lens[b]) : p.max_ctx);
  ctx64 = ctx64 < 0 ? 0 : (ctx64 > p.max_ctx ? p.max_ctx : ctx64);
  // append: one block per group encodes the new token (the last slot of the
  // context) and the others scan the context before it
  const int nb = APPEND ? static_cast<int>(gridDim.y) - 1 : scan_blocks(p);
  const int bx = APPEND ? static_cast<int>(blockIdx.y) - 1 : scan_block_index(p);
  if constexpr (APPEND) {
    if (bx < 0) {
      append_block<D, KW, VW>(p, bh, GE, nb, ring);
      return;
    }
    ctx64 = ctx64 > 0 ? ctx64 - 1 : 0;
  }
  const int ctx = static_cast<int>(ctx64);
  const int n_splits = (ctx + S - 1) / S;
  const int ns = (n_splits > bx) ? (n_splits - bx + nb - 1) / nb : 0;   // splits of this block
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = lane_id();
  const int kg = lane / 16;
  const int col = lane % 16;
  uint32_t mask[4];
  lane_masks(mask);
  const float kappa = (key_qjl(KW) && p.qjl) ? kSqrtHalfPi / static_cast<float>(D) : 0.f;
  const float cvmax = LOGITS ? 0.f : p.vcent[(1 << VW) - 1];
  if (!LOGITS && tid < NBV) svb[tid] = basis_coeff(p.vcent, VW, basis_mask(VW, tid));

  float m_run[NRG], l_run[NRG], accf[NRG];
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg) { m_run[rg] = -INFINITY; l_run[rg] = 0.f; accf[rg] = 0.f; }
  // tokens t < lim[rg] for the lane's head 4 rg + kg (causal in prefill)
  int lim[NRG];
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg) {
    int64_t l = p.pos0 ? static_cast<int64_t>(p.pos0[b]) + (h0 + 4 * rg + kg) / p.qgroup + 1 : ctx64;
    lim[rg] = static_cast<int>(l < 0 ? 0 : (l > ctx64 ? ctx64 : l));
  }

  SeqArrays sa;
  sa.cap = static_cast<int32_t>(p.cap);
  sa.nblk = static_cast<int32_t>(p.cap / kValueBlock);
  sa.kcodes = p.kcodes + bh * p.cap * REC;
  sa.kscal = reinterpret_cast<const uint8_t *>(p.kscalars) + bh * p.cap * key_scalar_bytes(KW);
  sa.vcodes = LOGITS ? nullptr : reinterpret_cast<const uint8_t *>(p.vcodes + bh * sa.nblk * VW * D);
  sa.vscal = LOGITS ? nullptr : reinterpret_cast<const uint8_t *>(p.vscalars) + bh * p.cap * 2;
  v4i a[NRG][NMF];
  float4 fh[NRG];
  v8bf16 a8[NRG][K8 ? D / 32 : 1];
  if constexpr (K8) {
    if (ns > 0) {
      // fp8 keys: the raw query rows, then the bf16 operands from them
      issue_q_rows<D>(p, bh, GE, ring + PREP_AT, wave);
      wait_vm<0>();
      lds_barrier();
      issue_split<D, KW, VW, LOGITS, SPLIT, NWAVE>(sa, bx, ring, wave);
      k8_operands<D, NRG>(p, GE, ring + PREP_AT, a8);
      lds_barrier();                               // every wave holds its operands
      for (int k = 1; k < min(ns, NST); ++k) issue_split<D, KW, VW, LOGITS, SPLIT, NWAVE>(sa, bx + k * nb, ring + k * SB, wave);
    }
  } else if constexpr (PREPARED) {
    if (ns > 0) {
      // the prepared operand fragments and head constants into the
      // preparation's region (separate from the stages), then every stage
      constexpr int64_t PSTR = prepared_stride(D, key_lm(KW));
      const uint8_t *src = p.prepared + (bh * p.n_hchunks + h0 / 8) * PSTR;
      constexpr int FW = NRG * NMF;                  // 1 KB fragments: 64 lanes x 16 bytes
      for (int f = wave; f < FW; f += NW) dma16_at(src + (f * kWave + lane) * 16, ring + PREP_AT + f * 1024);
      if (wave == 0 && lane < 8)
        dma16_at(src + PSTR - 128 + 16 * lane, ring + PREP_AT + PS::REC_FRAG);
      // every stage's key loads behind the record's, then a wait for the
      // record alone
      const int first = min(ns, NST);
      for (int k = 0; k < first; ++k) issue_split<D, KW, VW, LOGITS, SPLIT, NWAVE>(sa, bx + k * nb, ring + k * SB, wave);
      wait_splits<P>(first);
      lds_barrier();
      load_prepared<D, KW, NRG>(ring + PREP_AT, GE, a, fh);
    }
  } else {
    if (ns > 0) {
      // the preparation's inputs first, then the first splits that do not
      // overlap its scratch (all of them for the logit scan, the first one
      // for decode): their loads stream in during the preparation
      PrepIn<D, NWAVE> pin;
      issue_prep<D, KW, NRG, NWAVE>(p, bh, GE, ring + PREP_AT, wave, pin);
      const int first = SEP ? min(ns, NST) : 1;
      // waves with no part in the rotation or the sketch product issue their
      // key loads at once, behind their preparation loads; the others (the
      // preparation's critical path: issuing a split holds a wave for a
      // while) once their part is done
      const bool early = wave >= D / 32 && wave >= GE;
      // every wave's preparation loads go out before the first key load
      __builtin_amdgcn_s_barrier();
      if (early) {
        for (int k = 0; k < first; ++k) issue_split<D, KW, VW, LOGITS, SPLIT, NWAVE>(sa, bx + k * nb, ring + k * SB, wave);
        wait_splits<P>(first);                     // this wave's preparation load, issued before
      } else {
        wait_vm<0>();
      }
      group_prep<D, KW, NRG, NWAVE>(p, GE, ring + PREP_AT, pin, [&] {
        if (!early)
          for (int k = 0; k < first; ++k) issue_split<D, KW, VW, LOGITS, SPLIT, NWAVE>(sa, bx + k * nb, ring + k * SB, wave);
      }, a, fh);
      if constexpr (!SEP) {
        lds_barrier();                             // every wave holds its operands; the scratch is free
        for (int k = first; k < min(ns, NST); ++k) issue_split<D, KW, VW, LOGITS, SPLIT, NWAVE>(sa, bx + k * nb, ring + k * SB, wave);
      }
    }
  }

  for (int it = 0; it < ns; ++it) {
    uint8_t *buf = ring + (it % NST) * SB;
    const int sp = bx + it * nb;
    const int n = min(S, ctx - sp * S);
    wait_splits<P>(min(NST - 1, ns - 1 - it));
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
      const bool valid = tl < n;
      float lr[NRG];                               // the lane's heads' logits of key tl
      if constexpr (K8) {
        k8_tile_logits<D, NRG>(kb, a8, NRG, lr);
#pragma unroll
        for (int rg = 0; rg < NRG; ++rg) lr[rg] *= p.k_scale;
      } else {
        KeyTile<D, KW> kt;
#pragma unroll
        for (int q = 0; q < key_planes(KW); ++q) {
          if constexpr (D == 128) {
            const uint2 v = *reinterpret_cast<const uint2 *>(kb + (16 * q + col) * 16 + 8 * (kg >> 1));
            kt.w[q][0] = v.x;
            kt.w[q][D == 128 ? 1 : 0] = v.y;
          } else {
            kt.w[q][0] = *reinterpret_cast<const uint32_t *>(kb + col * REC + q * 8 + 4 * (kg >> 1));
          }
        }
        if constexpr (key_qjl(KW)) kt.sc = *reinterpret_cast<const uint32_t *>(wb + SH::OFF_S + 64 * u + 4 * col);
        else kt.sc = *reinterpret_cast<const uint16_t *>(wb + SH::OFF_S + 32 * u + 2 * col);
        v4i clm[NRG], cqj[NRG];
        key_tile_mfma<D, KW, NRG>(kt, a, mask, NRG, clm, cqj);
        const float kn = kt.norm(), kgm = kt.gamma();
#pragma unroll
        for (int rg = 0; rg < NRG; ++rg) lr[rg] = tile_logit<key_qjl(KW)>(clm[rg], cqj[rg], fh[rg], kn, kgm, kappa);
      }
      if constexpr (LOGITS) {
#pragma unroll
        for (int rg = 0; rg < NRG; ++rg) {
          const int hl = 4 * rg + kg;
          if (valid && hl < GE) p.logits[(b * n_q + kvh * G + h0 + hl) * p.max_ctx + sp * S + tl] = lr[rg];
        }
        (void)lg; (void)nvv;
      } else {
#pragma unroll
        for (int rg = 0; rg < NRG; ++rg) {
          const float l = lr[rg] * p.sm_scale;
          lg[u][rg] = (valid && sp * S + tl < lim[rg]) ? l : -INFINITY;
          mx[rg] = fmaxf(mx[rg], lg[u][rg]);
        }
        const uint16_t nvb =
            *reinterpret_cast<const uint16_t *>(wb + SH::OFF_S + 16 * SH::KSU * KT + 32 * u + 2 * col);
        const float nvf = f16_bits_to_float(nvb);
        nvv[u] = valid ? nvf : 0.f;
        nvm = fmaxf(nvm, nvv[u]);
      }
    }

    if constexpr (!LOGITS) {
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
      // (a head with no token yet keeps m = -inf: its weights are exp(-inf) = 0)
      float msub[NRG];
#pragma unroll
      for (int rg = 0; rg < NRG; ++rg) msub[rg] = (m_run[rg] == -INFINITY) ? 0.f : m_run[rg];
      float sw[NRG];
#pragma unroll
      for (int rg = 0; rg < NRG; ++rg) sw[rg] = 0.f;
#pragma unroll
      for (int u = 0; u < KT; ++u) {
        const int tl = 16 * (wave + NW * u) + col;
        const int vt = tl / 64, t64 = tl % 64;
        const int k = t64 & 7;
        const int kga = 2 * (t64 >> 5) + ((t64 >> 2) & 1);
        const int jb = (t64 >> 3) & 3, r = t64 & 3;
#pragma unroll
        for (int rg = 0; rg < NRG; ++rg) {
          const float e = __expf(lg[u][rg] - msub[rg]);
          l_run[rg] += e;
          const int fx = __float2int_rn(ldexpf(e * nvv[u], 7 - k + ew));
          sw[rg] = fmaf(static_cast<float>(fx), static_cast<float>(1 << k), sw[rg]);
          const uint32_t dig = signed_digits(k == 7 ? -fx : fx);
          uint8_t *dst = sfrag + (rg * VT + vt) * 1024 + (16 * kga + 4 * kg) * 16 + 4 * r + jb;
#pragma unroll
          for (int s = 0; s < 4; ++s) dst[16 * s] = static_cast<uint8_t>(dig >> (8 * s));
        }
      }
#pragma unroll
      for (int rg = 0; rg < NRG; ++rg) {
        const float t = row_sum16(sw[rg]);
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
        float swt = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) swt += spsw[w][4 * rg + kg];
        const float ssum = fmaf(2.0f, x[rg], -cvmax * static_cast<float>(swt)) * inv;
        accf[rg] = fmaf(accf[rg], alpha[rg], ssum);
      }
    }

    // 4. refill this stage (this wave's region only; its reads are done)
    if (it + NST < ns) {
      wait_lds();
      issue_split<D, KW, VW, LOGITS, SPLIT, NWAVE>(sa, sp + NST * nb, buf, wave);
    }
  }
  if constexpr (LOGITS) return;

  // partial of this block: {m, l, acc[D]} per head of the chunk
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg) {
    const float l = row_sum16(l_run[rg]);
    if (col == 0) spm[wave][4 * rg + kg] = l;
  }
  __syncthreads();
  float *part = p.partials + (bh * (nb + (APPEND ? 1 : 0)) + bx) * G * (D + 2);
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg) {
    const int hl = 4 * rg + kg;
    if (hl < GE) part[(h0 + hl) * (D + 2) + 2 + 16 * wave + col] = accf[rg];
  }
  if (wave == 0 && col == 0) {
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) {
      const int hl = 4 * rg + kg;
      if (hl < GE) {
        float l = 0.f;
        for (int w = 0; w < NW; ++w) l += spm[w][hl];
        part[(h0 + hl) * (D + 2)] = m_run[rg];
        part[(h0 + hl) * (D + 2) + 1] = l;
      }
    }
  }
}

template <int D, int KW, int VW, int NRG>
__global__ __launch_bounds__(4 * D) void decode_kernel(ScanParams p) {   // 4 D = (D / 16) waves
  scan_block<D, KW, VW, NRG, false>(p);
}

// Decode attention whose launch also appends the new token (one more block
// per group; the partials hold one more split).
template <int D, int KW, int VW, int NRG>
__global__ __launch_bounds__(4 * D) void append_decode_kernel(ScanParams p) {
  scan_block<D, KW, VW, NRG, false, true>(p);
}

// Waves per logit-scan block: twice the decode block's for chunks of up to 4
// heads (the A operands then fit in the registers of four waves per SIMD),
// so that the matrix and vector pipes of each SIMD can overlap across waves.
template <int D, int NRG>
struct LogitWaves {
  static constexpr int value = NRG == 1 ? D / 8 : D / 16;
};

template <int D, int KW, int NRG>
__global__ __launch_bounds__(kWave * (NRG == 1 ? D / 8 : D / 16)) void logits_kernel(ScanParams p) {
  constexpr int NWL = LogitWaves<D, NRG>::value;
  scan_block<D, KW, 1, NRG, true, false, false, NWL>(p);
}

// The logit scan from prepared queries (tq_prepare_queries).
template <int D, int KW, int NRG>
__global__ __launch_bounds__(kWave * (NRG == 1 ? D / 8 : D / 16)) void logits_prepared_kernel(ScanParams p) {
  constexpr int NWL = LogitWaves<D, NRG>::value;
  scan_block<D, KW, 1, NRG, true, false, true, NWL>(p);
}

// The query preparation of one (group, head chunk) alone, as a scan block
// does it, written out as a record of prepared_stride bytes: the operand
// fragments (as the scan blocks hold them in LDS) and the heads' constants.
template <int D, int KW, int NRG>
__global__ __launch_bounds__(4 * D) void prep_kernel(ScanParams p) {
  using PS = PrepShape<D, KW, NRG>;
  __shared__ __attribute__((aligned(1024))) uint8_t scratch[PS::BYTES];
  const int GE = min(4 * NRG, p.group - head_chunk0(p));
  const int64_t bh = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  PrepIn<D, D / 16> pin;
  issue_prep<D, KW, NRG>(p, bh, GE, scratch, wave, pin);
  wait_vm<0>();
  v4i a[NRG][PS::NMF];
  float4 fh[NRG];
  group_prep<D, KW, NRG>(p, GE, scratch, pin, [] {}, a, fh);
  // fragment f = rg NMF + mf (as the scan blocks hold it) is written by
  // wave f % NW from its registers; the constants from the scratch
  constexpr int64_t PSTR = prepared_stride(D, key_lm(KW));
  uint8_t *dst = p.prepared_w + (bh * p.n_hchunks + head_chunk0(p) / 8) * PSTR;
  constexpr int NW = D / 16;
  const int lane = lane_id();
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
    for (int mf = 0; mf < PS::NMF; ++mf) {
      const int f = rg * PS::NMF + mf;
      if (f % NW == wave) {
        const v4i &v = a[rg][mf];
        *reinterpret_cast<uint4 *>(dst + (f * kWave + lane) * 16) =
            make_uint4(static_cast<uint32_t>(v[0]), static_cast<uint32_t>(v[1]), static_cast<uint32_t>(v[2]),
                       static_cast<uint32_t>(v[3]));
      }
    }
  (void)fh;
  if (threadIdx.x < 8)
    *reinterpret_cast<uint4 *>(dst + PSTR - 128 + 16 * threadIdx.x) =
        *reinterpret_cast<const uint4 *>(scratch + PS::SCON + 16 * threadIdx.x);
}

// Merge of the split partials of one (batch, kv-head) group and head chunk
// (8 heads), one wave per head: log-sum-exp weights over the blocks, division
// by the softmax sum, inverse rotation out = diag(s_v) H acc / sqrt(D) (the
// wave butterflies, lane l holding coordinates l + 64 e), store. A kernel of
// its own: the partials are visible to it without any device-wide fence
// (inside one kernel that fence writes back every XCD's L2 per block).
constexpr int kMergeThreads = 8 * kWave;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(ScanParams p) {
  constexpr int E = D / kWave;
  const int G = p.group;
  const int hl = static_cast<int>(threadIdx.x) / kWave;   // head of the chunk
  const int h0 = 8 * blockIdx.x;
  if (hl >= min(8, G - h0)) return;                        // (no block barrier below)
  const int lane = lane_id();
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / p.n_kv;
  const int64_t kvh = bh % p.n_kv;
  const int nb = p.nb + p.append;                          // partials per group
  const int64_t pstride = static_cast<int64_t>(G) * (D + 2);
  const float *ph = p.partials + bh * nb * pstride + (h0 + hl) * (D + 2);
  // one pass over the partials, MB at a time: every load of a batch is
  // issued before any is used (the partials come from other XCDs' blocks,
  // so each round trip goes to memory), and the running sums are rescaled
  // when a batch raises the maximum. With at most MB partials this is the
  // plain max-then-sum merge.
  constexpr int MB = 8;
  float M = -INFINITY, L = 0.f;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int j0 = 0; j0 < nb; j0 += MB) {
    float mj[MB], lj[MB], aj[MB][E];
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      const float *pj = ph + min(j0 + u, nb - 1) * pstride;   // (batch tail: re-read, weight 0)
      mj[u] = pj[0];
      lj[u] = pj[1];
#pragma unroll
      for (int e = 0; e < E; ++e) aj[u][e] = pj[2 + lane + kWave * e];
    }
    float mx = M;
#pragma unroll
    for (int u = 0; u < MB; ++u)
      if (j0 + u < nb) mx = fmaxf(mx, mj[u]);
    const float r = (M == -INFINITY) ? 0.f : __expf(M - mx);
    L *= r;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] *= r;
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      const float w = (j0 + u >= nb || mj[u] == -INFINITY) ? 0.f : __expf(mj[u] - mx);
      L = fmaf(lj[u], w, L);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(aj[u][e], w, acc[e]);
    }
    M = mx;
  }
  float x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = (L > 0.f) ? acc[e] / L : 0.f;
  if constexpr (E == 2) {
    const float a0 = x[0] + x[1], a1 = x[0] - x[1];
    x[0] = a0;
    x[1] = a1;
  }
  const int64_t row = query_row(p, b, kvh, h0 + hl);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = lane + kWave * e;
    const float o = wave_fwht(x[e], lane) * p.vsigns[j] * (1.0f / sqrtf(static_cast<float>(D)));
    if (p.out_t == 0) static_cast<float *>(p.out)[row * D + j] = o;
    else static_cast<uint16_t *>(p.out)[row * D + j] = float_to_bf16_bits(o);
  }
}

// ------------------------------------------------------------------ dispatch

template <int D, int KW, int VW, bool APPEND>
static void launch_decode_kv(const ScanParams &p, dim3 grid, hipStream_t st) {
  dim3 block(4 * D);
  if constexpr (APPEND) {
    if (p.group > 4) hipLaunchKernelGGL((append_decode_kernel<D, KW, VW, 2>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((append_decode_kernel<D, KW, VW, 1>), grid, block, 0, st, p);
  } else {
    if (p.group > 4) hipLaunchKernelGGL((decode_kernel<D, KW, VW, 2>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((decode_kernel<D, KW, VW, 1>), grid, block, 0, st, p);
  }
}

// Grid of a scan launch: (blocks, groups, head chunks), or with the chunks
// interleaved into x (INTERLEAVE, more than one chunk and nb a multiple of
// 8: sets q.zin); APPEND: (groups, blocks + 1, chunks).
static inline dim3 scan_grid(ScanParams &q, bool append, bool interleave) {
  const uint32_t groups = static_cast<uint32_t>(q.batch) * q.n_kv;
  const uint32_t chunks = static_cast<uint32_t>(q.n_hchunks);
  q.zin = 0;
  if (append) return dim3(groups, static_cast<uint32_t>(q.nb + 1), chunks);
  if (interleave && chunks > 1 && q.nb % 8 == 0) {
    q.zin = q.n_hchunks;
    return dim3(static_cast<uint32_t>(q.nb) * chunks, groups, 1);
  }
  return dim3(static_cast<uint32_t>(q.nb), groups, chunks);
}

// MODE 0: the logit scan, 1: from prepared queries, 2: the preparation alone.
template <int D, int KW, int MODE>
static void launch_logits_k(const ScanParams &p, dim3 grid, hipStream_t st) {
  dim3 block(4 * D);
  const dim3 b1(kWave * LogitWaves<D, 1>::value), b2(kWave * LogitWaves<D, 2>::value);
  const bool two = p.group > 4;
  if constexpr (MODE == 0) {
    if (two) hipLaunchKernelGGL((logits_kernel<D, KW, 2>), grid, b2, 0, st, p);
    else hipLaunchKernelGGL((logits_kernel<D, KW, 1>), grid, b1, 0, st, p);
  } else if constexpr (MODE == 1) {
    if (two) hipLaunchKernelGGL((logits_prepared_kernel<D, KW, 2>), grid, b2, 0, st, p);
    else hipLaunchKernelGGL((logits_prepared_kernel<D, KW, 1>), grid, b1, 0, st, p);
  } else {
    dim3 g1(1, grid.y, grid.z);
    if (two) hipLaunchKernelGGL((prep_kernel<D, KW, 2>), g1, block, 0, st, p);
    else hipLaunchKernelGGL((prep_kernel<D, KW, 1>), g1, block, 0, st, p);
  }
}

// One launch per call: grid (blocks per group, groups, head chunks of 8
// heads); every block reads its keys once for its chunk. (A chunk of up to
// 4 heads is taken by the single-row-group kernel only when the whole group
// has at most 4 heads.)
// K0: 0 for full key records, kKeyMse for MSE-only ones (key width K0 + w).
template <int D, int MODE, int K0>
hipError_t launch_logits_m(const ScanParams &p, int kw, hipStream_t st) {
  if (p.batch == 0 || p.n_kv == 0 || (MODE != 2 && p.max_ctx == 0)) return hipSuccess;
  ScanParams q = p;
  const dim3 grid = MODE == 2 ? scan_grid(q, false, false) : scan_grid(q, false, true);
  switch (key_lm(kw)) {
    case 1: launch_logits_k<D, K0 + 1, MODE>(q, grid, st); break;
    case 2: launch_logits_k<D, K0 + 2, MODE>(q, grid, st); break;
    case 3: launch_logits_k<D, K0 + 3, MODE>(q, grid, st); break;
    default: launch_logits_k<D, K0 + 4, MODE>(q, grid, st);
  }
  return hipGetLastError();
}

// MSE-only key records (their kernels are instantiated in a translation
// unit of their own)
template <int D>
hipError_t launch_logits_msek_d(const ScanParams &p, int kw, int mode, hipStream_t st) {
  if (mode == 0) return launch_logits_m<D, 0, kKeyMse>(p, kw, st);
  if (mode == 1) return launch_logits_m<D, 1, kKeyMse>(p, kw, st);
  return launch_logits_m<D, 2, kKeyMse>(p, kw, st);
}

template <int D>
hipError_t launch_logits_d(const ScanParams &p, int kw, hipStream_t st) {
  return kw > kKeyMse ? launch_logits_msek_d<D>(p, kw, 0, st) : launch_logits_m<D, 0, 0>(p, kw, st);
}

template <int D>
hipError_t launch_logits_prepared_d(const ScanParams &p, int kw, hipStream_t st) {
  return kw > kKeyMse ? launch_logits_msek_d<D>(p, kw, 1, st) : launch_logits_m<D, 1, 0>(p, kw, st);
}

template <int D>
hipError_t launch_prepare_d(const ScanParams &p, int kw, hipStream_t st) {
  return kw > kKeyMse ? launch_logits_msek_d<D>(p, kw, 2, st) : launch_logits_m<D, 2, 0>(p, kw, st);
}

// One launch over (blocks, groups, head chunks of 8 heads), then the merge.
// APPEND: nb + 1 blocks per group, one of them encoding the group's new
// token (the append block of every head chunk encodes it, to the same
// bytes, for that chunk's partials).
template <int D, int KW, bool APPEND>
static void launch_decode_v(const ScanParams &p, int vw, dim3 grid, hipStream_t st) {
  switch (vw) {
    case 1: launch_decode_kv<D, KW, 1, APPEND>(p, grid, st); break;
    case 2: launch_decode_kv<D, KW, 2, APPEND>(p, grid, st); break;
    case 3: launch_decode_kv<D, KW, 3, APPEND>(p, grid, st); break;
    default: launch_decode_kv<D, KW, 4, APPEND>(p, grid, st);
  }
}

// The scan launch of decode attention over MSE-only key records (their
// kernels are instantiated in translation units of their own).
template <int D, bool APPEND>
void launch_decode_msek_d(const ScanParams &p, int kw, int vw, dim3 grid, hipStream_t st) {
  switch (key_lm(kw)) {
    case 1: launch_decode_v<D, kKeyMse + 1, APPEND>(p, vw, grid, st); break;
    case 2: launch_decode_v<D, kKeyMse + 2, APPEND>(p, vw, grid, st); break;
    case 3: launch_decode_v<D, kKeyMse + 3, APPEND>(p, vw, grid, st); break;
    default: launch_decode_v<D, kKeyMse + 4, APPEND>(p, vw, grid, st);
  }
}

template <int D, bool APPEND>
hipError_t launch_decode_da(const ScanParams &p, int kw, int vw, hipStream_t st) {
  if (p.batch == 0 || p.n_kv == 0) return hipSuccess;
  const uint32_t groups = static_cast<uint32_t>(p.batch) * p.n_kv;
  const uint32_t chunks = static_cast<uint32_t>(p.n_hchunks);
  ScanParams q = p;
  const dim3 grid = scan_grid(q, APPEND, true);
  switch (kw) {
    case 1: launch_decode_v<D, 1, APPEND>(q, vw, grid, st); break;
    case 2: launch_decode_v<D, 2, APPEND>(q, vw, grid, st); break;
    case 3: launch_decode_v<D, 3, APPEND>(q, vw, grid, st); break;
    case 4: launch_decode_v<D, 4, APPEND>(q, vw, grid, st); break;
    case kKeyFp8:
      if constexpr (!APPEND) launch_decode_v<D, kKeyFp8, false>(q, vw, grid, st);
      break;
    default: launch_decode_msek_d<D, APPEND>(q, kw, vw, grid, st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((merge_kernel<D>), dim3(chunks, groups), dim3(kMergeThreads), 0, st, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const ScanParams &p, int kw, int vw, hipStream_t st) {
  return launch_decode_da<D, false>(p, kw, vw, st);
}

template <int D>
hipError_t launch_append_decode_d(const ScanParams &p, int kw, int vw, hipStream_t st) {
  return launch_decode_da<D, true>(p, kw, vw, st);
}

}  // namespace tq
