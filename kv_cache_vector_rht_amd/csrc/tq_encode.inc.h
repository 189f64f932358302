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
// Mapping: a wave encodes 32 tokens (d = 128) or 64 (d = 64, two tiles of
// 32); every token is split over lanes t and t + 32, each holding half of
// every 32-coordinate block, 64 values per lane. The rotation
// H_D = H_{D/32} (x) H_32 runs its 32-point blocks on the matrix cores for
// 16-bit inputs (fp32 inputs: butterflies in registers and one stage across
// the half-waves). A ballot over the wave of one value slot's index bit
// yields two 32-bit value-code words (two coordinates of one 32-token
// block). Key records are assembled per lane pair; the QJL projection of
// each 32-token tile runs on the matrix cores (tq_qjl.h). MSE-only key
// records (the ablation without the QJL stage) take the key path's
// decisions and packing and stop there.
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

// From w = 2 bits on, the decisions use the codebook's symmetry
// (t[L-2-k] = -t[k], t[L/2-1] = 0): the sign of y gives the top index bit,
// a binary search of |y| over the upper half's L/2 - 1 thresholds gives
// j = #{t_{L/2+m} <= |y|}, and idx = L/2 + j (y >= 0) or L/2 - 1 - j
// (y < 0); the lower index bits are j's bits, inverted for y < 0. This is
// #{t <= y} except where a negative y equals a nonzero threshold exactly
// (that tie goes to the lower cell); y = 0 (either sign) goes up. Half the
// select work of the plain search at each level.
template <int W>
struct DecLevels {
  static constexpr bool kSym = W >= 2;
  Levels<kSym ? W - 1 : W> lv;
  // thresholds th[L-1] (LDS), scaled by s
  __device__ __forceinline__ void load(const float *th, float s) {
    lv.load(kSym ? th + (1 << W) / 2 : th);
#pragma unroll
    for (int k = 0; k < (kSym ? (1 << (W - 1)) - 1 : (1 << W) - 1); ++k) {
      lv.t[k] *= s;
      asm volatile("" : "+v"(lv.t[k]));   // scaled once, not after each select
    }
  }
};

// Lane masks m[q] of bit q of idx for one coordinate (y given unscaled, the
// thresholds scaled alike), and with CENT c = c[idx] from c_up, the upper
// half of the (symmetric) codebook.
template <int W, bool CENT>
__device__ __forceinline__ void decide_masks(float y, const DecLevels<W> &dl, const float (&c_up)[(1 << W) / 2],
                                             uint64_t (&m)[W], float &c) {
  if constexpr (DecLevels<W>::kSym) {
    const bool up = y >= 0.f;                       // also for y = -0
    bool jd[W - 1];
    decide<W - 1>(fabsf(y), dl.lv, jd);
    const uint64_t mu = __ballot(up);
    m[W - 1] = mu;
#pragma unroll
    for (int q = 0; q < W - 1; ++q) m[q] = ~(__ballot(jd[W - 2 - q]) ^ mu);
    if constexpr (CENT) {
      const float cp = pick<W - 1, 0>(c_up, jd);
      c = up ? cp : -cp;
    }
  } else {
    bool dec[W];
    decide<W>(y, dl.lv, dec);
#pragma unroll
    for (int q = 0; q < W; ++q) m[q] = __ballot(dec[W - 1 - q]);
    if constexpr (CENT) c = centroid<W>(c_up, dec);
  }
}

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

union Frag8 {
  uint4 u;
  v8bf b;
  v8h h;
};

// Output row r of a 32x32 MFMA tile is held by lane half (r / 4) % 2 as
// accumulator 4 (r / 8) + r % 4; letting row r stand for coordinate
// 16 ((r / 4) % 2) + 4 (r / 8) + r % 4 of the block gives lane half h the
// block's coordinates 16 h .. 16 h + 15 in accumulator order.
__host__ __device__ constexpr int mfma_row_coord(int r) { return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3); }

// XT: the input's type, 0 fp32, 1 bf16, 2 fp16.
//
// Lane layout (both head sizes): a wave holds NT = 128 / D tiles of 32
// tokens; lane (t, h) = (l % 32, l / 32) holds, for tile T, coordinates
// 32 b + 16 h + i (b < D / 32, i < 16) of token 32 T + t in
// v[(D / 2) T + 16 b + i]: 64 values per lane, each token split over the two
// half-waves.
// Threads per encode block: the block stages the codec once for its waves.
// (Blocks of 512 threads, at 3 or 4 waves per SIMD, measured slower: fewer
// resident waves per CU, or spills at 128 registers.)
constexpr int kEncThreads = 256;

// KIND: 0 values, 1 keys, 2 MSE-only keys (index planes and the norm only).
template <int D, int W, int KIND, int XT>
__global__ __launch_bounds__(kEncThreads) __attribute__((amdgpu_waves_per_eu(2, 8))) void encode_kernel(EncodeParams p) {
  constexpr bool KEY = KIND != 0;              // key record layout
  constexpr bool QJ = KIND == 1;               // with the QJL stage
  constexpr int L = 1 << W;
  constexpr int NT = 128 / D;                // 32-token tiles per wave (1 or 2)
  constexpr int TPW = 32 * NT;               // tokens per wave
  constexpr int CT = D / 2;                  // values per lane and tile
  constexpr int NB = D / 32;                 // 32-coordinate blocks
  __shared__ float s_cent[L];
  __shared__ float s_th[L];
  __shared__ __attribute__((aligned(16))) float s_sign[D];
  __shared__ __attribute__((aligned(16))) uint16_t s_sk[QJ ? D * (D + 8) : 8];
  // 16-bit input: A operands of the rotation's 32-point blocks,
  // [block b][K step e][lane][8 halves]. Lane l holds row l % 32, standing
  // for output coordinate rc = mfma_row_coord(l % 32), and input coordinates
  // k = 16 (l / 32) + 8 e + j: the entry is (-1)^popcount(rc & k) s[32 b + k]
  // (+-1 in the input's type), i.e. H_32 diag(s) restricted to the block.
  constexpr bool MFMA_ROT = XT != 0;
  __shared__ __attribute__((aligned(16))) uint32_t s_ha[MFMA_ROT ? NB * 2 * kWave * 4 : 4];
  if (threadIdx.x < L) s_cent[threadIdx.x] = p.centroids[threadIdx.x];
  if (threadIdx.x < L - 1) s_th[threadIdx.x] = p.thresholds[threadIdx.x];
  for (int i = threadIdx.x; i < D; i += blockDim.x) s_sign[i] = p.signs[i];
  if constexpr (MFMA_ROT) {
    constexpr uint32_t one = XT == 2 ? 0x3C00u : 0x3F80u;
    for (int idx = threadIdx.x; idx < NB * 2 * kWave * 4; idx += blockDim.x) {
      const int jj = idx & 3, ln = (idx >> 2) & 63, e = (idx >> 8) & 1, bb = idx >> 9;
      const int rc = mfma_row_coord(ln & 31);
      uint32_t w = 0u;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int k = 16 * (ln >> 5) + 8 * e + 2 * jj + u;
        const uint32_t neg = (static_cast<uint32_t>(__popc(static_cast<unsigned>(rc & k))) +
                              (p.signs[32 * bb + k] < 0.f ? 1u : 0u)) & 1u;
        w |= (one | (neg << 15)) << (16 * u);
      }
      s_ha[idx] = w;
    }
  }
  if constexpr (QJ) stage_sketch<D, kEncThreads>(p.sketch, s_sk);
  __syncthreads();

  const int lane = lane_id();
  const int tt = lane % 32;                  // token within a tile
  const int hv = lane / 32;                  // which half of every 32-coordinate block
  // each wave encodes token groups wave, wave + (waves in the grid), ...
  const int64_t wave_stride = static_cast<int64_t>(gridDim.x) * (blockDim.x / kWave);
  for (int64_t wave = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + (threadIdx.x / kWave);
       wave < p.n_waves; wave += wave_stride) {
    const int64_t seq = wave / p.groups_per_seq;
    const int64_t g = p.g0 + wave % p.groups_per_seq;
    int64_t pos[NT];                           // cache slot of this lane's token in tile T
    bool active[NT];
#pragma unroll
    for (int T = 0; T < NT; ++T) {
      pos[T] = g * TPW + 32 * T + tt;
      const int64_t t = pos[T] - p.t0;         // input token
      active[T] = (t >= 0) && (t < p.n_tok);
    }
    auto row = [&](int T) { return seq * p.x_seq_stride + (pos[T] - p.t0) * p.x_tok_stride; };

    float v[64];
    float n2[NT];                              // this lane's share of ||v||^2 per token
    if constexpr (MFMA_ROT) {
      // (a2) v = H_D diag(s) x with H_D = H_{D/32} (x) H_32: each 32-point
      // block on the matrix cores (exact +-1 operands, fp32 sums), then the
      // butterflies across blocks in registers
#pragma unroll
      for (int T = 0; T < NT; ++T) {
        Frag8 xb[NB][2];
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            if (active[T]) xb[bb][e].u = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.x) + row(T) + 32 * bb + 16 * hv + 8 * e);
            else xb[bb][e].u = make_uint4(0u, 0u, 0u, 0u);
          }
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
          v16f c = {};
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            Frag8 a;
            a.u = *reinterpret_cast<const uint4 *>(s_ha + ((bb * 2 + e) * kWave + lane) * 4);
            if constexpr (XT == 2) c = mfma_f16_32x32x16(a.h, xb[bb][e].h, c);
            else c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.b, xb[bb][e].b, c, 0, 0, 0);
          }
#pragma unroll
          for (int q = 0; q < 16; ++q) v[CT * T + 16 * bb + q] = c[q];
        }
        float *vt = v + CT * T;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if constexpr (NB == 4) {
            const float a0 = vt[i], a1 = vt[16 + i], a2 = vt[32 + i], a3 = vt[48 + i];
            const float b0 = a0 + a1, b1 = a0 - a1, b2 = a2 + a3, b3 = a2 - a3;
            vt[i] = b0 + b2; vt[16 + i] = b1 + b3; vt[32 + i] = b0 - b2; vt[48 + i] = b1 - b3;
          } else {
            const float a0 = vt[i], a1 = vt[16 + i];
            vt[i] = a0 + a1; vt[16 + i] = a0 - a1;
          }
        }
      }
    } else {
      // fp32 input: sign flip and the in-lane butterfly stages (coordinate
      // bits 0-3 and 5 up) per tile, then coordinate bit 4 across the
      // half-waves. Swapping a value with itself across half-waves leaves the
      // lower half's copy in the first register and the upper half's in the
      // second, in every lane.
      const float sgn = hv ? -1.f : 1.f;
#pragma unroll
      for (int T = 0; T < NT; ++T) {
        float *vt = v + CT * T;
        if (active[T]) {
#pragma unroll
          for (int bb = 0; bb < NB; ++bb) {
            float w[16];
            load_row_vec_f32<16>(static_cast<const float *>(p.x) + row(T) + 32 * bb + 16 * hv, w);
#pragma unroll
            for (int i = 0; i < 16; ++i) vt[16 * bb + i] = w[i];
          }
        } else {
#pragma unroll
          for (int i = 0; i < CT; ++i) vt[i] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < CT; ++i) vt[i] *= s_sign[32 * (i >> 4) + 16 * hv + (i & 15)];
        fwht_regs<CT>(*reinterpret_cast<float (*)[CT]>(vt));
#pragma unroll
        for (int i = 0; i < CT; ++i) {
          const uint32_t u = __float_as_uint(vt[i]);
          auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
          vt[i] = fmaf(sgn, __uint_as_float(r[1]), __uint_as_float(r[0]));
        }
      }
    }

    // (a1) norm from the rotated vector: ||H diag(s) x||^2 = D ||x||^2, the
    // two half-waves' shares added
    float nrm[NT], vn[NT];
    bool nz[NT];
    DecLevels<W> ls[NT];
#pragma unroll
    for (int T = 0; T < NT; ++T) {
      float s2 = 0.f;
#pragma unroll
      for (int i = 0; i < CT; ++i) s2 = fmaf(v[CT * T + i], v[CT * T + i], s2);
      const float o = swap_half_f(s2);
      n2[T] = hv ? (o + s2) : (s2 + o);
      nrm[T] = sqrtf(n2[T] * (1.0f / static_cast<float>(D)));
      // y = v / ||v|| (v = H diag(s) x, ||v|| = n sqrt(D)). The decisions
      // compare v with the thresholds scaled by ||v|| (y >= t <=> v >= t ||v||
      // up to one rounding), the residual takes y - c = fma(v, 1 / ||v||, -c);
      // the zero vector has v = 0, unscaled thresholds and y = 0.
      nz[T] = n2[T] > 0.f;
      vn[T] = nz[T] ? sqrtf(n2[T]) : 1.0f;
    }
    // (read from LDS per group: the unscaled thresholds stay out of the
    // registers that live across the loop)
    asm volatile("" ::: "memory");
#pragma unroll
    for (int T = 0; T < NT; ++T) ls[T].load(s_th, vn[T]);

    if constexpr (KEY) {
      // (a3) indices -> bit planes: each decision's lane mask is added in as
      // the carry of half + half into the 16-bit group of its block
      // (coordinate order reversed, so the first coordinate lands on bit 0);
      // (a4) residual, kept as r' = 2^10 r = fma(v, 2^10 / ||v||, -2^10 c),
      // the scale the QJL projection wants
      float rs[NT];
#pragma unroll
      for (int T = 0; T < NT; ++T) rs[T] = nz[T] ? 1024.0f / vn[T] : 0.f;
      float c_up[L / 2];
#pragma unroll
      for (int j = 0; j < L / 2; ++j) c_up[j] = 1024.0f * s_cent[L / 2 + j];
      uint32_t hw[W][4];                       // group (T, b) = 2 T + b (d = 64) or b (d = 128)
#pragma unroll
      for (int q = 0; q < W; ++q)
#pragma unroll
        for (int k = 0; k < 4; ++k) hw[q][k] = 0u;
#pragma unroll
      for (int i = 63; i >= 0; --i) {
        const int T = i / CT;
        uint64_t m[W];
        float cq;
        decide_masks<W, QJ>(v[i], ls[T], c_up, m, cq);
#pragma unroll
        for (int q = 0; q < W; ++q) {
          uint64_t carry;
          asm("v_addc_co_u32_e64 %0, %1, %0, %0, %2" : "+v"(hw[q][i / 16]), "=s"(carry) : "s"(m[q]));
        }
        if constexpr (QJ) {
          v[i] = fmaf(v[i], rs[T], -cq);
          asm volatile("" : "+v"(v[i]));  // consume the decisions here
        }
        // two values' decisions interleave (they fill each other's wait
        // states between a lane mask's write and its use as a carry)
        if (i % 2 == 0) __builtin_amdgcn_sched_barrier(0);
      }
      // plane words: word b of a token = its group b of lane half 0 | that of
      // lane half 1 << 16. d = 128: lane half h keeps words 2 h, 2 h + 1 of
      // its token; d = 64: word h of each of its two tokens.
      uint32_t pw[W][2];
#pragma unroll
      for (int q = 0; q < W; ++q) {
        if constexpr (D == 128) {
          const uint32_t send = hv ? (hw[q][0] | (hw[q][1] << 16)) : (hw[q][2] | (hw[q][3] << 16));
          auto r = __builtin_amdgcn_permlane32_swap(send, send, false, false);
          const uint32_t recv = hv ? r[0] : r[1];
          pw[q][0] = hv ? ((recv & 0xffffu) | (hw[q][2] << 16)) : (hw[q][0] | (recv << 16));
          pw[q][1] = hv ? ((recv >> 16) | (hw[q][3] << 16)) : (hw[q][1] | (recv & 0xffff0000u));
        } else {
          const uint32_t send = hv ? (hw[q][0] | (hw[q][2] << 16)) : (hw[q][1] | (hw[q][3] << 16));
          auto r = __builtin_amdgcn_permlane32_swap(send, send, false, false);
          const uint32_t recv = hv ? r[0] : r[1];
          pw[q][0] = hv ? ((recv & 0xffffu) | (hw[q][1] << 16)) : (hw[q][0] | (recv << 16));
          pw[q][1] = hv ? ((recv >> 16) | (hw[q][3] << 16)) : (hw[q][2] | (recv & 0xffff0000u));
        }
      }
      if constexpr (!QJ) {
        // MSE-only record: the W index planes, D/8 bytes each; scalar {norm}
        constexpr int REC = W * D / 8;
        constexpr int PB = D / 8;
#pragma unroll
        for (int T = 0; T < NT; ++T) {
          if (active[T]) {
            uint8_t *rec = static_cast<uint8_t *>(p.codes) + (seq * p.cap + pos[T]) * REC + (PB / 2) * hv;
#pragma unroll
            for (int q = 0; q < W; ++q) {
              if constexpr (D == 128) *reinterpret_cast<uint2 *>(rec + q * PB) = make_uint2(pw[q][0], pw[q][1]);
              else *reinterpret_cast<uint32_t *>(rec + q * PB) = pw[q][T];
            }
            if (hv == 0) p.scalars[seq * p.cap + pos[T]] = float_to_f16_bits(nrm[T]);
          }
        }
        continue;
      }
      float gamma[NT];
#pragma unroll
      for (int T = 0; T < NT; ++T) {
        float g2 = 0.f;
#pragma unroll
        for (int i = 0; i < CT; ++i) g2 = fmaf(v[CT * T + i], v[CT * T + i], g2);
        const float o = swap_half_f(g2);
        g2 = hv ? (o + g2) : (g2 + o);
        gamma[T] = sqrtf(g2) * (1.0f / 1024.0f);
      }

      // (a5) QJL sign bits sigma_j = [ (S r)_j >= 0 ], on the matrix cores
      constexpr int REC = (W + 1) * D / 8;
      constexpr int PB = D / 8;
#pragma unroll
      for (int T = 0; T < NT; ++T) {
        uint32_t sig[D / 32];
        qjl_tile<D>(s_sk, v + CT * T, sig);
        if (active[T]) {
          // (a6) record: W index planes then the sign plane, D/8 bytes each;
          // this lane writes bytes [PB/2 hv, PB/2 hv + PB/2) of every plane
          uint8_t *rec = static_cast<uint8_t *>(p.codes) + (seq * p.cap + pos[T]) * REC + (PB / 2) * hv;
          if constexpr (D == 128) {
#pragma unroll
            for (int q = 0; q < W; ++q)
              *reinterpret_cast<uint2 *>(rec + q * PB) = make_uint2(pw[q][0], pw[q][1]);
            *reinterpret_cast<uint2 *>(rec + W * PB) = make_uint2(sig[2 * hv], sig[2 * hv + 1]);
          } else {
#pragma unroll
            for (int q = 0; q < W; ++q) *reinterpret_cast<uint32_t *>(rec + q * PB) = pw[q][T];
            *reinterpret_cast<uint32_t *>(rec + W * PB) = sig[hv];
          }
          if (hv == 0) {
            const uint32_t sc = static_cast<uint32_t>(float_to_f16_bits(nrm[T])) |
                                (static_cast<uint32_t>(float_to_f16_bits(gamma[T])) << 16);
            reinterpret_cast<uint32_t *>(p.scalars)[seq * p.cap + pos[T]] = sc;
          }
        }
      }
    } else {
      // values: the ballot of one value slot gives, in its low half, the bits
      // of coordinate c0 = 32 b + i and, in its high half, of c0 + 16, for
      // the 32 tokens of one tile. The word of coordinate c of 32-token block
      // k goes to lane c % 64 of wr[k][.] (d = 128: k = c / 64 of block g;
      // d = 64: k = T, block 2 g + T).
      uint32_t wr[2][W];
#pragma unroll
      for (int q = 0; q < W; ++q) { wr[0][q] = 0u; wr[1][q] = 0u; }
      // (the decision's own lane mask, masked on the scalar unit: a ballot
      // of a combined condition would first widen it to a vector of 0/1)
      uint64_t valid[NT];
#pragma unroll
      for (int T = 0; T < NT; ++T) valid[T] = __ballot(active[T]);
      const float c_none[L / 2] = {};
      static_for<0, 64>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        constexpr int T = i / CT, b = (i % CT) / 16, j = i % 16;
        constexpr int c0 = 32 * b + j, c1 = c0 + 16;
        constexpr int k = (D == 128) ? c0 / 64 : T;
        uint64_t mq[W];
        float unused;
        decide_masks<W, false>(v[i], ls[T], c_none, mq, unused);
#pragma unroll
        for (int q = 0; q < W; ++q) {
          const uint64_t m = mq[q] & valid[T];
          write_lane<c0 % 64>(wr[k][q], static_cast<uint32_t>(m));
          write_lane<c1 % 64>(wr[k][q], static_cast<uint32_t>(m >> 32));
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      const int64_t nblk = p.cap / kValueBlock;
      uint32_t *words = static_cast<uint32_t *>(p.codes);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t vm = static_cast<uint32_t>(valid[D == 128 ? 0 : k]);
        if (vm == 0u) continue;
        const int64_t blk = (D == 128) ? g : 2 * g + k;
        const int coord = (D == 128) ? 64 * k + lane : lane;
        uint32_t *base = words + (seq * nblk + blk) * W * D + coord;
#pragma unroll
        for (int q = 0; q < W; ++q) {
          uint32_t w = wr[k][q];
          uint32_t *dst = base + q * D;
          if (vm != 0xffffffffu) w = (*dst & ~vm) | (w & vm);
          *dst = w;
        }
      }
#pragma unroll
      for (int T = 0; T < NT; ++T)
        if (active[T] && hv == 0) p.scalars[seq * p.cap + pos[T]] = float_to_f16_bits(nrm[T]);
    }
  }
}

// ---------------------------------------------------------------- dispatch

// Blocks of kEncThreads threads of `kernel` that fit on the current device at once:
// the grid is capped at that so that every block stages the codec once and
// its waves loop over the token groups. `cached` belongs to one kernel.
template <typename K>
static int64_t resident_blocks(K kernel, int (&cached)[64]) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1 << 30;
  if (cached[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kEncThreads, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || per_cu <= 0 || cus <= 0)
      return 1 << 30;
    cached[dev] = per_cu * cus;
  }
  return cached[dev];
}

template <int D, int W, int KIND, int XT>
static void launch_encode_x(const EncodeParams &p, hipStream_t st) {
  static int cached[64] = {};
  const auto kernel = encode_kernel<D, W, KIND, XT>;
  constexpr int wpb = kEncThreads / kWave;
  int64_t blocks = (p.n_waves + wpb - 1) / wpb;
  const int64_t cap = resident_blocks(kernel, cached);
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kEncThreads), 0, st, p);
}

template <int D, int W, int KIND>
static hipError_t launch_encode_dw(const EncodeParams &p, hipStream_t st) {
  switch (p.xt) {
    case 0: launch_encode_x<D, W, KIND, 0>(p, st); break;
    case 1: launch_encode_x<D, W, KIND, 1>(p, st); break;
    default: launch_encode_x<D, W, KIND, 2>(p, st); break;
  }
  return hipGetLastError();
}

template <int D, int KIND>
static hipError_t launch_encode_dk(const EncodeParams &p, int w, hipStream_t st) {
  switch (w) {
    case 1: return launch_encode_dw<D, 1, KIND>(p, st);
    case 2: return launch_encode_dw<D, 2, KIND>(p, st);
    case 3: return launch_encode_dw<D, 3, KIND>(p, st);
    default: return launch_encode_dw<D, 4, KIND>(p, st);
  }
}

template <int D>
hipError_t launch_encode_d(const EncodeParams &p, int w, int kind, hipStream_t st) {
  if (kind == 1) return launch_encode_dk<D, 1>(p, w, st);
  if (kind == 2) return launch_encode_dk<D, 2>(p, w, st);
  return launch_encode_dk<D, 0>(p, w, st);
}

}  // namespace tq
