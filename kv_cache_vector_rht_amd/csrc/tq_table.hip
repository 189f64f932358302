// The logit scan with the codebook in LDS: per-head nibble tables over the
// key bit planes (the formulation that keeps the codebook in LDS for the
// logits, kept beside the matrix-core scan of tq_decode.inc.h to measure
// the two against each other).
//
// Estimator as the logit scan ("TurboQuantとは？仕組み・実測精度・2026年7月
// 時点の実装状況", 第2段):
//   logit = n ( sum_i q'_i c[idx_i] + sqrt(pi/2)/D gamma sum_j p_j (2 sigma_j - 1) ),
// with both sums over bit planes (tq_mfma.h): sum_i q'_i c[idx_i] =
// sum_S 2 beta_S <q', x_S> - c[L-1] sum_i q'_i over the odd subsets S of the
// index bits, and sum_j p_j (2 sigma_j - 1) = 2 <p, sigma> - sum_j p_j.
// A plane's inner product is a sum of table entries: for every 4 coordinates
// (a nibble of the plane) a 16-entry table holds the sums of the matching
// coefficients (2 beta_S q' or 2 p) over the nibble's set bits.
//
// Two kernels: the preparation (q' = R q and p = S q' per head, fp32, into
// the workspace) and the scan (one lane per key; the tables of a chunk of 4
// heads built in LDS by every block).
#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_kernels.h"
#include "tq_mfma.h"

namespace tq {

namespace {

constexpr int kTabHeads = 4;          // heads per table block
constexpr int kTabThreads = 256;
constexpr float kTabSqrtHalfPi = 1.2533141373155002f;

// q' (rotation) and p = S q' of the heads [4 z, 4 z + 4) of group blockIdx.x,
// one wave per head: qp [groups][chunks][4 heads][2][D] fp32 (zeros for heads
// past the group).
template <int D>
__global__ __launch_bounds__(kTabThreads) void table_prep_kernel(ScanParams p, float *qp) {
  constexpr int E = D / kWave;
  __shared__ float sq[kTabHeads][D];
  const int64_t bh = blockIdx.x;
  const int64_t b = bh / p.n_kv, kvh = bh % p.n_kv;
  const int h = threadIdx.x / kWave, lane = lane_id();
  const int head = kTabHeads * static_cast<int>(blockIdx.y) + h;
  const bool live = head < p.group;
  float x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = E * lane + e;
    float v = 0.f;
    if (live) {
      const int64_t idx = ((b * p.n_kv + kvh) * p.group + head) * D + i;
      v = (p.xt == 0) ? static_cast<const float *>(p.q)[idx]
          : (p.xt == 1) ? bf16_bits_to_float(static_cast<const uint16_t *>(p.q)[idx])
                        : f16_bits_to_float(static_cast<const uint16_t *>(p.q)[idx]);
    }
    x[e] = v * p.ksigns[i];
  }
  if constexpr (E == 2) {
    const float a0 = x[0] + x[1], a1 = x[0] - x[1];
    x[0] = a0;
    x[1] = a1;
  }
  // (the butterflies over the lanes: index bit 0 in registers for D = 128)
  auto fwht = [lane](float v) {
    auto bfly = [lane](float own, float other, int bit) { return ((lane >> bit) & 1) ? other - own : own + other; };
    v = bfly(v, __shfl_xor(v, 1), 0);
    v = bfly(v, __shfl_xor(v, 2), 1);
    v = bfly(v, __shfl_xor(v, 4), 2);
    v = bfly(v, __shfl_xor(v, 8), 3);
    v = bfly(v, __shfl_xor(v, 16), 4);
    return bfly(v, __shfl_xor(v, 32), 5);
  };
#pragma unroll
  for (int e = 0; e < E; ++e) sq[h][E * lane + e] = fwht(x[e]) * (1.0f / sqrtf(static_cast<float>(D)));
  __syncthreads();
  float *dst = qp + (bh * gridDim.y + blockIdx.y) * kTabHeads * 2 * D;
  for (int o = threadIdx.x; o < kTabHeads * D; o += kTabThreads) {
    const int hh = o / D, j = o % D;
    float acc = 0.f;
    for (int k = 0; k < D; ++k) acc = fmaf(f16_bits_to_float(p.sketch[j * D + k]), sq[hh][k], acc);
    dst[(hh * 2) * D + j] = sq[hh][j];
    dst[(hh * 2 + 1) * D + j] = acc;
  }
}

// The scan: block (bx, group, chunk) takes the 256-key runs bx, bx + nb, ...
template <int D, int KW>
__global__ __launch_bounds__(kTabThreads) void table_scan_kernel(ScanParams p, const float *qp) {
  constexpr int NB = Basis<KW>::N;
  constexpr int NS = NB + 1;                      // basis planes + the sign plane
  constexpr int NG = D / 4;                       // nibbles per plane
  constexpr int NW32 = D / 32;                    // words per plane
  constexpr int L = 1 << KW;
  constexpr int REC = (KW + 1) * D / 8;
  __shared__ float tab[kTabHeads][NS][NG][16];
  __shared__ float cst[kTabHeads][2];
  __shared__ float beta[NB];
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / p.n_kv, kvh = bh % p.n_kv;
  const int h0 = kTabHeads * static_cast<int>(blockIdx.z);
  const int GE = min(kTabHeads, p.group - h0);
  const float *src = qp + (bh * gridDim.z + blockIdx.z) * kTabHeads * 2 * D;
  const int tid = threadIdx.x;
  if (tid < NB) beta[tid] = basis_coeff(p.kcent, KW, basis_mask(KW, tid));
  if (tid < kTabHeads * 2) {
    const int hh = tid / 2, which = tid % 2;       // 0: c[L-1] sum q', 1: sum p
    float s = 0.f;
    for (int i = 0; i < D; ++i) s += src[(hh * 2 + which) * D + i];
    cst[hh][which] = which ? s : p.kcent[L - 1] * s;
  }
  __syncthreads();
  for (int e = tid; e < kTabHeads * NS * NG * 16; e += kTabThreads) {
    const int n = e % 16, g = (e / 16) % NG, s = (e / (16 * NG)) % NS, hh = e / (16 * NG * NS);
    const float *v = src + (hh * 2 + (s == NB ? 1 : 0)) * D + 4 * g;
    const float coef = (s == NB) ? 2.0f : 2.0f * beta[s];
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) acc += ((n >> k) & 1) ? v[k] : 0.f;
    tab[hh][s][g][n] = coef * acc;
  }
  __syncthreads();

  const int n_keys = static_cast<int>(p.max_ctx);
  const int n_q = p.n_kv * p.group;
  const float kappa = kTabSqrtHalfPi / static_cast<float>(D);
  const uint8_t *codes = p.kcodes + bh * p.cap * REC;
  const uint32_t *scal = reinterpret_cast<const uint32_t *>(p.kscalars) + bh * p.cap;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kTabThreads; base < n_keys;
       base += static_cast<int64_t>(gridDim.x) * kTabThreads) {
    const int64_t t = base + tid;
    if (t >= n_keys) break;
    // the record's words (plane p, word wd at record word p NW32 + wd),
    // by 16-byte loads where the record size allows (d = 128), else 8-byte
    uint32_t w[KW + 1][NW32];
    if constexpr (REC % 16 == 0) {
      const uint4 *rec = reinterpret_cast<const uint4 *>(codes + t * REC);
#pragma unroll
      for (int u = 0; u < REC / 16; ++u) {
        const uint4 v = rec[u];
        const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) w[(4 * u + k) / NW32][(4 * u + k) % NW32] = vv[k];
      }
    } else {
      const uint2 *rec = reinterpret_cast<const uint2 *>(codes + t * REC);
#pragma unroll
      for (int u = 0; u < REC / 8; ++u) {
        const uint2 v = rec[u];
        w[(2 * u) / NW32][(2 * u) % NW32] = v.x;
        w[(2 * u + 1) / NW32][(2 * u + 1) % NW32] = v.y;
      }
    }
    const uint32_t sc = scal[t];
    float lm[kTabHeads], qj[kTabHeads];
#pragma unroll
    for (int hh = 0; hh < kTabHeads; ++hh) { lm[hh] = 0.f; qj[hh] = 0.f; }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int wd = 0; wd < NW32; ++wd) {
        uint32_t x = 0u;
        if (s == NB) {
          x = w[KW][wd];
        } else {
#pragma unroll
          for (int q = 0; q < KW; ++q)
            if ((Basis<KW>::M[s] >> q) & 1) x ^= w[q][wd];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int nib = (x >> (4 * j)) & 0xf;
          const int g = 8 * wd + j;
#pragma unroll
          for (int hh = 0; hh < kTabHeads; ++hh) {
            const float v = tab[hh][s][g][nib];
            if (s == NB) qj[hh] += v;
            else lm[hh] += v;
          }
        }
        // one plane word's lookups in flight at a time (else all of a key's
        // reads are hoisted, their sums sunk, and the registers spill)
#pragma unroll
        for (int hh = 0; hh < kTabHeads; ++hh) asm volatile("" : "+v"(lm[hh]), "+v"(qj[hh]));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const float n = f16_bits_to_float(static_cast<uint16_t>(sc & 0xffffu));
    const float gm = f16_bits_to_float(static_cast<uint16_t>(sc >> 16));
#pragma unroll
    for (int hh = 0; hh < kTabHeads; ++hh) {
      if (hh < GE) {
        const float l = n * fmaf(kappa * gm, qj[hh] - cst[hh][1], lm[hh] - cst[hh][0]);
        p.logits[(b * n_q + kvh * p.group + h0 + hh) * p.max_ctx + t] = l;
      }
    }
  }
}

template <int D>
hipError_t launch_table_d(const ScanParams &p, int kw, float *qp, hipStream_t st) {
  const uint32_t groups = static_cast<uint32_t>(p.batch) * p.n_kv;
  const uint32_t chunks = static_cast<uint32_t>((p.group + kTabHeads - 1) / kTabHeads);
  hipLaunchKernelGGL((table_prep_kernel<D>), dim3(groups, chunks), dim3(kTabThreads), 0, st, p, qp);
  // one block per run of 256 keys (each builds its tables: a few percent of
  // its scan), so that every CU holds several blocks
  const int64_t runs = (p.max_ctx + kTabThreads - 1) / kTabThreads;
  const dim3 grid(static_cast<uint32_t>(runs < 65535 ? runs : 65535), groups, chunks);
  switch (kw) {
    case 1: hipLaunchKernelGGL((table_scan_kernel<D, 1>), grid, dim3(kTabThreads), 0, st, p, qp); break;
    case 2: hipLaunchKernelGGL((table_scan_kernel<D, 2>), grid, dim3(kTabThreads), 0, st, p, qp); break;
    case 3: hipLaunchKernelGGL((table_scan_kernel<D, 3>), grid, dim3(kTabThreads), 0, st, p, qp); break;
    default: hipLaunchKernelGGL((table_scan_kernel<D, 4>), grid, dim3(kTabThreads), 0, st, p, qp);
  }
  return hipGetLastError();
}

}  // namespace

// q' and p of every head chunk: bytes of the table scan's workspace.
size_t table_workspace_bytes(int32_t batch, int32_t n_kv, int32_t group, int32_t d) {
  return static_cast<size_t>(batch) * n_kv * ((group + kTabHeads - 1) / kTabHeads) * kTabHeads * 2 * d *
         sizeof(float);
}

hipError_t launch_logits_table(const ScanParams &p, int d, int kw, float *qp, hipStream_t st) {
  if (p.batch == 0 || p.n_kv == 0 || p.max_ctx == 0) return hipSuccess;
  return d == 64 ? launch_table_d<64>(p, kw, qp, st) : launch_table_d<128>(p, kw, qp, st);
}

}  // namespace tq
