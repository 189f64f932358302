// Row-wise top-k of a score matrix: the ranking step of inner-product search
// over a coded database. The pages name vector-search indexes as a target of
// the same codes and estimator, ranked by inner product ("メモリの壁を砕く圧縮
// 革命、TurboQuant始動", sections TurboQuantの全体像 and 仕組みをほどく); the
// scores come from the logit scan over the coded vectors.
//
// Two launches per call:
//  1. one block per (row, 4096-column chunk): the chunk's k largest scores
//     by radix selection on order-preserving 32-bit keys, written to the
//     workspace in column order (at most k per chunk);
//  2. one block per row: the same selection over the row's candidates, then
//     a bitonic sort of the k winners (score descending, column ascending on
//     ties) and the store.
// Ties at the k-th score go to the smaller column in both stages, so the
// result is the first k entries of the row in (score desc, column asc)
// order. A NaN score ranks above +Inf; -0.0 ranks as +0.0.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_kernels.h"

namespace tq {
namespace {

constexpr int kThreads = 256;
constexpr int kPer = kTopkChunk / kThreads;   // chunk columns per thread
constexpr int kCopies = 16;                   // histogram copies (lane % 16)

// Larger float -> larger key (sign-magnitude to offset binary).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(v, d);
    if (lane >= d) v += t;
  }
  return v;
}

// Inclusive prefix sum over the block (threads in order); sh: 4 ints.
__device__ __forceinline__ int block_incl_scan(int v, int *sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_incl_scan(v, lane);
  if (lane == 63) sh[w] = v;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) before += (i < w) ? sh[i] : 0;
  __syncthreads();
  return v + before;
}

struct SelectShared {
  int hist[256 * kCopies];   // [digit][copy]
  int sh[8];
};

// The k-th largest key T among the block's items and how many of the items
// equal to T belong to the k largest (need). Every thread visits its items
// with each(f), f(key); k <= number of items.
template <class Each>
__device__ __forceinline__ void radix_select(Each each, int k, SelectShared &s, uint32_t &T, int &need) {
  const int lane = threadIdx.x & 63;
  uint32_t prefix = 0, mask = 0;
  need = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256 * kCopies; i += kThreads) s.hist[i] = 0;
    __syncthreads();
    const int copy = lane % kCopies;
    each([&](uint32_t u) {
      if ((u & mask) == prefix) atomicAdd(&s.hist[((u >> shift) & 255u) * kCopies + copy], 1);
    });
    __syncthreads();
    if (threadIdx.x < 64) {
      // lane l: digits 255 - 4l .. 252 - 4l, from the top
      int c[4], sum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int dg = 255 - 4 * lane - j;
        int t = 0;
#pragma unroll
        for (int cp = 0; cp < kCopies; ++cp) t += s.hist[dg * kCopies + cp];
        c[j] = t;
        sum += t;
      }
      const int incl = wave_incl_scan(sum, lane);
      const int excl = incl - sum;
      if (excl < need && need <= incl) {
        int acc = excl, j = 0;
#pragma unroll
        for (int jj = 0; jj < 3; ++jj)
          if (acc + c[j] < need) { acc += c[j]; ++j; }
        s.sh[4] = 255 - 4 * lane - j;
        s.sh[5] = need - acc;
      }
    }
    __syncthreads();
    prefix |= static_cast<uint32_t>(s.sh[4]) << shift;
    mask |= 255u << shift;
    need = s.sh[5];
    __syncthreads();
  }
  T = prefix;
}

// Emit the k largest items in column order: every item above T and the
// first `need` items equal to T. each(f) visits f(key, column) in column
// order within the thread (threads hold consecutive column ranges);
// emit(pos, key, column) with pos in [0, k).
template <class Each, class Emit>
__device__ __forceinline__ void compact(Each each, uint32_t T, int need, SelectShared &s, Emit emit) {
  int gt = 0, eq = 0;
  each([&](uint32_t u, uint32_t) {
    gt += (u > T) ? 1 : 0;
    eq += (u == T) ? 1 : 0;
  });
  const int eq_before = block_incl_scan(eq, s.sh) - eq;
  const int take = min(max(need - eq_before, 0), eq);
  const int sel = gt + take;
  int pos = block_incl_scan(sel, s.sh) - sel;
  int seen = 0;
  each([&](uint32_t u, uint32_t col) {
    bool keep = u > T;
    if (u == T) keep = (seen++ < take);
    if (keep) emit(pos++, u, col);
  });
}

__global__ __launch_bounds__(kThreads) void topk_chunk_kernel(const float *__restrict__ scores, int64_t ld,
                                                              int64_t n_cols, int k, int64_t row0, int64_t n_chunks,
                                                              uint64_t *__restrict__ cand) {
  __shared__ SelectShared s;
  const int64_t row = row0 + blockIdx.y;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kTopkChunk;
  const int len = static_cast<int>((n_cols - c0 < kTopkChunk) ? n_cols - c0 : kTopkChunk);
  const float *src = scores + row * ld + c0;
  const int lo = threadIdx.x * kPer;
  const int cnt = min(max(len - lo, 0), kPer);
  uint32_t u[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) u[j] = (j < cnt) ? order_key(src[lo + j]) : 0u;
  const int kc = min(k, len);
  uint32_t T;
  int need;
  radix_select([&](auto f) {
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (j < cnt) f(u[j]);
  }, kc, s, T, need);
  uint64_t *out = cand + (row * n_chunks + blockIdx.x) * k;
  compact([&](auto f) {
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (j < cnt) f(u[j], static_cast<uint32_t>(c0 + lo + j));
  }, T, need, s, [&](int pos, uint32_t key, uint32_t col) {
    out[pos] = (static_cast<uint64_t>(key) << 32) | col;
  });
}

__global__ __launch_bounds__(kThreads) void topk_final_kernel(const float *__restrict__ scores, int64_t ld,
                                                              int64_t n_cols, int k, int64_t row0, int64_t n_chunks,
                                                              const uint64_t *__restrict__ cand,
                                                              float *__restrict__ top_scores,
                                                              int32_t *__restrict__ top_idx) {
  __shared__ SelectShared s;
  __shared__ uint64_t srt[kTopkMaxK];
  const int64_t row = row0 + blockIdx.x;
  const int64_t last = n_cols - (n_chunks - 1) * kTopkChunk;
  const int64_t m = (n_chunks - 1) * k + ((last < k) ? last : k);   // the row's candidates, in column order
  const uint64_t *c = cand + row * n_chunks * k;
  const int64_t per = (m + kThreads - 1) / kThreads;
  const int64_t lo = threadIdx.x * per;
  const int64_t hi = (lo + per < m) ? lo + per : m;
  uint32_t T;
  int need;
  radix_select([&](auto f) {
    for (int64_t i = lo; i < hi; ++i) f(static_cast<uint32_t>(c[i] >> 32));
  }, k, s, T, need);
  // winners -> (key, ~column) composites; padding 0 sorts below every winner
  int P = 1;
  while (P < k) P <<= 1;
  for (int i = threadIdx.x; i < P; i += kThreads) srt[i] = 0;
  __syncthreads();
  compact([&](auto f) {
    for (int64_t i = lo; i < hi; ++i) f(static_cast<uint32_t>(c[i] >> 32), static_cast<uint32_t>(c[i]));
  }, T, need, s, [&](int pos, uint32_t key, uint32_t col) {
    srt[pos] = (static_cast<uint64_t>(key) << 32) | (0xffffffffu - col);
  });
  __syncthreads();
  // bitonic sort, descending
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < P / 2; t += kThreads) {
        const int i = 2 * t - (t & (stride - 1));
        const int j = i + stride;
        const bool desc = (i & size) == 0;
        const uint64_t a = srt[i], b = srt[j];
        if ((a < b) == desc) { srt[i] = b; srt[j] = a; }
      }
      __syncthreads();
    }
  }
  for (int r = threadIdx.x; r < k; r += kThreads) {
    const uint32_t col = 0xffffffffu - static_cast<uint32_t>(srt[r]);
    top_idx[row * k + r] = static_cast<int32_t>(col);
    top_scores[row * k + r] = scores[row * ld + col];
  }
}

}  // namespace

hipError_t launch_topk(const float *scores, int64_t n_rows, int64_t n_cols, int64_t ld, int k, float *top_scores,
                       int32_t *top_idx, uint64_t *cand, hipStream_t st) {
  const int64_t n_chunks = (n_cols + kTopkChunk - 1) / kTopkChunk;
  for (int64_t r0 = 0; r0 < n_rows; r0 += 65535) {
    const int64_t nr = (n_rows - r0 < 65535) ? n_rows - r0 : 65535;
    hipLaunchKernelGGL(topk_chunk_kernel, dim3(static_cast<uint32_t>(n_chunks), static_cast<uint32_t>(nr)),
                       dim3(kThreads), 0, st, scores, ld, n_cols, k, r0, n_chunks, cand);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_final_kernel, dim3(static_cast<uint32_t>(nr)), dim3(kThreads), 0, st, scores, ld,
                       n_cols, k, r0, n_chunks, cand, top_scores, top_idx);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tq
