// Row-wise top-k of a score matrix: the ranking step of inner-product search
// over a coded database. The pages name vector-search indexes as a target of
// the same codes and estimator, ranked by inner product ("メモリの壁を砕く圧縮
// 革命、TurboQuant始動", sections TurboQuantの全体像 and 仕組みをほどく); the
// scores come from the logit scan over the coded vectors.
//
// Select passes, then a sort:
//  1. one block per (row, 4096-column chunk): the chunk's k largest scores
//     by radix selection on order-preserving 32-bit keys, written to the
//     workspace in column order (at most k per chunk);
//  2. while a row has more than 4096 candidates, the same selection over
//     chunks of 4096 candidates (each pass shrinks them at least 4-fold);
//  3. one block per row: the k largest of the last <= 4096 candidates,
//     sorted (score descending, column ascending on ties) by a bitonic sort,
//     stored.
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
static_assert(kThreads == 256, "one thread per digit");

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

// Digit histogram in kCopies copies (copy = lane % kCopies), digit-major
// with an odd row pitch: lanes adding to one digit hit distinct banks, and a
// thread summing one digit's copies reads a bank pattern free of conflicts.
constexpr int kPitch = kCopies + 1;

struct SelectShared {
  int hist[256 * kPitch];
  int4 tot[64];              // per-digit totals, digits 4i .. 4i+3
  int sh[8];
};

// A key prefix T (the bits under M) that splits the block's items: every
// item whose masked key exceeds T is among the k largest, and so are the
// first `need` items whose masked key equals T. The digits are refined from
// the top until that bucket is taken whole or the key is exhausted. Every
// thread visits its items with each(f), f(key); k <= number of items.
template <class Each>
__device__ __forceinline__ void radix_select(Each each, int k, SelectShared &s, uint32_t &T, uint32_t &M, int &need) {
  const int lane = threadIdx.x & 63;
  uint32_t prefix = 0, mask = 0;
  need = k;
  for (int i = threadIdx.x; i < 256 * kPitch; i += kThreads) s.hist[i] = 0;
  __syncthreads();
  for (int shift = 24; shift >= 0; shift -= 8) {
    const int copy = lane % kCopies;
    each([&](uint32_t u) {
      if ((u & mask) == prefix) atomicAdd(&s.hist[((u >> shift) & 255u) * kPitch + copy], 1);
    });
    __syncthreads();
    {
      // one thread per digit: its total, and the copies cleared for the next
      // round (two barriers pass before any thread adds to them again)
      const int dg = threadIdx.x;             // kThreads == 256 digits
      int t = 0;
#pragma unroll
      for (int cp = 0; cp < kCopies; ++cp) {
        t += s.hist[dg * kPitch + cp];
        s.hist[dg * kPitch + cp] = 0;
      }
      reinterpret_cast<int *>(s.tot)[dg] = t;
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      // lane l: digits 255 - 4l .. 252 - 4l, from the top
      const int4 q = s.tot[63 - lane];
      const int c[4] = {q.w, q.z, q.y, q.x};
      const int sum = c[0] + c[1] + c[2] + c[3];
      const int incl = wave_incl_scan(sum, lane);
      const int excl = incl - sum;
      if (excl < need && need <= incl) {
        int acc = excl, j = 0;
#pragma unroll
        for (int jj = 0; jj < 3; ++jj)
          if (acc + c[j] < need) { acc += c[j]; ++j; }
        s.sh[4] = 255 - 4 * lane - j;
        s.sh[5] = need - acc;
        s.sh[6] = (need - acc == c[j]) ? 1 : 0;   // the whole bucket is taken
      }
    }
    __syncthreads();
    // (wave 0 writes sh[4..6] again only after two more barriers)
    prefix |= static_cast<uint32_t>(s.sh[4]) << shift;
    mask |= 255u << shift;
    need = s.sh[5];
    if (s.sh[6]) break;
  }
  T = prefix;
  M = mask;
}

// Emit the k largest items in column order: every item whose masked key is
// above T and the first `need` items whose masked key equals T. each(f) visits f(key, column) in column
// order within the thread (threads hold consecutive column ranges);
// emit(pos, key, column) with pos in [0, k).
template <class Each, class Emit>
__device__ __forceinline__ void compact(Each each, uint32_t T, uint32_t M, int need, SelectShared &s, Emit emit) {
  int gt = 0, eq = 0;
  each([&](uint32_t u, uint32_t) {
    gt += ((u & M) > T) ? 1 : 0;
    eq += ((u & M) == T) ? 1 : 0;
  });
  const int eq_before = block_incl_scan(eq, s.sh) - eq;
  const int take = min(max(need - eq_before, 0), eq);
  const int sel = gt + take;
  int pos = block_incl_scan(sel, s.sh) - sel;
  int seen = 0;
  each([&](uint32_t u, uint32_t col) {
    bool keep = (u & M) > T;
    if ((u & M) == T) keep = (seen++ < take);
    if (keep) emit(pos++, u, col);
  });
}

// One block per (row, chunk of kTopkChunk items): the chunk's min(k, len)
// largest items, written in column order at out + row * out_stride +
// chunk * k. FROM_SCORES: the items are the row's scores (column = position);
// else (key, column) pairs from an earlier pass, in column order.
template <bool FROM_SCORES>
__global__ __launch_bounds__(kThreads) void topk_select_kernel(const void *__restrict__ in, int64_t in_stride,
                                                               int64_t m, int k, int64_t row0,
                                                               uint64_t *__restrict__ out, int64_t out_stride,
                                                               bool vec4) {
  __shared__ SelectShared s;
  const int64_t row = row0 + blockIdx.y;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kTopkChunk;
  const int len = static_cast<int>((m - c0 < kTopkChunk) ? m - c0 : kTopkChunk);
  const int lo = threadIdx.x * kPer;
  const int cnt = min(max(len - lo, 0), kPer);
  uint32_t u[kPer], col[kPer];
  if constexpr (FROM_SCORES) {
    const float *src = static_cast<const float *>(in) + row * in_stride + c0 + lo;
    if (vec4 && cnt == kPer) {
#pragma unroll
      for (int j = 0; j < kPer; j += 4) {
        const float4 v = *reinterpret_cast<const float4 *>(src + j);
        u[j] = order_key(v.x); u[j + 1] = order_key(v.y); u[j + 2] = order_key(v.z); u[j + 3] = order_key(v.w);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kPer; ++j) u[j] = (j < cnt) ? order_key(src[j]) : 0u;
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) col[j] = static_cast<uint32_t>(c0 + lo + j);
  } else {
    const uint64_t *src = static_cast<const uint64_t *>(in) + row * in_stride + c0 + lo;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint64_t v = (j < cnt) ? src[j] : 0ull;
      u[j] = static_cast<uint32_t>(v >> 32);
      col[j] = static_cast<uint32_t>(v);
    }
  }
  const int kc = min(k, len);
  uint32_t T, M;
  int need;
  radix_select([&](auto f) {
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (j < cnt) f(u[j]);
  }, kc, s, T, M, need);
  uint64_t *dst = out + row * out_stride + static_cast<int64_t>(blockIdx.x) * k;
  compact([&](auto f) {
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (j < cnt) f(u[j], col[j]);
  }, T, M, need, s, [&](int pos, uint32_t key, uint32_t c) {
    dst[pos] = (static_cast<uint64_t>(key) << 32) | c;
  });
}

// One block per row: the k largest of the row's last m <= kTopkChunk
// candidates (column order), sorted (key descending, column ascending) by a
// bitonic sort in LDS, stored with their original scores.
__global__ __launch_bounds__(kThreads) void topk_sort_kernel(const float *__restrict__ scores, int64_t ld,
                                                             const uint64_t *__restrict__ cand, int64_t cand_stride,
                                                             int m, int k, int64_t row0,
                                                             float *__restrict__ top_scores,
                                                             int32_t *__restrict__ top_idx) {
  __shared__ SelectShared s;
  __shared__ uint64_t srt[kTopkMaxK];
  const int64_t row = row0 + blockIdx.x;
  const uint64_t *c = cand + row * cand_stride;
  const int lo = threadIdx.x * kPer;
  const int cnt = min(max(m - lo, 0), kPer);
  uint32_t u[kPer], col[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const uint64_t v = (j < cnt) ? c[lo + j] : 0ull;
    u[j] = static_cast<uint32_t>(v >> 32);
    col[j] = static_cast<uint32_t>(v);
  }
  uint32_t T, M;
  int need;
  radix_select([&](auto f) {
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (j < cnt) f(u[j]);
  }, k, s, T, M, need);
  // winners -> (key, ~column) composites; padding 0 sorts below every winner
  int P = 1;
  while (P < k) P <<= 1;
  for (int i = threadIdx.x; i < P; i += kThreads) srt[i] = 0;
  __syncthreads();
  compact([&](auto f) {
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (j < cnt) f(u[j], col[j]);
  }, T, M, need, s, [&](int pos, uint32_t key, uint32_t cl) {
    srt[pos] = (static_cast<uint64_t>(key) << 32) | (0xffffffffu - cl);
  });
  __syncthreads();
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
    const uint32_t cl = 0xffffffffu - static_cast<uint32_t>(srt[r]);
    top_idx[row * k + r] = static_cast<int32_t>(cl);
    top_scores[row * k + r] = scores[row * ld + cl];
  }
}

int64_t chunks_of(int64_t m) { return (m + kTopkChunk - 1) / kTopkChunk; }

// Candidates left after a select pass over m items per row.
int64_t after_pass(int64_t m, int k) {
  const int64_t n = chunks_of(m);
  const int64_t last = m - (n - 1) * kTopkChunk;
  return (n - 1) * k + ((last < k) ? last : k);
}

}  // namespace

// The two candidate buffers (pairs per row): the first pass's output and the
// second's; later passes alternate between them and only shrink.
void topk_buffers(int64_t n_cols, int k, int64_t &stride_a, int64_t &stride_b) {
  stride_a = chunks_of(n_cols) * k;
  stride_b = chunks_of(stride_a) * k;
}

hipError_t launch_topk(const float *scores, int64_t n_rows, int64_t n_cols, int64_t ld, int k, float *top_scores,
                       int32_t *top_idx, uint64_t *cand, hipStream_t st) {
  int64_t sa, sb;
  topk_buffers(n_cols, k, sa, sb);
  uint64_t *bufs[2] = {cand, cand + n_rows * sa};
  const int64_t strides[2] = {sa, sb};
  const bool vec4 = (ld % 4 == 0) && (reinterpret_cast<uintptr_t>(scores) % 16 == 0);
  for (int64_t r0 = 0; r0 < n_rows; r0 += 65535) {
    const uint32_t nr = static_cast<uint32_t>((n_rows - r0 < 65535) ? n_rows - r0 : 65535);
    hipLaunchKernelGGL(topk_select_kernel<true>, dim3(static_cast<uint32_t>(chunks_of(n_cols)), nr), dim3(kThreads),
                       0, st, scores, ld, n_cols, k, r0, bufs[0], strides[0], vec4);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int64_t m = after_pass(n_cols, k);
    int cur = 0;
    while (m > kTopkChunk) {
      hipLaunchKernelGGL(topk_select_kernel<false>, dim3(static_cast<uint32_t>(chunks_of(m)), nr), dim3(kThreads),
                         0, st, bufs[cur], strides[cur], m, k, r0, bufs[cur ^ 1], strides[cur ^ 1], false);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      m = after_pass(m, k);
      cur ^= 1;
    }
    hipLaunchKernelGGL(topk_sort_kernel, dim3(nr), dim3(kThreads), 0, st, scores, ld, bufs[cur], strides[cur],
                       static_cast<int>(m), k, r0, top_scores, top_idx);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tq
