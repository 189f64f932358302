// fp8 key records for the k8v4 cache shape (fp8 keys, 4-bit TurboQuant
// values; "TurboQuantとは？仕組み・実測精度・2026年7月時点の実装状況", sections
// 「精度劣化ゼロ」の出所と、マージ後に判明した実測値 and the vLLM section list
// it as the most conservative preset): each key coordinate is stored as an
// OCP e4m3fn byte of x / scale, rounded to nearest even, finite values
// beyond +-448 saturating (NaN stays NaN). The decode kernels read these
// records with the key width kKeyFp8.
#include <cfloat>
#include <cmath>

#include "tq_device.h"
#include "tq_kernels.h"

namespace tq {
namespace {

// The 8 coordinates of one unit as floats. VEC: the unit's elements are
// 16-byte aligned (one 16-byte load for 16-bit inputs, two for fp32).
template <int XT, bool VEC>
__device__ __forceinline__ void load8(const void *x, int64_t x0, float (&y)[8]) {
  if constexpr (VEC) {
    if constexpr (XT == 0) {
      const float4 a = *reinterpret_cast<const float4 *>(static_cast<const float *>(x) + x0);
      const float4 b = *reinterpret_cast<const float4 *>(static_cast<const float *>(x) + x0 + 4);
      y[0] = a.x; y[1] = a.y; y[2] = a.z; y[3] = a.w;
      y[4] = b.x; y[5] = b.y; y[6] = b.z; y[7] = b.w;
    } else {
      const uint4 a = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + x0);
      const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint16_t lo = static_cast<uint16_t>(w[e] & 0xffffu), hi = static_cast<uint16_t>(w[e] >> 16);
        y[2 * e] = XT == 1 ? bf16_bits_to_float(lo) : f16_bits_to_float(lo);
        y[2 * e + 1] = XT == 1 ? bf16_bits_to_float(hi) : f16_bits_to_float(hi);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (XT == 0) y[e] = static_cast<const float *>(x)[x0 + e];
      else if constexpr (XT == 1) y[e] = bf16_bits_to_float(static_cast<const uint16_t *>(x)[x0 + e]);
      else y[e] = f16_bits_to_float(static_cast<const uint16_t *>(x)[x0 + e]);
    }
  }
}

// One thread per 8 consecutive coordinates of a token, one 8-byte store.
// POW2: scale is a power of two, so x / scale = x * (1 / scale) exactly
// (both are the exact quotient rounded once).
template <int XT, bool VEC, bool POW2>
__global__ __launch_bounds__(256) void encode_fp8_kernel(EncodeParams p, int d, float scale, int64_t n_units) {
  const int per_tok = d / 8;
  const float inv = 1.0f / scale;
  for (int64_t u = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; u < n_units;
       u += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t tok = u / per_tok;
    const int c8 = static_cast<int>(u % per_tok);
    const int64_t s = tok / p.n_tok, t = tok % p.n_tok;
    const int64_t x0 = s * p.x_seq_stride + t * p.x_tok_stride + 8 * c8;
    float y[8];
    load8<XT, VEC>(p.x, x0, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = POW2 ? y[e] * inv : __fdiv_rn(y[e], scale);
      y[e] = (fabsf(v) > 448.0f) ? copysignf(448.0f, v) : v;
    }
    int w0 = 0, w1 = 0;
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], w0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], w1, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
    uint8_t *dst = static_cast<uint8_t *>(p.codes) + ((s * p.cap + p.t0 + t) * d + 8 * c8);
    *reinterpret_cast<uint2 *>(dst) = make_uint2(static_cast<uint32_t>(w0), static_cast<uint32_t>(w1));
  }
}

template <int XT, bool VEC>
void launch_fp8_x(const EncodeParams &p, int d, float scale, int64_t n_units, dim3 grid, hipStream_t st) {
  int ex = 0;
  const bool pow2 = std::frexp(scale, &ex) == 0.5f && scale >= FLT_MIN;   // (1 / scale finite)
  if (pow2) hipLaunchKernelGGL((encode_fp8_kernel<XT, VEC, true>), grid, dim3(256), 0, st, p, d, scale, n_units);
  else hipLaunchKernelGGL((encode_fp8_kernel<XT, VEC, false>), grid, dim3(256), 0, st, p, d, scale, n_units);
}

template <int XT>
void launch_fp8_t(const EncodeParams &p, int d, float scale, int64_t n_units, dim3 grid, hipStream_t st) {
  // every unit starts 8 elements into a row: 16-byte aligned when the base
  // and both strides are (in bytes)
  const int64_t esz = XT == 0 ? 4 : 2;
  const bool vec = reinterpret_cast<uintptr_t>(p.x) % 16 == 0 && (p.x_seq_stride * esz) % 16 == 0 &&
                   (p.x_tok_stride * esz) % 16 == 0;
  if (vec) launch_fp8_x<XT, true>(p, d, scale, n_units, grid, st);
  else launch_fp8_x<XT, false>(p, d, scale, n_units, grid, st);
}

}  // namespace

hipError_t launch_encode_fp8(const EncodeParams &p, int d, float scale, hipStream_t st) {
  const int64_t n_units = p.n_waves * p.n_tok * (d / 8);    // n_waves carries n_seq here
  if (n_units == 0) return hipSuccess;
  int64_t blocks = (n_units + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const dim3 grid(static_cast<uint32_t>(blocks));
  if (p.xt == 0) launch_fp8_t<0>(p, d, scale, n_units, grid, st);
  else if (p.xt == 1) launch_fp8_t<1>(p, d, scale, n_units, grid, st);
  else launch_fp8_t<2>(p, d, scale, n_units, grid, st);
  return hipGetLastError();
}

}  // namespace tq
