// fp8 key records for the k8v4 cache shape (fp8 keys, 4-bit TurboQuant
// values; "TurboQuantとは？仕組み・実測精度・2026年7月時点の実装状況", sections
// 「精度劣化ゼロ」の出所と、マージ後に判明した実測値 and the vLLM section list
// it as the most conservative preset): each key coordinate is stored as an
// OCP e4m3fn byte of x / scale, rounded to nearest even, finite values
// beyond +-448 saturating (NaN stays NaN). The decode kernels read these
// records with the key width kKeyFp8.
#include "tq_device.h"
#include "tq_kernels.h"

namespace tq {
namespace {

// One thread per 8 consecutive coordinates of a token: 8 loads, one 8-byte store.
__global__ __launch_bounds__(256) void encode_fp8_kernel(EncodeParams p, int d, float scale, int64_t n_units) {
  const int per_tok = d / 8;
  for (int64_t u = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; u < n_units;
       u += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t tok = u / per_tok;
    const int c8 = static_cast<int>(u % per_tok);
    const int64_t s = tok / p.n_tok, t = tok % p.n_tok;
    const int64_t x0 = s * p.x_seq_stride + t * p.x_tok_stride + 8 * c8;
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v;
      if (p.xt == 0) v = static_cast<const float *>(p.x)[x0 + e];
      else if (p.xt == 1) v = bf16_bits_to_float(static_cast<const uint16_t *>(p.x)[x0 + e]);
      else v = f16_bits_to_float(static_cast<const uint16_t *>(p.x)[x0 + e]);
      v = __fdiv_rn(v, scale);
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

}  // namespace

hipError_t launch_encode_fp8(const EncodeParams &p, int d, float scale, hipStream_t st) {
  const int64_t n_units = p.n_waves * p.n_tok * (d / 8);    // n_waves carries n_seq here
  if (n_units == 0) return hipSuccess;
  int64_t blocks = (n_units + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(encode_fp8_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, st, p, d, scale, n_units);
  return hipGetLastError();
}

}  // namespace tq
