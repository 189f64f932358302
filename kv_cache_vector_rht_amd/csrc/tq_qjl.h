// QJL projection of a key residual: sigma_j = [ (S r)_j >= 0 ], j < D.
// "TurboQuantとは？仕組み・実測精度・2026年7月時点の実装状況", section 第2段:
// the 1-bit sign of a Johnson-Lindenstrauss random projection of the
// residual. S is fp16 [D][D], row j = projection direction j.
#pragma once

#include "tq_device.h"

namespace tq {

// Per-lane fp32 dot products, S rows read with wave-uniform addresses.
// r: the lane's residual (registers); sig: D/32 words, bit j%32 of word j/32.
template <int D>
__device__ __forceinline__ void qjl_signs(const uint16_t *__restrict__ sketch, const float (&r)[D],
                                          uint32_t (&sig)[D / 32]) {
#pragma unroll
  for (int jw = 0; jw < D / 32; ++jw) {
    uint32_t word = 0u;
    for (int jb = 0; jb < 32; ++jb) {
      const int j = jw * 32 + jb;
      const uint32_t *row = reinterpret_cast<const uint32_t *>(sketch + static_cast<int64_t>(j) * D);
      float z = 0.f;
#pragma unroll
      for (int k = 0; k < D; k += 2) {
        const uint32_t two = row[k / 2];
        z = fmaf(f16_bits_to_float(static_cast<uint16_t>(two & 0xffffu)), r[k], z);
        z = fmaf(f16_bits_to_float(static_cast<uint16_t>(two >> 16)), r[k + 1], z);
      }
      word |= static_cast<uint32_t>(z >= 0.f) << jb;
    }
    sig[jw] = word;
  }
}

}  // namespace tq
