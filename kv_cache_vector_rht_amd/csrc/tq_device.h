// Device-side helpers shared by the libtq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

constexpr int kWave = 64;
constexpr int kValueBlock = 32;   // tokens per value-code block

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ float f16_bits_to_float(uint16_t b) {
  _Float16 h = __builtin_bit_cast(_Float16, b);
  return static_cast<float>(h);
}

// IEEE round-to-nearest-even float -> fp16 (v_cvt_f16_f32 in the default mode).
__device__ __forceinline__ uint16_t float_to_f16_bits(float f) {
  _Float16 h = static_cast<_Float16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

// Round-to-nearest-even float -> bf16; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Element loads from the three input dtypes.
struct LoadF32 {
  using T = float;
  static __device__ __forceinline__ float get(const float *p, int64_t i) { return p[i]; }
};
struct LoadBF16 {
  using T = uint16_t;
  static __device__ __forceinline__ float get(const uint16_t *p, int64_t i) {
    return bf16_bits_to_float(p[i]);
  }
};
struct LoadF16 {
  using T = uint16_t;
  static __device__ __forceinline__ float get(const uint16_t *p, int64_t i) {
    return f16_bits_to_float(p[i]);
  }
};

// Load D consecutive elements of one row into registers as float.
template <int D, typename L>
__device__ __forceinline__ void load_row(const typename L::T *row, float (&v)[D]);

template <int D>
__device__ __forceinline__ void load_row_vec_f32(const float *row, float (&v)[D]) {
#pragma unroll
  for (int i = 0; i < D; i += 4) {
    float4 q = *reinterpret_cast<const float4 *>(row + i);
    v[i] = q.x; v[i + 1] = q.y; v[i + 2] = q.z; v[i + 3] = q.w;
  }
}

template <int D, bool BF16>
__device__ __forceinline__ void load_row_vec_16(const uint16_t *row, float (&v)[D]) {
#pragma unroll
  for (int i = 0; i < D; i += 8) {
    uint4 q = *reinterpret_cast<const uint4 *>(row + i);
    uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint16_t lo = static_cast<uint16_t>(w[k] & 0xffffu);
      uint16_t hi = static_cast<uint16_t>(w[k] >> 16);
      if (BF16) {
        v[i + 2 * k] = bf16_bits_to_float(lo);
        v[i + 2 * k + 1] = bf16_bits_to_float(hi);
      } else {
        v[i + 2 * k] = f16_bits_to_float(lo);
        v[i + 2 * k + 1] = f16_bits_to_float(hi);
      }
    }
  }
}

// ------------------------------------------------------------------ transform

// Unnormalised Walsh-Hadamard transform of a register-resident vector in
// natural (Sylvester) order: after the call v = H v, H[i][j] = (-1)^popcount(i&j).
template <int D>
__device__ __forceinline__ void fwht_regs(float (&v)[D]) {
#pragma unroll
  for (int h = 1; h < D; h <<= 1) {
#pragma unroll
    for (int i = 0; i < D; i += 2 * h) {
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        float a = v[j];
        float b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
    }
  }
}

// ------------------------------------------------------------------ reductions

// Lane exchange inside rows of 16 lanes with DPP (no LDS round trip).
// quad_perm [1,0,3,2] and [2,3,0,1], then rotations of the row by 4 and 8:
// after the four steps every lane holds the reduction over its row.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __uint_as_float(dpp_u<CTRL>(__float_as_uint(v)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint64_t r = static_cast<uint64_t>(dpp_u<CTRL>(static_cast<uint32_t>(u))) |
                     (static_cast<uint64_t>(dpp_u<CTRL>(static_cast<uint32_t>(u >> 32))) << 32);
  return __builtin_bit_cast(double, r);
}

__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x124>(v));
  return fmaxf(v, dpp_f<0x128>(v));
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x124>(v);
  return v + dpp_f<0x128>(v);
}
__device__ __forceinline__ double row_sum16d(double v) {
  v += dpp_d<0xB1>(v);
  v += dpp_d<0x4E>(v);
  v += dpp_d<0x124>(v);
  return v + dpp_d<0x128>(v);
}

// Whole-wave reductions: rows by DPP, then the four row results.
__device__ __forceinline__ float wave_max(float v) {
  v = row_max16(v);
  const float a = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 0));
  const float b = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 16));
  const float c = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 32));
  const float d = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
  const float a = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 0));
  const float b = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 16));
  const float c = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 32));
  const float d = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 48));
  return (a + b) + (c + d);
}

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & (kWave - 1); }

// The other half-wave's copy of x (lane l <-> lane l ^ 32).
__device__ __forceinline__ float swap_half_f(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float((lane_id() < 32) ? r[1] : r[0]);
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int I>
struct IntC {
  static constexpr int value = I;
};
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (B < E) {
    f(IntC<B>{});
    static_for<B + 1, E>(f);
  }
}

}  // namespace tq
