// Device-side scalar helpers shared by the HIP kernels of the Q1 library.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "q1_internal.h"

namespace q1 {

// ---------------------------------------------------------------------------
// Scalar conversions (device)
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)b);
  return (float)h;
}

template <bool BF16>
__device__ __forceinline__ float meta_to_f32(uint32_t b) {
  return BF16 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
}

// fp32 -> bf16, round to nearest even (NaN stays NaN, quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// fp32 -> fp16 with the hardware conversion (round to nearest even).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ void store_out(void* out, int32_t dtype, int64_t idx, float v) {
  if (dtype == F32) {
    static_cast<float*>(out)[idx] = v;
  } else if (dtype == BF16) {
    static_cast<uint16_t*>(out)[idx] = (uint16_t)f32_to_bf16_bits(v);
  } else {
    static_cast<uint16_t*>(out)[idx] = (uint16_t)f32_to_f16_bits(v);
  }
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }

// Add split-K partial sums [KS][M][units] for units [u0, u1) in the fixed
// order k = 0..KS-1 and write the output: y[m][u] (single mode) or
// h[m][r] = bf16(SiLU(g) * up) with g, up = units 2r, 2r+1 (pair mode).
template <int M>
__device__ __forceinline__ void splitk_finish(const float* partial, int KS, int64_t units, int pair, void* out,
                                              int32_t out_dtype, int64_t out_ld, int64_t u0, int64_t u1, int tid,
                                              int nthreads) {
  if (!pair) {
    const int64_t n = u1 - u0;
    for (int64_t idx = tid; idx < (int64_t)M * n; idx += nthreads) {
      const int m = (int)(idx / n);
      const int64_t u = u0 + (idx - (int64_t)m * n);
      float s = 0.f;
      for (int k = 0; k < KS; ++k) s += partial[((int64_t)k * M + m) * units + u];
      store_out(out, out_dtype, m * out_ld + u, s);
    }
  } else {
    const int64_t n = (u1 - u0) >> 1;
    for (int64_t idx = tid; idx < (int64_t)M * n; idx += nthreads) {
      const int m = (int)(idx / n);
      const int64_t r = (u0 >> 1) + (idx - (int64_t)m * n);
      float g = 0.f, up = 0.f;
      for (int k = 0; k < KS; ++k) {
        g += partial[((int64_t)k * M + m) * units + 2 * r];
        up += partial[((int64_t)k * M + m) * units + 2 * r + 1];
      }
      static_cast<uint16_t*>(out)[m * out_ld + r] = (uint16_t)f32_to_bf16_bits(silu_f32(g) * up);
    }
  }
}

}  // namespace q1
