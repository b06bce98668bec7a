// Device helpers shared by the HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// float -> bfloat16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// fp32 dot of two packed bf16 pairs plus an accumulator (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Sum over aligned segments of `width` lanes (width a power of two <= 64).
__device__ __forceinline__ float seg_sum(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Store one activation value in the storage type (bf16 bits or fp32).
template <int ACT>
__device__ __forceinline__ void store_act(void* base, size_t idx, float v) {
  if constexpr (ACT == 1) {
    reinterpret_cast<uint16_t*>(base)[idx] = f32_to_bf16(v);
  } else {
    reinterpret_cast<float*>(base)[idx] = v;
  }
}

template <int ACT>
__device__ __forceinline__ float load_act(const void* base, size_t idx) {
  if constexpr (ACT == 1) {
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
  } else {
    return reinterpret_cast<const float*>(base)[idx];
  }
}

}  // namespace moe
