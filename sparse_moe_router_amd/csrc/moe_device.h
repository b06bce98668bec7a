// Device helpers shared by the HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// float -> bfloat16 bits, round to nearest even (v_cvt_pk_bf16_f32; NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// fp32 dot of two packed bf16 pairs plus an accumulator (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ---- cross-lane reductions without LDS: DPP within rows of 16 lanes, then
// v_permlane16_swap / v_permlane32_swap across rows.  Every lane of a segment
// ends with the same (bitwise identical) result.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16
constexpr int kDppRor8 = 0x128;       // lane i <- lane (i + 8) mod 16 within 16

// {own value, value of the lane 16 (or 32) apart}, in some order
__device__ __forceinline__ void swap16(uint32_t v, uint32_t* a, uint32_t* b) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  *a = r[0]; *b = r[1];
}
__device__ __forceinline__ void swap32(uint32_t v, uint32_t* a, uint32_t* b) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  *a = r[0]; *b = r[1];
}

// Sum over aligned segments of `width` lanes (a power of two <= 64).
__device__ __forceinline__ float seg_sum(float v, int width) {
  if (width >= 2) v += dpp_f<kDppXor1>(v);
  if (width >= 4) v += dpp_f<kDppXor2>(v);
  if (width >= 8) v += dpp_f<kDppHalfMirror>(v);
  if (width >= 16) v += dpp_f<kDppMirror>(v);
  if (width >= 32) {
    uint32_t a, b;
    swap16(__float_as_uint(v), &a, &b);
    v = __uint_as_float(a) + __uint_as_float(b);
  }
  if (width >= 64) {
    uint32_t a, b;
    swap32(__float_as_uint(v), &a, &b);
    v = __uint_as_float(a) + __uint_as_float(b);
  }
  return v;
}

__device__ __forceinline__ float wave_sum(float v) { return seg_sum(v, 64); }

// Wave-wide maximum / minimum of 32-bit integers (every lane gets it).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u<kDppXor1>(v));
  v = max(v, dpp_u<kDppXor2>(v));
  v = max(v, dpp_u<kDppHalfMirror>(v));
  v = max(v, dpp_u<kDppMirror>(v));
  uint32_t a, b;
  swap16(v, &a, &b);
  v = max(a, b);
  swap32(v, &a, &b);
  return max(a, b);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u<kDppXor1>(v));
  v = min(v, dpp_u<kDppXor2>(v));
  v = min(v, dpp_u<kDppHalfMirror>(v));
  v = min(v, dpp_u<kDppMirror>(v));
  uint32_t a, b;
  swap16(v, &a, &b);
  v = min(a, b);
  swap32(v, &a, &b);
  return min(a, b);
}

__device__ __forceinline__ int wave_min_i32(int v) {
  v = min(v, (int)dpp_u<kDppXor1>((uint32_t)v));
  v = min(v, (int)dpp_u<kDppXor2>((uint32_t)v));
  v = min(v, (int)dpp_u<kDppHalfMirror>((uint32_t)v));
  v = min(v, (int)dpp_u<kDppMirror>((uint32_t)v));
  uint32_t a, b;
  swap16((uint32_t)v, &a, &b);
  v = min((int)a, (int)b);
  swap32((uint32_t)v, &a, &b);
  return min((int)a, (int)b);
}

// Wave-wide maximum of a 64-bit key (every lane gets it).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  auto mx = [](uint64_t a, uint64_t b) { return a > b ? a : b; };
  auto join = [](uint32_t hi, uint32_t lo) { return ((uint64_t)hi << 32) | lo; };
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  v = mx(v, join(dpp_u<kDppXor1>(hi), dpp_u<kDppXor1>(lo)));
  lo = (uint32_t)v; hi = (uint32_t)(v >> 32);
  v = mx(v, join(dpp_u<kDppXor2>(hi), dpp_u<kDppXor2>(lo)));
  lo = (uint32_t)v; hi = (uint32_t)(v >> 32);
  v = mx(v, join(dpp_u<kDppHalfMirror>(hi), dpp_u<kDppHalfMirror>(lo)));
  lo = (uint32_t)v; hi = (uint32_t)(v >> 32);
  v = mx(v, join(dpp_u<kDppMirror>(hi), dpp_u<kDppMirror>(lo)));
  uint32_t l0, l1, h0, h1;
  lo = (uint32_t)v; hi = (uint32_t)(v >> 32);
  swap16(lo, &l0, &l1); swap16(hi, &h0, &h1);
  v = mx(join(h0, l0), join(h1, l1));
  lo = (uint32_t)v; hi = (uint32_t)(v >> 32);
  swap32(lo, &l0, &l1); swap32(hi, &h0, &h1);
  return mx(join(h0, l0), join(h1, l1));
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
