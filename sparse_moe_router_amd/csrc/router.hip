// Router logits and top-K selection (page 2 "Layer 1: On-Demand MoE Expert
// Scheduling": a light gating network picks the top-K experts of each token;
// page 3 "The 'Doorbell' Mechanism": the device decides each token's expert ids).
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// logits[t][e] = sum_i W[e][i] x[t][i] + b[e].  One wave per router row e, the
// row streamed as float4 per lane (64 lanes x 16 B = 1 KiB per instruction),
// NT tokens per pass so the row is read from HBM once and re-read from cache
// for later token chunks.
template <int ACT, int NT>
__global__ __launch_bounds__(256) void k_router_logits(RouterArgs a) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= a.E) return;
  const int nf = a.H >> 2;
  typedef float f4v __attribute__((ext_vector_type(4)));
  const f4v* wrow = reinterpret_cast<const f4v*>(a.w + (size_t)e * a.H);
  const float bias = a.b ? a.b[e] : 0.0f;
  for (int t0 = blockIdx.y * NT; t0 < a.T; t0 += gridDim.y * NT) {
    float acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = 0.0f;
    for (int f = lane; f < nf; f += 64) {
      const f4v w = __builtin_nontemporal_load(wrow + f);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        if (t0 + j < a.T) {
          float4 xv;
          const size_t base = (size_t)(t0 + j) * a.H + 4 * (size_t)f;
          if constexpr (ACT == 1) {
            const uint2 b2 = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(a.x) + base);
            xv.x = bf16_to_f32(b2.x & 0xffffu);
            xv.y = bf16_to_f32(b2.x >> 16);
            xv.z = bf16_to_f32(b2.y & 0xffffu);
            xv.w = bf16_to_f32(b2.y >> 16);
          } else {
            xv = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.x) + base);
          }
          acc[j] = fmaf(w.x, xv.x, acc[j]);
          acc[j] = fmaf(w.y, xv.y, acc[j]);
          acc[j] = fmaf(w.z, xv.z, acc[j]);
          acc[j] = fmaf(w.w, xv.w, acc[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const float v = seg_sum(acc[j], 64);
      if (lane == 0 && t0 + j < a.T) a.logits[(size_t)(t0 + j) * a.E + e] = v + bias;
    }
  }
}

// Order-preserving map of a float to uint32 (NaN treated as -inf); every real
// value maps to >= 0x007fffff, so 0 can mark "already taken".
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f != f) f = -INFINITY;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
    const uint64_t w = ((uint64_t)hi << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}

// One wave per token: K rounds of wave arg-max over the token's E logits held
// in LDS (largest logit, equal logits -> lower expert id), then the softmax of
// the K selected logits relative to the largest.
__global__ __launch_bounds__(64) void k_topk(RouterArgs a) {
  extern __shared__ uint32_t lds[];
  uint32_t* keys = lds;                          // [E]
  int32_t* chosen = reinterpret_cast<int32_t*>(lds + a.E);  // [K]
  const int t = blockIdx.x, lane = threadIdx.x;
  const float* lg = a.logits + (size_t)t * a.E;
  for (int e = lane; e < a.E; e += 64) keys[e] = order_key(lg[e]);
  __syncthreads();
  for (int k = 0; k < a.K; ++k) {
    uint64_t best = 0;
    for (int e = lane; e < a.E; e += 64) {
      const uint64_t c = ((uint64_t)keys[e] << 32) | (uint32_t)(0xffffffffu - (uint32_t)e);
      best = c > best ? c : best;
    }
    best = wave_max_u64(best);
    const int id = (int)(0xffffffffu - (uint32_t)best);
    if ((id & 63) == lane) keys[id] = 0u;  // the owning lane is the only reader of keys[id]
    if (lane == 0) chosen[k] = id;
  }
  __syncthreads();
  const float l0 = lg[chosen[0]];
  float part = 0.0f;
  for (int k = lane; k < a.K; k += 64) part += expf(lg[chosen[k]] - l0);
  const float total = seg_sum(part, 64);
  for (int k = lane; k < a.K; k += 64) {
    const int id = chosen[k];
    a.ids[(size_t)t * a.K + k] = id;
    a.wts[(size_t)t * a.K + k] = expf(lg[id] - l0) / total;
  }
}

hipError_t launch_router_logits(const RouterArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const dim3 block(256);
  if (a.T == 1) {
    const dim3 grid((a.E + 3) / 4, 1);
    if (a.act == MOE_ACT_BF16) k_router_logits<1, 1><<<grid, block, 0, s>>>(a);
    else k_router_logits<0, 1><<<grid, block, 0, s>>>(a);
  } else {
    const int chunks = (a.T + 3) / 4;
    const dim3 grid((a.E + 3) / 4, chunks < 64 ? chunks : 64);
    if (a.act == MOE_ACT_BF16) k_router_logits<1, 4><<<grid, block, 0, s>>>(a);
    else k_router_logits<0, 4><<<grid, block, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const RouterArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const size_t lds = (size_t)(a.E + a.K) * 4;
  k_topk<<<dim3(a.T), dim3(64), lds, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
