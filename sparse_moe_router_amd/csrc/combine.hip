// Weighted combine of the expert outputs (shared expert with weight 1, then
// the K routed experts with their renormalised router weights, in slot order;
// page 5 "The model is large on paper, sparse in practice": 10 routed + 1
// shared expert per token), and the dequantisation test hook.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// One thread per 4 consecutive outputs of one token; fixed summation order, so
// the result is bitwise reproducible.
constexpr int kSlotBatch = 12;  // slots whose loads are issued together

template <int ACT>
__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  const int h4 = a.H >> 2;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)a.T * h4) return;
  const int t = (int)(idx / h4), j4 = (int)(idx % h4);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k0 = 0; k0 < a.K; k0 += kSlotBatch) {
    int pos[kSlotBatch];
    float w[kSlotBatch];
    float4 o[kSlotBatch];
#pragma unroll
    for (int i = 0; i < kSlotBatch; ++i) {  // clamped slot: loads outside conditional blocks
      const size_t q = (size_t)t * a.K + min(k0 + i, a.K - 1);
      pos[i] = a.pair_pos[q];
      w[i] = a.w[q];
    }
#pragma unroll
    for (int i = 0; i < kSlotBatch; ++i) o[i] = reinterpret_cast<const float4*>(a.o)[(size_t)pos[i] * h4 + j4];
    if (k0 == 0 && a.so) acc = reinterpret_cast<const float4*>(a.so)[idx];  // the shared expert comes first
#pragma unroll
    for (int i = 0; i < kSlotBatch; ++i) {
      if (k0 + i < a.K) {
        acc.x = fmaf(w[i], o[i].x, acc.x);
        acc.y = fmaf(w[i], o[i].y, acc.y);
        acc.z = fmaf(w[i], o[i].z, acc.z);
        acc.w = fmaf(w[i], o[i].w, acc.w);
      }
    }
  }
  reinterpret_cast<float4*>(a.y)[idx] = acc;
  if (a.x_next) {
    const size_t e = idx * 4;
    store_act<ACT>(a.x_next, e + 0, load_act<ACT>(a.x_resid, e + 0) + acc.x);
    store_act<ACT>(a.x_next, e + 1, load_act<ACT>(a.x_resid, e + 1) + acc.y);
    store_act<ACT>(a.x_next, e + 2, load_act<ACT>(a.x_resid, e + 2) + acc.z);
    store_act<ACT>(a.x_next, e + 3, load_act<ACT>(a.x_resid, e + 3) + acc.w);
  }
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const size_t n = (size_t)a.T * (a.H / 4);
  const dim3 grid((unsigned)((n + 255) / 256));
  if (a.act == MOE_ACT_BF16) k_combine<MOE_ACT_BF16><<<grid, 256, 0, s>>>(a);
  else k_combine<MOE_ACT_F32><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

// out[r][c] = the format's dequantised weight, one element per thread.
template <int QF>
__global__ __launch_bounds__(256) void k_dequant(QMat m, int rows, int cols, float* out) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)rows * cols) return;
  const int r = (int)(idx / cols), c = (int)(idx % cols);
  const int G = cols / kGroup;
  const float s = f16_to_f32(m.scales[(size_t)r * G + c / kGroup]);
  if constexpr (QF == MOE_Q4_SYM_G32) {
    const uint32_t byte = m.codes[(size_t)r * (cols / 2) + c / 2];
    const int u = (c & 1) ? (int)(byte >> 4) : (int)(byte & 15u);
    out[idx] = s * (float)(u - 8);
  } else if constexpr (QF == MOE_Q3_SYM_G32) {
    const uint8_t* g = m.codes + (size_t)r * (G * 12) + (size_t)(c / kGroup) * 12;
    const int i = c % kGroup;
    const int u = (int)(((uint32_t)g[i / 4] >> (2 * (i % 4))) & 3u) | (int)((((uint32_t)g[8 + i / 8] >> (i % 8)) & 1u) << 2);
    out[idx] = s * (float)(u - 4);
  } else {
    const uint32_t byte = m.codes[(size_t)r * (cols / 4) + c / 4];
    const int u = (int)((byte >> (2 * (c & 3))) & 3u);
    out[idx] = fmaf(s, (float)u, f16_to_f32(m.mins[(size_t)r * G + c / kGroup]));
  }
}

hipError_t launch_dequant(const QMat& m, int qfmt, int rows, int cols, float* out, hipStream_t s) {
  const size_t n = (size_t)rows * cols;
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  by_qfmt(qfmt, [&](auto q) { k_dequant<decltype(q)::value><<<grid, 256, 0, s>>>(m, rows, cols, out); });
  return hipGetLastError();
}

}  // namespace moe
