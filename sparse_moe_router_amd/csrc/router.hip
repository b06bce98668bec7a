// Router logits and top-K selection (page 2 "Layer 1: On-Demand MoE Expert
// Scheduling": a light gating network picks the top-K experts of each token;
// page 3 "The 'Doorbell' Mechanism": the device decides each token's expert
// ids, which then stay on the device).
#include "moe_internal.h"
#include "topk.h"

namespace moe {

constexpr int kSmallRoutePairs = 256;

// logits[t][e] = sum_i W[e][i] x[t][i] + b[e].  One wave per router row e,
// NCH chunks of 256 elements (one float4 per lane each; chunks past H load a
// clamped in-range address and are zeroed).  For each pass of NT tokens the
// activations and the row are all requested before the first multiply.
template <int ACT, int NT, int NCH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void k_router_logits(RouterArgs a) {
  typedef float f4v __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= a.E) return;
  const float* wrow = a.w + (size_t)e * a.H;
  int col[NCH];
  bool ok[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int i = c * 256 + lane * 4;
    ok[c] = i < a.H;
    col[c] = ok[c] ? i : a.H - 4;
  }
  for (int t0 = blockIdx.y * NT; t0 < a.T; t0 += gridDim.y * NT) {
    f4v xs[NT][NCH];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const size_t row = (size_t)min(t0 + j, a.T - 1) * a.H;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        if constexpr (ACT == 1) {
          const uint2 b2 = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(a.x) + row + col[c]);
          xs[j][c][0] = bf16_to_f32(b2.x & 0xffffu);
          xs[j][c][1] = bf16_to_f32(b2.x >> 16);
          xs[j][c][2] = bf16_to_f32(b2.y & 0xffffu);
          xs[j][c][3] = bf16_to_f32(b2.y >> 16);
        } else {
          xs[j][c] = *reinterpret_cast<const f4v*>(reinterpret_cast<const float*>(a.x) + row + col[c]);
        }
      }
    }
    f4v w[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) w[c] = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(wrow + col[c]));
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      if (!ok[c]) w[c] = f4v{0.f, 0.f, 0.f, 0.f};
    float acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        s = fmaf(w[c][0], xs[j][c][0], s);
        s = fmaf(w[c][1], xs[j][c][1], s);
        s = fmaf(w[c][2], xs[j][c][2], s);
        s = fmaf(w[c][3], xs[j][c][3], s);
      }
      acc[j] = wave_sum(s);
    }
    if (lane == 0) {
      const float bias = a.b ? a.b[e] : 0.0f;
#pragma unroll
      for (int j = 0; j < NT; ++j)
        if (t0 + j < a.T) a.logits[(size_t)(t0 + j) * a.E + e] = acc[j] + bias;
    }
  }
}

// One wave per token, E <= 1024 (logits in registers).
template <int PL>
__global__ __launch_bounds__(256) void k_topk_regs(RouterArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  wave_topk_regs<PL>(a.logits + (size_t)t * a.E, a.E, a.K, lane, a.ids + (size_t)t * a.K, a.wts + (size_t)t * a.K,
                     nullptr);
}

// One wave per token for any E <= 8192: candidates in LDS.
__global__ __launch_bounds__(64) void k_topk_lds(RouterArgs a) {
  extern __shared__ uint32_t lds[];
  uint32_t* keys = lds;                                     // [E]
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
    const int id = key_id(best);
    if ((id & 63) == lane) keys[id] = 0u;  // the owning lane is the only reader of keys[id]
    if (lane == 0) chosen[k] = id;
  }
  __syncthreads();
  const float l0 = lg[chosen[0]];
  float part = 0.0f;
  for (int k = lane; k < a.K; k += 64) part += expf(lg[chosen[k]] - l0);
  const float total = wave_sum(part);
  for (int k = lane; k < a.K; k += 64) {
    const int id = chosen[k];
    a.ids[(size_t)t * a.K + k] = id;
    a.wts[(size_t)t * a.K + k] = expf(lg[id] - l0) / total;
  }
}

// Small batches (T*K <= 256, E <= 1024): top-K of every token and the stable
// token -> expert permutation in one block.  Pair p = t*K + k gets rank
// #{q : (e_q, q) < (e_p, p)}; offsets[e] is the first rank with expert >= e.
template <int PL>
__global__ __launch_bounds__(256) void k_route_small(RouterArgs a, PermuteArgs pm) {
  __shared__ int32_t s_ids[kSmallRoutePairs];
  __shared__ int32_t s_sorted[kSmallRoutePairs];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int t = wave; t < a.T; t += 4)
    wave_topk_regs<PL>(a.logits + (size_t)t * a.E, a.E, a.K, lane, a.ids + (size_t)t * a.K,
                       a.wts + (size_t)t * a.K, s_ids + t * a.K);
  __syncthreads();
  const int n = a.T * a.K, p = threadIdx.x;
  if (p < n) {
    const int e = s_ids[p];
    int rank = 0;
    for (int q = 0; q < n; ++q) {
      const int eq = s_ids[q];
      rank += (eq < e) | ((eq == e) & (q < p));
    }
    pm.sorted_pairs[rank] = p;
    pm.pair_pos[p] = rank;
    s_sorted[rank] = e;
  }
  __syncthreads();
  for (int e = threadIdx.x; e <= a.E; e += 256) {
    int lo = 0, hi = n;  // first rank with expert >= e
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_sorted[mid] < e) lo = mid + 1; else hi = mid;
    }
    pm.offsets[e] = lo;
  }
}

template <int ACT, int NT>
static void router_nch(const RouterArgs& a, dim3 grid, hipStream_t s) {
  const int nch = (a.H + 255) / 256;
  const dim3 block(256);
  if (nch <= 1) k_router_logits<ACT, NT, 1><<<grid, block, 0, s>>>(a);
  else if (nch <= 2) k_router_logits<ACT, NT, 2><<<grid, block, 0, s>>>(a);
  else if (nch <= 4) k_router_logits<ACT, NT, 4><<<grid, block, 0, s>>>(a);
  else if (nch <= 8) k_router_logits<ACT, NT, 8><<<grid, block, 0, s>>>(a);
  else k_router_logits<ACT, NT, 16><<<grid, block, 0, s>>>(a);
}

hipError_t launch_router_logits(const RouterArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int chunks = (a.T + 3) / 4;
  const dim3 grid((a.E + 3) / 4, a.T == 1 ? 1 : (chunks < 64 ? chunks : 64));
  if (a.T == 1) {
    if (a.act == MOE_ACT_BF16) router_nch<1, 1>(a, grid, s);
    else router_nch<0, 1>(a, grid, s);
  } else {
    if (a.act == MOE_ACT_BF16) router_nch<1, 4>(a, grid, s);
    else router_nch<0, 4>(a, grid, s);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const RouterArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.E <= 64 * kRegLogits) {
    const dim3 g((a.T + 3) / 4), b(256);
    switch (regs_per_lane(a.E)) {
      case 1: k_topk_regs<1><<<g, b, 0, s>>>(a); break;
      case 2: k_topk_regs<2><<<g, b, 0, s>>>(a); break;
      case 4: k_topk_regs<4><<<g, b, 0, s>>>(a); break;
      case 8: k_topk_regs<8><<<g, b, 0, s>>>(a); break;
      default: k_topk_regs<16><<<g, b, 0, s>>>(a); break;
    }
  } else {
    const size_t lds = (size_t)(a.E + a.K) * 4;
    k_topk_lds<<<dim3(a.T), dim3(64), lds, s>>>(a);
  }
  return hipGetLastError();
}

bool route_small_ok(int T, int K, int E) { return (int64_t)T * K <= kSmallRoutePairs && E <= 64 * kRegLogits; }

hipError_t launch_route_small(const RouterArgs& a, const PermuteArgs& p, hipStream_t s) {
  switch (regs_per_lane(a.E)) {
    case 1: k_route_small<1><<<1, 256, 0, s>>>(a, p); break;
    case 2: k_route_small<2><<<1, 256, 0, s>>>(a, p); break;
    case 4: k_route_small<4><<<1, 256, 0, s>>>(a, p); break;
    case 8: k_route_small<8><<<1, 256, 0, s>>>(a, p); break;
    default: k_route_small<16><<<1, 256, 0, s>>>(a, p); break;
  }
  return hipGetLastError();
}

}  // namespace moe
