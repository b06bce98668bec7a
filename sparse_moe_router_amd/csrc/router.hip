// Router logits and top-K selection (page 2 "Layer 1: On-Demand MoE Expert
// Scheduling": a light gating network picks the top-K experts of each token;
// page 3 "The 'Doorbell' Mechanism": the device decides each token's expert
// ids, which then stay on the device).
#include "moe_internal.h"
#include "topk.h"

namespace moe {

constexpr int kSmallRoutePairs = 256;

// logits[t][e] = sum_i W[e][i] x[t][i] + b[e].  One wave per router row e
// (blocks of 4 waves, or of one wave for one token),
// NCH chunks of 256 elements (one float4 per lane each; chunks past H load a
// clamped in-range address and are zeroed).  For each pass of NT tokens the
// activations and the row are all requested before the first multiply.
template <int ACT, int NT, int NCH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void k_router_logits(RouterArgs a) {
  typedef float f4v __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (e >= a.E) return;
  const float* wrow = a.w + (size_t)e * a.H;
  const float bias = a.b ? a.b[e] : 0.0f;  // requested first: not a round trip after the sum
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
#pragma unroll
      for (int j = 0; j < NT; ++j)
        if (t0 + j < a.T) a.logits[(size_t)(t0 + j) * a.E + e] = acc[j] + bias;
    }
  }
}

// ---------------------------------------------------------------------------
// Many tokens (bf16 activations): the logits as a GEMM on the matrix cores.
// Each fp32 router weight w is split exactly into three bf16 parts,
//   hi = w truncated to bf16,  mid = (w - hi) truncated,  lo = w - hi - mid,
// (every difference is exact in fp32 and lo has at most 8 significant bits),
// so with bf16 x every product x * part is exact in fp32 and the MFMA chain
// lo, mid, hi accumulates sum_k x_k w_k in fp32 like any fp32 dot product,
// over 3 H exact terms.  The split is done in registers per 32-k step.
// Block: 64 tokens x 64 experts, 4 waves; wave w owns experts n0 + 16 w ..
// + 15 and all 64 tokens (4 MFMA tiles of 16 x 16); the x tile is staged
// through LDS in 128-k chunks (double buffered), shared by the 4 waves.
constexpr int kRouterMfmaMinTokens = 128;
constexpr int kRM = 64, kRN = 64, kRKC = 128;
constexpr int kRRow = kRKC + 8;  // bf16 per LDS row (+8: conflict-free 16-byte reads)

typedef __bf16 rbf16x8_t __attribute__((ext_vector_type(8)));
typedef float rf32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t ru32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ rf32x4_t router_mfma(ru32x4_t a, ru32x4_t b, rf32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(rbf16x8_t, a), __builtin_bit_cast(rbf16x8_t, b),
                                                 c, 0, 0, 0);
}

// Two fp32 weights -> their hi, mid and lo bf16 parts, packed as pairs (element 0 low).
__device__ __forceinline__ void split3(float w0, float w1, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  const uint32_t b0 = __float_as_uint(w0), b1 = __float_as_uint(w1);
  const float h0 = __uint_as_float(b0 & 0xffff0000u), h1 = __uint_as_float(b1 & 0xffff0000u);
  const float r0 = w0 - h0, r1 = w1 - h1;
  const uint32_t rb0 = __float_as_uint(r0), rb1 = __float_as_uint(r1);
  const float m0 = __uint_as_float(rb0 & 0xffff0000u), m1 = __uint_as_float(rb1 & 0xffff0000u);
  const uint32_t l0 = __float_as_uint(r0 - m0), l1 = __float_as_uint(r1 - m1);
  hi = __builtin_amdgcn_perm(b1, b0, 0x07060302u);  // top halves: (b0 >> 16) | (b1 & 0xffff0000)
  mid = __builtin_amdgcn_perm(rb1, rb0, 0x07060302u);
  lo = __builtin_amdgcn_perm(l1, l0, 0x07060302u);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_router_mfma(RouterArgs a) {
  __shared__ __align__(16) uint16_t s_x[2][kRM * kRRow];
  const int m0 = blockIdx.x * kRM, n0 = blockIdx.y * kRN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ln = lane & 15, lc = lane >> 4;
  const int nchunks = (a.H + kRKC - 1) / kRKC;

  // staging: thread -> token row r = tid / 4, 32-k slice q = tid % 4 of the chunk (4 x 16 bytes)
  const int r = threadIdx.x >> 2, q = threadIdx.x & 3;
  const uint16_t* xrow = reinterpret_cast<const uint16_t*>(a.x) + (size_t)min(m0 + r, a.T - 1) * a.H;
  ru32x4_t st[4];  // native vectors: with HIP's uint4 the compiler kept this array in scratch memory
  auto load_x = [&](int kc) {
    const int k = min(kc * kRKC + q * 32, a.H - 32);  // past H: any in-range slice, never used
    const ru32x4_t* src = reinterpret_cast<const ru32x4_t*>(xrow + k);
#pragma unroll
    for (int i = 0; i < 4; ++i) st[i] = src[i];
  };
  auto store_x = [&](int buf) {
    ru32x4_t* dst = reinterpret_cast<ru32x4_t*>(&s_x[buf][r * kRRow + q * 32]);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = st[i];
  };

  // B: this lane's expert row and k offset within a 32-k step
  const int e = min(n0 + wave * 16 + ln, a.E - 1);
  const float* wrow = a.w + (size_t)e * a.H + lc * 8;
  rf32x4_t acc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) acc[mt] = rf32x4_t{0.f, 0.f, 0.f, 0.f};

  // this lane's 8 weights of each 32-k step of a chunk, prefetched one chunk ahead
  float4 wv[4][2], wn[4][2];
  auto load_w = [&](int kc, float4 (&w)[4][2]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = min(kc * kRKC + j * 32, a.H - 32);  // past H: any in-range step, never used
      w[j][0] = *reinterpret_cast<const float4*>(wrow + k);
      w[j][1] = *reinterpret_cast<const float4*>(wrow + k + 4);
    }
  };

  load_x(0);
  load_w(0, wv);
  store_x(0);
  __syncthreads();
  for (int kc = 0; kc < nchunks; ++kc) {
    const int buf = kc & 1;
    const int steps = min(kRKC, a.H - kc * kRKC) / 32;  // H is a multiple of 32
    // the next chunk's loads and LDS store are branch-free (indices clamped;
    // after the last chunk they fill a buffer that is never read), so the
    // staged values stay in registers and no wait lands before the products
    load_x(kc + 1);
    load_w(kc + 1, wn);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < steps) {
        uint32_t h[4], m[4], l[4];
        split3(wv[j][0].x, wv[j][0].y, h[0], m[0], l[0]);
        split3(wv[j][0].z, wv[j][0].w, h[1], m[1], l[1]);
        split3(wv[j][1].x, wv[j][1].y, h[2], m[2], l[2]);
        split3(wv[j][1].z, wv[j][1].w, h[3], m[3], l[3]);
        const ru32x4_t hi = {h[0], h[1], h[2], h[3]}, mid = {m[0], m[1], m[2], m[3]}, lo = {l[0], l[1], l[2], l[3]};
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const ru32x4_t xa = *reinterpret_cast<const ru32x4_t*>(&s_x[buf][(mt * 16 + ln) * kRRow + j * 32 + lc * 8]);
          acc[mt] = router_mfma(xa, lo, acc[mt]);
          acc[mt] = router_mfma(xa, mid, acc[mt]);
          acc[mt] = router_mfma(xa, hi, acc[mt]);
        }
      }
    }
    store_x(buf ^ 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wv[j][0] = wn[j][0];
      wv[j][1] = wn[j][1];
    }
    __syncthreads();
  }

  // D lane l holds tokens 4 (l / 16) + i of each M tile, expert ln of the wave's 16
  const int en = n0 + wave * 16 + ln;
  if (en < a.E) {
    const float bias = a.b ? a.b[en] : 0.0f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = m0 + mt * 16 + lc * 4 + i;
        if (t < a.T) a.logits[(size_t)t * a.E + en] = acc[mt][i] + bias;
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

__device__ __forceinline__ const float* lg_row(const RouterArgs& a, int t) { return a.logits + (size_t)t * a.E; }

// Small batches (T*K <= 256, E <= 1024): top-K of every token and the stable
// token -> expert permutation in one block of NWV waves (one token per wave
// up to NWV tokens; 16 waves up to E = 512, 4 above, whose selection state
// needs more registers).  Pair p = t*K + k gets rank
// #{q : (e_q, q) < (e_p, p)}; offsets[e] is the first rank with expert >= e.
template <int PL, int NWV>
__global__ __launch_bounds__(64 * NWV) void k_route_small(RouterArgs a, PermuteArgs pm) {
  __shared__ int32_t s_ids[kSmallRoutePairs];
  __shared__ int32_t s_sorted[kSmallRoutePairs];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if constexpr (PL <= 8) {
    if (a.K <= 64) {  // consecutive experts per lane: one wave maximum and one ballot per round
      for (int t = wave; t < a.T; t += NWV) {
        const float* lg = a.logits + (size_t)t * a.E;
        LaneSorted<PL> ls;
        ls.load(lg, a.E, lane);
        uint32_t mine = 0, top = 0;  // lane k keeps the key of round k
        for (int k = 0; k < a.K; ++k) {
          const uint32_t m = ls.round(lane, k, s_ids + t * a.K);
          if (k == 0) top = m;
          if (lane == k) mine = m;
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        write_topk(mine, s_ids[t * a.K + min(lane, a.K - 1)], top, a.K, lane, a.ids + (size_t)t * a.K,
                   a.wts + (size_t)t * a.K);
      }
    } else {
      for (int t = wave; t < a.T; t += NWV)
        wave_topk_regs<PL>(lg_row(a, t), a.E, a.K, lane, a.ids + (size_t)t * a.K, a.wts + (size_t)t * a.K,
                           s_ids + t * a.K);
    }
  } else {
    for (int t = wave; t < a.T; t += NWV)
      wave_topk_regs<PL>(lg_row(a, t), a.E, a.K, lane, a.ids + (size_t)t * a.K, a.wts + (size_t)t * a.K,
                         s_ids + t * a.K);
  }
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
  for (int e = threadIdx.x; e <= a.E; e += 64 * NWV) {
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
  // one token: one wave per block, so that the E rows spread over every CU
  const dim3 block(a.T == 1 ? 64 : 256);
  if (a.T == 1) grid.x = a.E;
  if (nch <= 1) k_router_logits<ACT, NT, 1><<<grid, block, 0, s>>>(a);
  else if (nch <= 2) k_router_logits<ACT, NT, 2><<<grid, block, 0, s>>>(a);
  else if (nch <= 4) k_router_logits<ACT, NT, 4><<<grid, block, 0, s>>>(a);
  else if (nch <= 8) k_router_logits<ACT, NT, 8><<<grid, block, 0, s>>>(a);
  else k_router_logits<ACT, NT, 16><<<grid, block, 0, s>>>(a);
}

hipError_t launch_router_logits(const RouterArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.act == MOE_ACT_BF16 && a.T >= kRouterMfmaMinTokens) {
    k_router_mfma<<<dim3((a.T + kRM - 1) / kRM, (a.E + kRN - 1) / kRN), 256, 0, s>>>(a);
    return hipGetLastError();
  }
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
    case 1: k_route_small<1, 16><<<1, 64 * 16, 0, s>>>(a, p); break;
    case 2: k_route_small<2, 16><<<1, 64 * 16, 0, s>>>(a, p); break;
    case 4: k_route_small<4, 16><<<1, 64 * 16, 0, s>>>(a, p); break;
    case 8: k_route_small<8, 16><<<1, 64 * 16, 0, s>>>(a, p); break;
    default: k_route_small<16, 4><<<1, 64 * 4, 0, s>>>(a, p); break;
  }
  return hipGetLastError();
}

}  // namespace moe
