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
//
// The operands reach LDS by the DMA path (global_load_lds: lane i of an
// instruction lands at the wave-uniform LDS base + 16 i) in chunks of 64 k,
// each instruction reading whole 64-byte runs of a row per four lanes (a quad
// of lanes reading four different rows costs the address unit four times as
// many requests).  Within a chunk the MFMA steps s = 0, 1 take, in lane
// group c, the k = 16 c + 8 s + e (e < 8): a permutation of the chunk's k,
// the same for x and W, so the dot products are unchanged.  Layouts, with
// every DMA instruction's kilobyte at a 1040-byte stride (16 bytes of skew):
//   x: instruction j < 8 holds rows j + 8 m (m < 8), 128 bytes each;
//   W: instruction 4 nt + j holds rows 16 nt + j + 4 m (m < 4), 256 bytes
//      each, rotated by 4 m 16-byte units,
// so that the 16 lanes of a read phase hit 16 distinct bank groups.
// Two tilings (64 tokens by 16 NT experts per block, 4 waves):
//   split over k (NT = 1, fewer than 1024 tokens): each wave streams a
//     quarter of the chunks through its own LDS ring, and the 4 partial
//     tiles are added in LDS in wave order (a fixed order);
//   split over experts (NT = 4): the waves share one ring, wave w owns the
//     16 experts of tile w.
// Workgroups are dealt round-robin over the 8 XCDs, so the blocks are
// numbered such that those of one token tile share an XCD (and its L2 copy of
// the x tile).  H must be a multiple of 64 (else the fp32 router runs).
constexpr int kRouterMfmaMinTokens = 64;
constexpr int kRouterWideTokens = 1024;  // from here on: split over experts
constexpr int kRChunkK = 64;             // k per chunk
constexpr int kRInst = 1040;             // LDS bytes per DMA instruction (1 KiB + skew)

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

template <int NT, bool SPLITK, int RING>
__global__ __launch_bounds__(256) void k_router_mfma(RouterArgs a, int nblocks, int per_xcd) {
  constexpr int XI = 8, WI = 4 * NT;                    // DMA instructions per chunk: x, W
  constexpr int CHUNK = (XI + WI) * kRInst;             // bytes of one ring slot
  constexpr int RINGS = SPLITK ? 4 : 1;                 // one ring per wave, or one per block
  constexpr int INST_W = SPLITK ? XI + WI : (XI + WI) / 4;  // DMA instructions per wave per chunk
  __shared__ __align__(16) uint8_t s_ring[RINGS * RING * CHUNK];
  const int bl = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  const int mblocks = (a.T + 63) / 64;
  if (bl >= mblocks * nblocks) return;  // whole block: before any barrier
  const int m0 = (bl / nblocks) * 64, n0 = (bl % nblocks) * 16 * NT;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln = lane & 15, lc = lane >> 4;
  const int nchunks = a.H / kRChunkK;
  int c0 = 0, c1 = nchunks;
  if constexpr (SPLITK) {
    const int per = (nchunks + 3) / 4;
    c0 = min(wave * per, nchunks);
    c1 = min(c0 + per, nchunks);  // c0 == c1: this wave adds zeros
  }
  uint8_t* ring = s_ring + (SPLITK ? wave * RING * CHUNK : 0);

  // this lane's source of each of the wave's DMA instructions (byte offset of
  // chunk 0; chunk c adds 128 c for x, 256 c for W) and its destination
  // instruction index within a ring slot.  Rows past T or E read the last row;
  // their results are dropped.
  const uint8_t* src[INST_W];
  int cstride[INST_W], dst[INST_W];
#pragma unroll
  for (int i = 0; i < INST_W; ++i) {
    const int J = SPLITK ? i : wave * INST_W + i;  // instruction of the chunk
    dst[i] = J;
    if (J < XI) {  // x: row j + 8 m, unit lane % 8
      const int m = lane >> 3, row = min(m0 + J + 8 * m, a.T - 1);
      src[i] = reinterpret_cast<const uint8_t*>(a.x) + (size_t)row * a.H * 2 + (lane & 7) * 16;
      cstride[i] = kRChunkK * 2;
    } else {  // W: tile nt, row 16 nt + j + 4 m, unit (p - 4 m) mod 16 at position p
      const int jw = J - XI, nt = jw >> 2, j = jw & 3, m = lane >> 4, p = lane & 15;
      const int row = min(n0 + 16 * nt + j + 4 * m, a.E - 1);
      src[i] = reinterpret_cast<const uint8_t*>(a.w) + (size_t)row * a.H * 4 + ((p - 4 * m) & 15) * 16;
      cstride[i] = kRChunkK * 4;
    }
  }
  auto issue = [&](int c, int slot) {  // chunk c (clamped: past the end, a slot that is never read)
    const int cc = min(c, c1 - 1);
#pragma unroll
    for (int i = 0; i < INST_W; ++i)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src[i] + (size_t)cc * cstride[i]),
                                       static_cast<void*>(ring + slot * CHUNK + dst[i] * kRInst), 16, 0, 0);
  };

  // read addresses (within a slot) of the MFMA operands of step s:
  //   A, tile mt: row R = 16 mt + ln -> instruction R % 8, offset 128 (R / 8) + 16 (2 lc + s)
  //   B, tile nt, half h: row n = ln -> instruction 8 + 4 nt + n % 4,
  //      offset 256 (n / 4) + 16 ((4 lc + 2 s + h + 4 (n / 4)) mod 16)
  constexpr int NTW = SPLITK ? NT : 1;  // N tiles this wave computes
  const int nt0 = SPLITK ? 0 : wave;
  int aoff[4], boff[NTW];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int R = 16 * mt + ln;
    aoff[mt] = (R & 7) * kRInst + (R >> 3) * 128 + 32 * lc;
  }
#pragma unroll
  for (int t = 0; t < NTW; ++t) boff[t] = (XI + 4 * (nt0 + t) + (ln & 3)) * kRInst + (ln >> 2) * 256;
  const int brot = 4 * lc + 4 * (ln >> 2);  // unit of (s, h) = (0, 0) before the mod

  rf32x4_t acc[4][NTW];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[mt][t] = rf32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int slot) {
    const uint8_t* base = ring + slot * CHUNK;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      ru32x4_t xa[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) xa[mt] = *reinterpret_cast<const ru32x4_t*>(base + aoff[mt] + 16 * s);
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const rf32x4_t w0 = *reinterpret_cast<const rf32x4_t*>(base + boff[t] + 16 * ((brot + 2 * s) & 15));
        const rf32x4_t w1 = *reinterpret_cast<const rf32x4_t*>(base + boff[t] + 16 * ((brot + 2 * s + 1) & 15));
        uint32_t h[4], m[4], l[4];
        split3(w0[0], w0[1], h[0], m[0], l[0]);
        split3(w0[2], w0[3], h[1], m[1], l[1]);
        split3(w1[0], w1[1], h[2], m[2], l[2]);
        split3(w1[2], w1[3], h[3], m[3], l[3]);
        const ru32x4_t hi = {h[0], h[1], h[2], h[3]}, mid = {m[0], m[1], m[2], m[3]}, lo = {l[0], l[1], l[2], l[3]};
        // each tile takes lo, mid, hi in that order; the 4 tiles interleave
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt][t] = router_mfma(xa[mt], lo, acc[mt][t]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt][t] = router_mfma(xa[mt], mid, acc[mt][t]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt][t] = router_mfma(xa[mt], hi, acc[mt][t]);
      }
    }
  };

  // the DMA writes LDS behind the compiler's back: its completion is awaited
  // with vmcnt (the wave's DMA instructions complete in order; the loop
  // issues no other vector-memory load), with a memory clobber
  if (c0 < c1) {
#pragma unroll
    for (int r = 0; r < RING - 1; ++r) issue(c0 + r, r);
    for (int c = c0; c < c1; ++c) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(INST_W * (RING - 2)) : "memory");
      if constexpr (!SPLITK) __syncthreads();  // every wave's part of chunk c is in; chunk c - 1 is done
      __builtin_amdgcn_sched_barrier(0);
      issue(c + RING - 1, (c - c0 + RING - 1) % RING);
      compute((c - c0) % RING);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the clamped tail loads land before the ring is reused

  if constexpr (SPLITK) {
    // partial tiles of waves 1..3 -> LDS (the ring's first bytes), added by wave 0 in wave order
    rf32x4_t* part = reinterpret_cast<rf32x4_t*>(s_ring);
    __syncthreads();
    if (wave > 0) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) part[((wave - 1) * 4 + mt) * 64 + lane] = acc[mt][0];
    }
    __syncthreads();
    if (wave > 0) return;
    for (int w = 1; w < 4; ++w)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt][0] += part[((w - 1) * 4 + mt) * 64 + lane];
  }

  // D lane l holds tokens 4 (l / 16) + i of each M tile, expert l % 16 of the N tile
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int en = n0 + 16 * (nt0 + t) + ln;
    if (en >= a.E) continue;
    const float bias = a.b ? a.b[en] : 0.0f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tk = m0 + mt * 16 + lc * 4 + i;
        if (tk < a.T) a.logits[(size_t)tk * a.E + en] = acc[mt][t][i] + bias;
      }
  }
}

template <int NT, bool SPLITK, int RING>
static void router_mfma(const RouterArgs& a, hipStream_t s) {
  const int nblocks = (a.E + 16 * NT - 1) / (16 * NT);
  const int total = (a.T + 63) / 64 * nblocks;
  const int per_xcd = (total + 7) / 8;
  k_router_mfma<NT, SPLITK, RING><<<dim3(8 * per_xcd), dim3(256), 0, s>>>(a, nblocks, per_xcd);
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
  __shared__ __align__(16) int32_t s_ids[kSmallRoutePairs];
  __shared__ int32_t s_sorted[kSmallRoutePairs];
  __shared__ int32_t s_wcount[kSmallRoutePairs / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = a.T * a.K;
  // positions past the pairs hold a sentinel above every expert id (the rank
  // loop reads them four at a time)
  for (int q = n + threadIdx.x; q < ((n + 3) & ~3); q += 64 * NWV) s_ids[q] = 0x7fffffff;
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
  const int p = threadIdx.x;
  if (p < n) {
    const int e = s_ids[p];
    int rank = 0;
    const int4* s4 = reinterpret_cast<const int4*>(s_ids);
#pragma unroll 4
    for (int q4 = 0; q4 < (n + 3) >> 2; ++q4) {
      const int4 v = s4[q4];
      const int q = 4 * q4;
      rank += (v.x < e) | ((v.x == e) & (q < p));
      rank += (v.y < e) | ((v.y == e) & (q + 1 < p));
      rank += (v.z < e) | ((v.z == e) & (q + 2 < p));
      rank += (v.w < e) | ((v.w == e) & (q + 3 < p));
    }
    pm.sorted_pairs[rank] = p;
    pm.pair_pos[p] = rank;
    if (pm.sorted_tok) pm.sorted_tok[rank] = p / a.K;
    s_sorted[rank] = e;
  }
  __syncthreads();
  if (pm.work) {
    // the distinct experts in sorted order: position y starts one if it is
    // the first of its expert; u = the number of starts before y
    const int y = threadIdx.x;
    const int e = y < n ? s_sorted[y] : -1;
    const bool first = y < n && (y == 0 || s_sorted[y - 1] != e);
    const uint64_t m = __ballot(first);
    if (y < kSmallRoutePairs && lane == 0) s_wcount[wave] = __popcll(m);
    __syncthreads();
    int u = __popcll(m & ((1ull << lane) - 1ull)), U = 0;
    for (int w = 0; w < kSmallRoutePairs / 64 && w < NWV; ++w) {
      if (w < wave) u += s_wcount[w];
      U += s_wcount[w];
    }
    int4* work = reinterpret_cast<int4*>(pm.work);
    if (first) {
      int lo = y + 1, hi = n;  // end of the run: first position with expert > e
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_sorted[mid] <= e) lo = mid + 1; else hi = mid;
      }
      work[u] = make_int4(e, y, lo - y, 0);
    }
    if (y >= U && y < n) work[y] = make_int4(-1, 0, 0, 0);
  }
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
  if (a.act == MOE_ACT_BF16 && a.T >= kRouterMfmaMinTokens && a.H % kRChunkK == 0) {
    // rings of two chunks: a third slot measured no faster (the loop is bound
    // by its split and MFMA work, not by the DMA's latency)
    if (a.T >= kRouterWideTokens) router_mfma<4, false, 2>(a, s);
    else router_mfma<1, true, 2>(a, s);
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
