// Expert SwiGLU FFNs with in-register dequantisation, for few tokens per
// expert (decode, speculative verify, small batches).  The expert weights are
// the dominant bytes of the layer and are streamed from HBM once per expert
// (low-bit weights: page 1 "How Strata Makes the Impossible Possible"; SwiGLU
// expert sub-networks: page 2 "Layer 1"; shared expert: page 5).
//
// Work split: one wave owns RPW rows of one matrix of one expert and all the
// expert's tokens.  A row's 32-element groups are spread over LPR lanes (one
// group per lane at H = 2048: each lane loads 16 B of 4-bit codes and one fp16
// scale per row); partial dot products are reduced over those LPR lanes.
#include "gemv_one.h"
#include "topk.h"

namespace moe {

// Which token list a block works on: a routed expert (its slice of the sorted
// pairs) or the shared expert (all tokens).  Block row y visits sorted
// positions y, y + ny, ... and takes the expert whose slice starts there (the
// expert of position j is ids[sorted_pairs[j]]), so each expert is handled by
// exactly one block row and needs two dependent loads to find.
struct Work {
  int expert;   // routed expert id, or -1 for the shared expert
  int lo, n;    // sorted positions [lo, lo + n) or tokens [0, n)
  int pair0;    // sorted_pairs[lo] (routed)
};

__device__ __forceinline__ bool next_routed(const FfnArgs& a, int ny, int* pos, Work* w) {
  const int n = a.T * a.K;
  for (; *pos < n; *pos += ny) {
    const int j = *pos;
    const int pj = a.sorted_pairs[j];
    const int pp = j > 0 ? a.sorted_pairs[j - 1] : pj;
    const int e = a.ids[pj];
    if (j == 0 || a.ids[pp] != e) {
      const int cnt = a.offsets[e + 1] - j;
      if (on_mfma(a, cnt)) continue;  // the grouped GEMM takes this expert
      w->expert = e;
      w->lo = j;
      w->pair0 = pj;
      w->n = cnt;
      *pos += ny;
      return true;
    }
  }
  return false;
}

// Occupancy the register budget is sized for: the decode shapes (one token
// chunk, one group per lane) fit four waves per SIMD.
constexpr int waves_per_simd(int act, int nt, int gpl) {
  return (act == MOE_ACT_BF16 && gpl == 1) ? (nt == 1 ? 4 : 2) : 1;
}

// gate/up + SwiGLU of one expert (or the shared expert) for the wave's RPW
// rows:  h[j][r] = round_act(silu(Wg[r].x_t) * (Wu[r].x_t)).  The activations
// of the first chunk of tokens, then the weights, are all requested before the
// first arithmetic (the memory counter completes in issue order); the weight
// rows are loaded once and reused for every chunk of NT tokens.  tok(jj) gives
// the token of the expert's jj-th pair.
template <int QF, int ACT, int NT, int GPL, int RPW, typename TokFn>
__device__ __forceinline__ void gateup_rows(const FfnArgs& a, const Work& wk, bool shared, int rbase, int rsub,
                                            int sub, int lpr_log2, TokFn tok) {
  const int LPR = 1 << lpr_log2, RPI = 64 >> lpr_log2;
  const int G = a.H / kGroup;
  const int r0 = rbase + rsub;
  bool gok[GPL];
#pragma unroll
  for (int gi = 0; gi < GPL; ++gi) gok[gi] = sub + gi * LPR < G;
  void* out = shared ? a.hs : a.h;
  XGroup<QF, ACT> xg[NT][GPL];
  auto load_x = [&](int c0) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int jj = c0 + min(j, wk.n - 1 - c0);  // clamped: duplicates past the end
      const int t = tok(jj);
#pragma unroll
      for (int gi = 0; gi < GPL; ++gi)
        xg[j][gi].load_raw(a.x, (size_t)t * a.H + (size_t)min(sub + gi * LPR, G - 1) * kGroup);
    }
  };
  load_x(0);
  __builtin_amdgcn_sched_barrier(0);  // keep the activation loads ahead of the weight loads
  const bool keep = hot_expert(a, shared, wk.expert);
  const MatView vg = expert_view<QF>(shared ? a.sgate : a.gate, shared ? 0 : wk.expert, a.I, a.H, keep);
  const MatView vu = expert_view<QF>(shared ? a.sup : a.up, shared ? 0 : wk.expert, a.I, a.H, keep);
  RowTile<QF, RPW, GPL> tg, tu;
  tg.load(vg, rbase, rsub, RPI, a.I, sub, LPR);
  tu.load(vu, rbase, rsub, RPI, a.I, sub, LPR);
  __builtin_amdgcn_sched_barrier(0);  // ... and every load issued before the arithmetic
  for (int c0 = 0; c0 < wk.n; c0 += NT) {
    const int nt = min(NT, wk.n - c0);
    if (c0 > 0) load_x(c0);
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int gi = 0; gi < GPL; ++gi) xg[j][gi].prep();
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      __builtin_amdgcn_sched_barrier(0);  // one row at a time: unpacked codes stay few
      const int r = r0 + rr * RPI;
      float ga[NT], ua[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) { ga[j] = 0.f; ua[j] = 0.f; }
#pragma unroll
      for (int gi = 0; gi < GPL; ++gi) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          if (j < nt) {
            const float g1 = group_acc<QF, ACT>(ga[j], tg.c[rr][gi], tg.s[rr][gi], tg.m[rr][gi], xg[j][gi]);
            const float u1 = group_acc<QF, ACT>(ua[j], tu.c[rr][gi], tu.s[rr][gi], tu.m[rr][gi], xg[j][gi]);
            ga[j] = gok[gi] ? g1 : ga[j];
            ua[j] = gok[gi] ? u1 : ua[j];
          }
        }
      }
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        if (j < nt) {
          const float gs = seg_sum(ga[j], LPR);
          const float us = seg_sum(ua[j], LPR);
          if (sub == 0 && r < a.I) {
            const size_t row = shared ? (size_t)(c0 + j) : (size_t)(wk.lo + c0 + j);
            store_act<ACT>(out, row * a.I + r, silu(gs) * us);
          }
        }
      }
    }
  }
}

template <int QF, int ACT, int NT, int GPL, int RPW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(waves_per_simd(ACT, NT, GPL)))) void k_gateup(
    FfnArgs a, int ny, int lpr_log2) {
  const bool shared = (int)blockIdx.y == ny;  // the extra last row of blocks
  if (shared && on_mfma(a, a.T)) return;
  int pos = blockIdx.y;
  Work wk;
  if (shared) { wk.expert = -1; wk.lo = 0; wk.n = a.T; wk.pair0 = 0; }
  else if (!next_routed(a, ny, &pos, &wk)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int LPR = 1 << lpr_log2, RPI = 64 >> lpr_log2;
  const int rbase = (blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(wave)) * RPW * RPI;
  for (;;) {
    auto tok = [&](int jj) {
      return shared ? jj : ((jj == 0 ? wk.pair0 : a.sorted_pairs[wk.lo + jj]) / a.K);
    };
    gateup_rows<QF, ACT, NT, GPL, RPW>(a, wk, shared, rbase, lane >> lpr_log2, lane & (LPR - 1), lpr_log2, tok);
    if (shared || !next_routed(a, ny, &pos, &wk)) return;
  }
}

// ---- one token, H <= 2048 (one 32-element group per lane) ----------------

constexpr int kFusedRpw1 = 2;  // rows per wave of the one-token gate/up kernels

// gate/up + SwiGLU of RPW rows (rbase ..) of one expert for one token, with
// the weight rows already requested and x in LDS; h row hrow.
template <int QF, int RPW>
__device__ __forceinline__ void gateup_rows1(const FfnArgs& a, bool shared, int hrow, int rbase, int lane,
                                             const RowTile<QF, RPW, 1>& tg, const RowTile<QF, RPW, 1>& tu,
                                             const XLds& xs) {
  XGroup<QF, MOE_ACT_BF16> xg;
  read_x1<QF>(xs, lane, xg);
  const bool gok = lane < a.H / kGroup;
  float v[2 * RPW];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    __builtin_amdgcn_sched_barrier(0);  // one row at a time: unpacked codes stay few
    const float gv = group_acc<QF, MOE_ACT_BF16>(0.f, tg.c[rr][0], tg.s[rr][0], tg.m[rr][0], xg);
    const float uv = group_acc<QF, MOE_ACT_BF16>(0.f, tu.c[rr][0], tu.s[rr][0], tu.m[rr][0], xg);
    v[rr] = gok ? gv : 0.f;
    v[RPW + rr] = gok ? uv : 0.f;
  }
  float g, u;
  reduce_gu1<RPW>(v, lane, &g, &u);
  constexpr int kStride = RPW == 1 ? 32 : 32 / RPW;
  const int rr = lane / kStride, r = rbase + rr;
  if (lane < 32 && (lane & (kStride - 1)) == 0 && r < a.I)
    store_act<MOE_ACT_BF16>(shared ? a.hs : a.h, (size_t)hrow * a.I + r, silu(g) * u);
}

// Standalone gate/up for one token (moe_expert_gate_up_q, T = 1): block row
// k < K computes pair k, whose expert is ids[k], into h row pair_pos[k] (the
// rank of (ids[k], k)), both from one load of the K ids; row K is the shared
// expert.  Wave 0 requests x before the ids and the weights, and stages it
// in LDS while the weights are in flight.
template <int QF, int RPW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(waves_per_simd(MOE_ACT_BF16, 1, 1)))) void
k_gateup1(FfnArgs a) {
  __shared__ XLds xs;
  const int K = a.K, y = blockIdx.y;
  const bool shared = y == K;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // (loads complete in order: requested after the weights, x could only be
  // staged once they had landed)
  XGroup<QF, MOE_ACT_BF16> xg;
  if (wave == 0) load_x1<QF>(a.x, a.H, lane, xg);
  int e = 0, hrow = 0;
  if (!shared) {
    const int id = a.ids[min(lane, K - 1)];
    e = __builtin_amdgcn_readlane(id, y);
    hrow = __popcll(__ballot(lane < K && (id < e || (id == e && lane < y))));
  }
  const int rbase = (blockIdx.x * 4 + wave) * RPW;
  RowTile<QF, RPW, 1> tg, tu;
  const bool keep = hot_expert(a, shared, e);
  tg.load(expert_view<QF>(shared ? a.sgate : a.gate, e, a.I, a.H, keep), rbase, 0, 1, a.I, lane, 64);
  tu.load(expert_view<QF>(shared ? a.sup : a.up, e, a.I, a.H, keep), rbase, 0, 1, a.I, lane, 64);
  if (wave == 0) put_x1<QF>(xg, lane, xs);
  __syncthreads();
  gateup_rows1<QF, RPW>(a, shared, hrow, rbase, lane, tg, tu, xs);
}

bool gateup1_ok(const FfnArgs& a) {
  return a.T == 1 && a.act == MOE_ACT_BF16 && a.H <= 64 * kGroup && a.K <= 64;
}

// down projection:  o[j][r] = Wd[r] . h_j   (fp32 out); h rows of an expert are
// contiguous in sorted order, so no index is loaded before the weights.
template <int QF, int ACT, int NT, int GPL, int RPW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(waves_per_simd(ACT, NT, GPL)))) void k_down(FfnArgs a, int ny,
                                                                                    int lpr_log2) {
  const bool shared = (int)blockIdx.y == ny;
  if (shared && on_mfma(a, a.T)) return;
  int pos = blockIdx.y;
  Work wk;
  if (shared) { wk.expert = -1; wk.lo = 0; wk.n = a.T; }
  else if (!next_routed(a, ny, &pos, &wk)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int LPR = 1 << lpr_log2, RPI = 64 >> lpr_log2;
  const int sub = lane & (LPR - 1), rsub = lane >> lpr_log2;
  const int G = a.I / kGroup;
  const int rbase = (blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(wave)) * RPW * RPI;
  const int r0 = rbase + rsub;
  bool gok[GPL];
#pragma unroll
  for (int gi = 0; gi < GPL; ++gi) gok[gi] = sub + gi * LPR < G;
  const void* hin = shared ? a.hs : a.h;
  float* out = shared ? a.so : a.o;
  for (;;) {
    XGroup<QF, ACT> hg[NT][GPL];
    auto load_h = [&](int c0) {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const size_t row = (shared ? 0 : (size_t)wk.lo) + (size_t)(c0 + min(j, wk.n - 1 - c0));
#pragma unroll
        for (int gi = 0; gi < GPL; ++gi)
          hg[j][gi].load_raw(hin, row * a.I + (size_t)min(sub + gi * LPR, G - 1) * kGroup);
      }
    };
    load_h(0);
    __builtin_amdgcn_sched_barrier(0);
    const MatView vd = expert_view<QF>(shared ? a.sdown : a.down, shared ? 0 : wk.expert, a.H, a.I,
                                       hot_expert(a, shared, wk.expert));
    RowTile<QF, RPW, GPL> td;
    td.load(vd, rbase, rsub, RPI, a.H, sub, LPR);
    __builtin_amdgcn_sched_barrier(0);
    for (int c0 = 0; c0 < wk.n; c0 += NT) {
      const int nt = min(NT, wk.n - c0);
      if (c0 > 0) load_h(c0);
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int gi = 0; gi < GPL; ++gi) hg[j][gi].prep();
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr) {
        __builtin_amdgcn_sched_barrier(0);
        const int r = r0 + rr * RPI;
        float acc[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[j] = 0.f;
#pragma unroll
        for (int gi = 0; gi < GPL; ++gi) {
#pragma unroll
          for (int j = 0; j < NT; ++j) {
            if (j < nt) {
              const float v1 = group_acc<QF, ACT>(acc[j], td.c[rr][gi], td.s[rr][gi], td.m[rr][gi], hg[j][gi]);
              acc[j] = gok[gi] ? v1 : acc[j];
            }
          }
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          if (j < nt) {
            const float v = seg_sum(acc[j], LPR);
            if (sub == 0 && r < a.H) {
              const size_t row = shared ? (size_t)(c0 + j) : (size_t)(wk.lo + c0 + j);
              out[row * a.H + r] = v;
            }
          }
        }
      }
    }
    if (shared || !next_routed(a, ny, &pos, &wk)) return;
  }
}

// lanes per row (power of two) and groups per lane for a row of `cols`
static void lane_split(int cols, int* lpr_log2, int* gpl) {
  const int G = cols / kGroup;
  int l = 0;
  while ((1 << l) < G && l < 6) ++l;
  *lpr_log2 = l;
  *gpl = (G + (1 << l) - 1) >> l;
}

constexpr int kRPW = 4;

template <int QF, int ACT, int NT>
static hipError_t dispatch_gpl(const FfnArgs& a, bool gateup, hipStream_t s) {
  const int cols = gateup ? a.H : a.I;
  const int rows = gateup ? a.I : a.H;
  int lpr_log2, gpl;
  lane_split(cols, &lpr_log2, &gpl);
  const int rpi = 64 >> lpr_log2;
  const int rows_per_block = 4 * kRPW * rpi;
  // routed rows of blocks: one per selected pair up to E (an expert per block
  // row when every expert is distinct), then one extra row for the shared expert
  const int ny = min(a.E, a.T * a.K);
  const bool with_shared = a.n_shared && (gateup ? a.hs != nullptr : a.so != nullptr);
  const dim3 grid((rows + rows_per_block - 1) / rows_per_block, ny + (with_shared ? 1 : 0));
  const dim3 block(256);
  if (gpl == 1) {
    if (gateup) k_gateup<QF, ACT, NT, 1, kRPW><<<grid, block, 0, s>>>(a, ny, lpr_log2);
    else k_down<QF, ACT, NT, 1, kRPW><<<grid, block, 0, s>>>(a, ny, lpr_log2);
  } else {
    if (gateup) k_gateup<QF, ACT, NT, 2, kRPW><<<grid, block, 0, s>>>(a, ny, lpr_log2);
    else k_down<QF, ACT, NT, 2, kRPW><<<grid, block, 0, s>>>(a, ny, lpr_log2);
  }
  return hipGetLastError();
}

template <int QF>
static hipError_t dispatch_act(const FfnArgs& a, bool gateup, hipStream_t s) {
  if (a.act == MOE_ACT_F32) return dispatch_gpl<QF, MOE_ACT_F32, 4>(a, gateup, s);
  if (a.T == 1) return dispatch_gpl<QF, MOE_ACT_BF16, 1>(a, gateup, s);
  return dispatch_gpl<QF, MOE_ACT_BF16, 4>(a, gateup, s);
}

// rows per wave of the standalone one-token gate/up: the same as the fused
// kernel's, so that both reduce in the same order and give the same bits
constexpr int kGateup1Rpw = kFusedRpw1;

template <int QF>
static hipError_t gateup1_q(const FfnArgs& a, hipStream_t s) {
  const dim3 grid((a.I + 4 * kGateup1Rpw - 1) / (4 * kGateup1Rpw), a.K + (a.n_shared && a.hs ? 1 : 0));
  k_gateup1<QF, kGateup1Rpw><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gateup(const FfnArgs& args, hipStream_t s) {
  if (args.T == 0) return hipSuccess;
  FfnArgs a = args;
  a.mfma_min = mfma_split(a);
  if (a.mfma_min > 0) {
    const hipError_t e = launch_mfma_gateup(a, s);
    if (e != hipSuccess || a.mfma_min == 1) return e;
  }
  if (gateup1_ok(a))
    return by_qfmt(a.qfmt, [&](auto q) { return gateup1_q<decltype(q)::value>(a, s); });
  if (gateup_sb_ok(a)) return launch_gateup_sb(a, s);
  return by_qfmt(a.qfmt, [&](auto q) { return dispatch_act<decltype(q)::value>(a, true, s); });
}

template <int QF> static hipError_t down1_q(const FfnArgs& a, hipStream_t s);
bool down1_ok(const FfnArgs& a);

hipError_t launch_down(const FfnArgs& args, hipStream_t s) {
  if (args.T == 0) return hipSuccess;
  FfnArgs a = args;
  a.mfma_min = mfma_split(a);
  if (a.mfma_min > 0) {
    const hipError_t e = launch_mfma_down(a, s);
    if (e != hipSuccess || a.mfma_min == 1) return e;
  }
  if (down1_ok(a)) return by_qfmt(a.qfmt, [&](auto q) { return down1_q<decltype(q)::value>(a, s); });
  if (down_sb_ok(a)) return launch_down_sb(a, s);
  return by_qfmt(a.qfmt, [&](auto q) { return dispatch_act<decltype(q)::value>(a, false, s); });
}


// ============================================================================
// Fused decode path (few tokens): the expert kernels compute the routing they
// need themselves, so a layer is three kernels: router logits, gate/up, and
// (one token) down projection with the weighted combine.

constexpr int kFusedMaxPairs = 128;
constexpr int kFusedMaxK1 = 16;  // top-K of the one-token path

// gate/up with the top-K and the stable token -> expert ordering recomputed in
// every block from the router logits (2 KiB per token at E = 512): block row y
// is sorted position y and works only if it is its expert's first position.
// The block at (0, 0) writes the routing outputs (ids, weights, offsets,
// sorted_pairs, pair_pos) exactly as moe_router_topk and moe_permute do.
template <int QF, int NT, int PL, int RPW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(waves_per_simd(MOE_ACT_BF16, NT, 1)))) void
k_fused_gateup(RouterArgs r, PermuteArgs pm, FfnArgs a, int lpr_log2) {
  __shared__ int32_t s_ids[kFusedMaxPairs];
  __shared__ int32_t s_pair[kFusedMaxPairs];
  __shared__ int32_t s_exp[kFusedMaxPairs];
  const int n = a.T * a.K;
  const bool shared = (int)blockIdx.y == n;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  Work wk;
  if (shared) {
    wk.expert = -1; wk.lo = 0; wk.n = a.T; wk.pair0 = 0;
  } else {
    const bool lead = blockIdx.x == 0 && blockIdx.y == 0;
    for (int t = wave; t < a.T; t += 4)
      wave_topk_regs<PL>(r.logits + (size_t)t * r.E, r.E, r.K, lane, lead ? r.ids + (size_t)t * r.K : nullptr,
                         lead ? r.wts + (size_t)t * r.K : nullptr, s_ids + t * r.K);
    __syncthreads();
    const int p = threadIdx.x;
    if (p < n) {
      const int e = s_ids[p];
      int rank = 0;
      for (int q = 0; q < n; ++q) {
        const int eq = s_ids[q];
        rank += (eq < e) | ((eq == e) & (q < p));
      }
      s_pair[rank] = p;
      s_exp[rank] = e;
      if (lead) {
        pm.sorted_pairs[rank] = p;
        pm.pair_pos[p] = rank;
      }
    }
    __syncthreads();
    if (lead) {
      for (int e = threadIdx.x; e <= r.E; e += 256) {
        int lo = 0, hi = n;  // first rank with expert >= e
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (s_exp[mid] < e) lo = mid + 1; else hi = mid;
        }
        pm.offsets[e] = lo;
      }
    }
    const int y = blockIdx.y;
    const int e = s_exp[y];
    if (y > 0 && s_exp[y - 1] == e) return;  // not the expert's first position
    int cnt = 1;
    while (y + cnt < n && s_exp[y + cnt] == e) ++cnt;
    wk.expert = e; wk.lo = y; wk.n = cnt; wk.pair0 = s_pair[y];
  }
  const int LPR = 1 << lpr_log2, RPI = 64 >> lpr_log2;
  const int rbase = (blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(wave)) * RPW * RPI;
  auto tok = [&](int jj) { return shared ? jj : s_pair[wk.lo + jj] / a.K; };
  gateup_rows<QF, MOE_ACT_BF16, NT, 1, RPW>(a, wk, shared, rbase, lane >> lpr_log2, lane & (LPR - 1), lpr_log2, tok);
}

// One token: block row k < K computes the expert picked in selection round k
// and writes h row k (h in slot order, as k_fused_down1 reads it); row K is
// the shared expert.  Wave 0 of a block runs the selection and stops after
// round k (one selecting wave per block: every block of the row repeats the
// same selection, so it is kept off the other waves' SIMDs, and at raised
// priority, ahead of other blocks' dequantisation), so the rows of the first
// picks stream their weights while the later picks are still being selected;
// wave 1 meanwhile stages x in LDS.  The block at (0, K - 1) runs every round
// and writes ids and weights as moe_router_topk does.
template <int QF, int PL, int RPW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(waves_per_simd(MOE_ACT_BF16, 1, 1)))) void
k_fused_gateup1(RouterArgs r, FfnArgs a) {
  __shared__ int32_t s_pick[64];  // expert id of each selection round
  __shared__ XLds xs;
  const int K = a.K;
  const int y = blockIdx.y;
  const bool shared = y == K;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rbase = (blockIdx.x * 4 + wave) * RPW;
  RowTile<QF, RPW, 1> tg, tu;
  if (shared) {  // no selection: the weights go out first
    const bool keep = hot_expert(a, true, 0);
    tg.load(expert_view<QF>(a.sgate, 0, a.I, a.H, keep), rbase, 0, 1, a.I, lane, 64);
    tu.load(expert_view<QF>(a.sup, 0, a.I, a.H, keep), rbase, 0, 1, a.I, lane, 64);
  }
  if (wave == 1) stage_x1<QF>(a.x, a.H, lane, xs);
  if (!shared && wave == 0) {
    __builtin_amdgcn_s_setprio(3);
    LaneSorted<PL> ls;
    ls.load(r.logits, r.E, lane);
    uint32_t mine = 0, top = 0;  // lane k keeps the key of round k
#pragma unroll
    for (int k = 0; k < kFusedMaxK1; ++k) {  // unrolled: the candidate registers stay in place
      if (k <= y) {
        const uint32_t m = ls.round(lane, k, s_pick);
        if (k == 0) top = m;
        if (lane == k) mine = m;
      }
    }
    if (blockIdx.x == 0 && y == K - 1) {
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      write_topk(mine, s_pick[min(lane, K - 1)], top, K, lane, r.ids, r.wts);
    }
    __builtin_amdgcn_s_setprio(0);
  }
  __syncthreads();
  if (!shared) {
    const int e = __builtin_amdgcn_readfirstlane(s_pick[y]);
    const bool keep = hot_expert(a, false, e);
    tg.load(expert_view<QF>(a.gate, e, a.I, a.H, keep), rbase, 0, 1, a.I, lane, 64);
    tu.load(expert_view<QF>(a.up, e, a.I, a.H, keep), rbase, 0, 1, a.I, lane, 64);
  }
  gateup_rows1<QF, RPW>(a, shared, shared ? 0 : y, rbase, lane, tg, tu, xs);
}

// ---- one token, down projection -------------------------------------------
// 8 lanes per row (8 rows per wave instruction), lane sub of a row owning the
// groups sub + 8 j (j < GPL, GPL = ceil(I / 256)): no lane idles at I = 768.
// Each wave works on SPW slots (slot = wave + NW js, NW waves per block; the
// shared expert is slot K).  It stages the h of its own slots in its LDS region first (prepared
// once per (slot, group) instead of once per row group), then reads the
// weights' groups against it.  A slot's dot product is accumulated in the
// lane over j, then reduced over the row's 8 lanes with three DPP steps.
// The standalone and the fused kernels share this code, so their o values
// are the same bits.
constexpr int kDownLpr1 = 8;
constexpr int kDown1MaxWaves = 16;  // waves per block: one per slot up to 16 slots

// LDS words of one wave's staged h (16 words of pairs + the offset term per
// (slot, group)), rounded up to 16 bytes; a block holds one per wave
__host__ __device__ constexpr int down1_wave_words(int spw, int G) { return (17 * spw * G + 3) & ~3; }

template <int QF, int SPW, int GPL>
struct Down1Wave {
  RowTile<QF, 1, GPL> tw[SPW];
  uint4* q;   // this wave's staged h: q[(js * 4 + i) * G + g]
  float* c;   //                       c[js * G + g]
  int G;

  // stage h rows hrow[js] (of hs when sh[js]) and request the weight rows of
  // experts e[js]; the h loads go out first (they do not wait on the ids).
  __device__ __forceinline__ void load(const FfnArgs& a, const int (&hrow)[SPW], const bool (&sh)[SPW],
                                       const int (&e)[SPW], int rbase, int lane, uint32_t* lds) {
    G = a.I / kGroup;
    q = reinterpret_cast<uint4*>(lds);
    c = reinterpret_cast<float*>(lds + 16 * SPW * G);
    constexpr int kRounds = (SPW * 32 + 63) / 64;  // items per lane (G <= 32)
    XGroup<QF, MOE_ACT_BF16> xg[kRounds];
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const int it = min(lane + 64 * r, SPW * G - 1);  // clamped: items past the end repeat the last
      const int js = it / G, g = it - js * G;
      // js is not uniform: pick the row by selects over the wave's slots
      int row = hrow[0];
      bool s0 = sh[0];
#pragma unroll
      for (int k = 1; k < SPW; ++k) { row = js == k ? hrow[k] : row; s0 = js == k ? sh[k] : s0; }
      xg[r].load_raw(s0 ? a.hs : a.h, (size_t)row * a.I + (size_t)g * kGroup);
    }
    // keep the h loads ahead of the weight loads: loads complete in order, so
    // h can then be staged while the weight rows are still in flight
    __builtin_amdgcn_sched_barrier(0);
    const int rsub = lane >> 3, sub = lane & 7;
#pragma unroll
    for (int js = 0; js < SPW; ++js)
      tw[js].load(expert_view<QF>(sh[js] ? a.sdown : a.down, e[js], a.H, a.I, hot_expert(a, sh[js], e[js])), rbase,
                  rsub, kDownLpr1, a.H, sub,
                  kDownLpr1);
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const int it = lane + 64 * r;
      xg[r].prep();
      if (it < SPW * G) {
        const int js = it / G, g = it - js * G;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          q[(js * 4 + i) * G + g] = make_uint4(xg[r].p[4 * i], xg[r].p[4 * i + 1], xg[r].p[4 * i + 2], xg[r].p[4 * i + 3]);
        c[js * G + g] = xg[r].c;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  }

  // o of slot js for the lane's row (every lane of the row gets it)
  __device__ __forceinline__ float dot(int js, int lane) const {
    const int sub = lane & 7;
    float acc = 0.f;
#pragma unroll
    for (int gi = 0; gi < GPL; ++gi) {
      const int g = min(sub + 8 * gi, G - 1);
      XGroup<QF, MOE_ACT_BF16> xg;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = q[(js * 4 + i) * G + g];
        xg.p[4 * i] = v.x; xg.p[4 * i + 1] = v.y; xg.p[4 * i + 2] = v.z; xg.p[4 * i + 3] = v.w;
      }
      xg.c = c[js * G + g];
      xg.sx = xg.c;
      const float v = group_acc<QF, MOE_ACT_BF16>(acc, tw[js].c[0][gi], tw[js].s[0][gi], tw[js].m[0][gi], xg);
      acc = sub + 8 * gi < G ? v : acc;
    }
    acc += dpp_f<kDppXor1>(acc);
    acc += dpp_f<kDppXor2>(acc);
    acc += dpp_f<kDppHalfMirror>(acc);
    return acc;
  }
};

// One token: down projection of the shared expert and the K selected experts
// for the block's 8 rows, combined in slot order:
//   y[r] = o_shared[r] + sum_k w[k] o_k[r]   (the arithmetic of k_down1 + k_combine)
// h holds the routed rows in slot order (row k: the expert of slot k), as
// k_fused_gateup1 writes them.  The slots are split over the block's waves;
// the per-slot o values meet in LDS and 8 threads combine them.  The routing
// values are read with scalar loads.
template <int QF, int SPW, int GPL>
__global__ __launch_bounds__(64 * kDown1MaxWaves) void k_fused_down1(FfnArgs a, CombineArgs c) {
  const int NW = blockDim.x >> 6;  // slot = wave + NW js
  extern __shared__ __align__(16) uint32_t lds_d1[];
  __shared__ float s_o[kDown1MaxWaves * SPW][8];  // [slot][row of the block]
  __shared__ float s_w[kDown1MaxWaves * SPW];     // combine weights
  const int K = a.K;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rbase = blockIdx.x * 8;
  const bool has_shared = a.so != nullptr;
  const int nslots = K + (has_shared ? 1 : 0);
  // the combine's inputs are requested now and used after the products; the
  // loads are branch-free (clamped indices) and their values stay untouched
  // until the weights are requested, so no wave waits for them first
  const float wv = c.w[min((int)threadIdx.x, K - 1)];
  // bf16 bits of the residual of row rbase + threadIdx.x % 8 (without a
  // residual, a word of the weights stands in, unused)
  const uint16_t* rp = c.x_next ? reinterpret_cast<const uint16_t*>(c.x_resid) : reinterpret_cast<const uint16_t*>(c.w);
  const uint32_t rraw = rp[c.x_next ? min(rbase + (int)(threadIdx.x & 7), a.H - 1) : 0];
  int hrow[SPW], e[SPW];
  bool sh[SPW];
#pragma unroll
  for (int js = 0; js < SPW; ++js) {
    const int slot = min(wave + NW * js, nslots - 1);  // clamped: slots past the end are computed but unused
    sh[js] = has_shared && slot == K;
    hrow[js] = sh[js] ? 0 : slot;
    e[js] = sh[js] ? 0 : __builtin_amdgcn_readfirstlane(a.ids[min(slot, K - 1)]);
  }
  Down1Wave<QF, SPW, GPL> dw;
  dw.load(a, hrow, sh, e, rbase, lane, lds_d1 + wave * down1_wave_words(SPW, a.I / kGroup));
  if (threadIdx.x < K) s_w[threadIdx.x] = wv;
#pragma unroll
  for (int js = 0; js < SPW; ++js) {
    const int slot = wave + NW * js;
    const float o = dw.dot(js, lane);
    if (slot < nslots && (lane & 7) == 0) s_o[slot][lane >> 3] = o;
  }
  __syncthreads();
  if (threadIdx.x < 8) {
    const int i = threadIdx.x, r = rbase + i;
    float acc = has_shared ? s_o[K][i] : 0.f;
    for (int k = 0; k < K; ++k) acc = fmaf(s_w[k], s_o[k][i], acc);
    if (r < a.H) {
      c.y[r] = acc;
      if (c.x_next) store_act<MOE_ACT_BF16>(c.x_next, r, bf16_to_f32(rraw) + acc);
    }
  }
}

// Standalone down projection for one token (moe_expert_down_q, T = 1): wave
// slots as above; pair k reads h row pair_pos[k] and writes o row pair_pos[k]
// (the rank of (ids[k], k), from one load of the ids), the shared expert hs
// and so.
template <int QF, int SPW, int GPL>
__global__ __launch_bounds__(64 * kDown1MaxWaves) void k_down1(FfnArgs a) {
  const int NW = blockDim.x >> 6;  // slot = wave + NW js
  extern __shared__ __align__(16) uint32_t lds_d1[];
  const int K = a.K;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rbase = blockIdx.x * 8;
  const bool has_shared = a.so != nullptr;
  const int nslots = K + (has_shared ? 1 : 0);
  const int id = a.ids[min(lane, K - 1)];
  int hrow[SPW], e[SPW];
  bool sh[SPW];
#pragma unroll
  for (int js = 0; js < SPW; ++js) {
    const int slot = min(wave + NW * js, nslots - 1);
    sh[js] = has_shared && slot == K;
    const int ek = __builtin_amdgcn_readlane(id, min(slot, K - 1));
    e[js] = sh[js] ? 0 : ek;
    hrow[js] = sh[js] ? 0 : (int)__popcll(__ballot(lane < K && (id < ek || (id == ek && lane < slot))));
  }
  Down1Wave<QF, SPW, GPL> dw;
  dw.load(a, hrow, sh, e, rbase, lane, lds_d1 + wave * down1_wave_words(SPW, a.I / kGroup));
  const int r = rbase + (lane >> 3);
#pragma unroll
  for (int js = 0; js < SPW; ++js) {
    const int slot = wave + NW * js;
    const float o = dw.dot(js, lane);
    if (slot < nslots && (lane & 7) == 0 && r < a.H) (sh[js] ? a.so : a.o)[(size_t)hrow[js] * a.H + r] = o;
  }
}

bool down1_ok(const FfnArgs& a) {
  return a.T == 1 && a.act == MOE_ACT_BF16 && a.I <= 32 * kGroup && a.K + 1 <= kDown1MaxWaves * 2;
}

bool fused_decode_ok(int T, int K, int E, int H, int I, int act) {
  return act == MOE_ACT_BF16 && T == 1 && T * K <= kFusedMaxPairs && K <= 64 && E <= 64 * kRegLogits && H <= 64 * kGroup &&
         I <= 64 * kGroup;
}

// One token through k_fused_gateup1 (selection state in LaneSorted: E <= 512)
// and k_fused_down1, with h in slot order between them.
bool fused_down1_ok(int T, int K, int E, int I) { return T == 1 && K <= kFusedMaxK1 && E <= 512 && I <= 32 * kGroup; }

template <int QF>
static hipError_t fused_gateup_pl(const RouterArgs& r, const PermuteArgs& pm, const FfnArgs& a, hipStream_t s) {
  int lpr_log2, gpl;
  lane_split(a.H, &lpr_log2, &gpl);
  const int rpi = 64 >> lpr_log2;
  // one token (fused_decode_ok): 2 rows per wave (twice the blocks, each with
  // less to stream after its routing)
  const int rows_per_block = 4 * kFusedRpw1 * rpi;
  const dim3 grid((a.I + rows_per_block - 1) / rows_per_block, a.T * a.K + (a.n_shared && a.hs ? 1 : 0));
  const int pl = regs_per_lane(a.E);
  if (fused_down1_ok(a.T, a.K, a.E, a.I)) {  // h in slot order for k_fused_down1
    // one group of H per lane, kFusedRpw1 rows per wave
    const dim3 grid1((a.I + 4 * kFusedRpw1 - 1) / (4 * kFusedRpw1), a.K + (a.n_shared && a.hs ? 1 : 0));
    auto go1 = [&](auto kern) { kern<<<grid1, 256, 0, s>>>(r, a); };
    switch (pl) {
      case 1: go1(k_fused_gateup1<QF, 1, kFusedRpw1>); break;
      case 2: go1(k_fused_gateup1<QF, 2, kFusedRpw1>); break;
      case 4: go1(k_fused_gateup1<QF, 4, kFusedRpw1>); break;
      default: go1(k_fused_gateup1<QF, 8, kFusedRpw1>); break;
    }
    return hipGetLastError();
  }
  // one token with K > 16 or E > 512: the general form (selection per block
  // row, h in sorted order for the down and combine launches)
  auto go = [&](auto kern) { kern<<<grid, 256, 0, s>>>(r, pm, a, lpr_log2); };
  switch (pl) {
    case 1: go(k_fused_gateup<QF, 1, 1, kFusedRpw1>); break;
    case 2: go(k_fused_gateup<QF, 1, 2, kFusedRpw1>); break;
    case 4: go(k_fused_gateup<QF, 1, 4, kFusedRpw1>); break;
    case 8: go(k_fused_gateup<QF, 1, 8, kFusedRpw1>); break;
    default: go(k_fused_gateup<QF, 1, 16, kFusedRpw1>); break;
  }
  return hipGetLastError();
}

hipError_t launch_fused_gateup(const RouterArgs& r, const PermuteArgs& pm, const FfnArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  return by_qfmt(a.qfmt, [&](auto q) { return fused_gateup_pl<decltype(q)::value>(r, pm, a, s); });
}

// one wave per slot up to 16 slots (SPW = 1), else two slots per wave;
// GPL groups per lane (<= 4)
#define MOE_DOWN1_DISPATCH(KERN, ...)                                                         \
  do {                                                                                        \
    const int G_ = a.I / kGroup, gpl_ = (G_ + kDownLpr1 - 1) / kDownLpr1;                     \
    const int nslots_ = a.K + (a.so ? 1 : 0);                                                 \
    const int spw_ = nslots_ <= kDown1MaxWaves ? 1 : 2;                                       \
    const int nw_ = (nslots_ + spw_ - 1) / spw_;                                              \
    const dim3 grid_((a.H + 7) / 8);                                                          \
    auto go_ = [&](auto kern, int spw) {                                                      \
      kern<<<grid_, 64 * nw_, (size_t)nw_ * down1_wave_words(spw, G_) * 4, s>>>(__VA_ARGS__); \
    };                                                                                        \
    auto by_gpl_ = [&](auto k1, auto k2, auto k3, auto k4, int spw) {                         \
      if (gpl_ <= 1) go_(k1, spw); else if (gpl_ == 2) go_(k2, spw);                          \
      else if (gpl_ == 3) go_(k3, spw); else go_(k4, spw);                                    \
    };                                                                                        \
    if (spw_ == 1) by_gpl_(KERN<QF, 1, 1>, KERN<QF, 1, 2>, KERN<QF, 1, 3>, KERN<QF, 1, 4>, 1); \
    else by_gpl_(KERN<QF, 2, 1>, KERN<QF, 2, 2>, KERN<QF, 2, 3>, KERN<QF, 2, 4>, 2);           \
  } while (0)

template <int QF>
static hipError_t fused_down1_q(const FfnArgs& a, const CombineArgs& c, hipStream_t s) {
  MOE_DOWN1_DISPATCH(k_fused_down1, a, c);
  return hipGetLastError();
}

template <int QF>
static hipError_t down1_q(const FfnArgs& a, hipStream_t s) {
  MOE_DOWN1_DISPATCH(k_down1, a);
  return hipGetLastError();
}

hipError_t launch_fused_down1(const FfnArgs& a, const CombineArgs& c, hipStream_t s) {
  return by_qfmt(a.qfmt, [&](auto q) { return fused_down1_q<decltype(q)::value>(a, c, s); });
}

}  // namespace moe
