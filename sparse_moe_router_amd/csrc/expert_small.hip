// Expert SwiGLU FFNs for small batches (a few tokens per expert: speculative
// verify, batched decode, the stack at batch 8), with in-register dequant
// (low-bit weights: page 1 "How Strata Makes the Impossible Possible"; SwiGLU
// expert sub-networks: page 2 "Layer 1"; shared expert: page 5).
//
// Work row y is sorted position y (the pairs sorted by expert, as
// moe_permute orders them) and works only if y is its expert's first
// position; then it owns all of the expert's tokens (sorted positions y ..
// y + n - 1).  With the small-batch routing's work list, row y is instead the
// y-th distinct expert.  Work row T K is the shared expert (all T tokens),
// dispatched first.  The expert's weight rows are loaded once; the tokens'
// activations are staged in LDS, prepared, chunk by chunk.  Both kernels
// unpack the codes once for all the tokens.
#include "gemv_one.h"

namespace moe {

constexpr int kSbTok = 8;  // tokens staged per chunk
constexpr int kSbRpw = 2;  // gate/up rows per wave
constexpr int kSbLpr = 8;  // down: lanes per row
constexpr int kSbMaxPairs = 256;  // T K of the small-batch path (one block row per sorted position)

// The expert of block row y: first sorted position lo and token count n, or
// false when y is not the first position of its expert.  Shared row: y == ny.
// With the routing's work list, block row y takes its u = y-th distinct
// expert instead (one load, and the rows past the last expert exit at once).
__device__ __forceinline__ bool sb_work(const FfnArgs& a, int ny, int y, int* expert, int* lo, int* n) {
  if (y == ny) {
    *expert = -1; *lo = 0; *n = a.T;
    return !on_mfma(a, a.T);
  }
  if (a.work) {
    const int4 w = reinterpret_cast<const int4*>(a.work)[y];
    if (w.x < 0) return false;
    *expert = w.x; *lo = w.y; *n = w.z;
    return !on_mfma(a, w.z);
  }
  const int p = a.sorted_pairs[y];
  const int pp = y > 0 ? a.sorted_pairs[y - 1] : p;
  const int e = a.ids[p];
  if (y > 0 && a.ids[pp] == e) return false;
  *expert = e; *lo = y; *n = a.offsets[e + 1] - y;
  return !on_mfma(a, *n);  // the grouped GEMM takes an expert with many tokens
}

// Block row of the grid -> work row: the shared expert's row (ny), which has
// every token, goes first in dispatch order, then the experts' rows.
__device__ __forceinline__ int sb_row(int ny) {
  return (int)gridDim.y > ny ? ((int)blockIdx.y == 0 ? ny : (int)blockIdx.y - 1) : (int)blockIdx.y;
}

// token of the expert's jj-th sorted position
__device__ __forceinline__ int sb_token(const FfnArgs& a, bool shared, int lo, int jj) {
  return shared ? jj : a.sorted_tok ? a.sorted_tok[lo + jj] : a.sorted_pairs[lo + jj] / a.K;
}

// gate/up + SwiGLU: wave w owns rows (blockIdx.x * 4 + w) * RPW .. + RPW - 1
// of gate and up, one 32-element group of H per lane (H <= 2048).
template <int QF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_gateup_sb(FfnArgs a, int ny) {
  __shared__ XLds xs[kSbTok];
  constexpr int RPW = kSbRpw;
  static_assert(kSbTok == 8, "the first chunk is two tokens per wave");
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int y = sb_row(ny);
  // tokens of the first chunk's positions y + wave and y + wave + 4, read
  // with the expert lookup (clamped in range; used only below the count);
  // with a work list, from the expert's first position once it is known
  int tok0[2];
#pragma unroll
  for (int k = 0; k < 2; ++k)
    tok0[k] = y == ny || a.work ? wave + 4 * k : a.sorted_pairs[min(y + wave + 4 * k, ny - 1)] / a.K;
  int e, lo, n;
  if (!sb_work(a, ny, y, &e, &lo, &n)) return;
  const bool shared = e < 0;
  if (a.work && !shared) {
#pragma unroll
    for (int k = 0; k < 2; ++k) tok0[k] = a.sorted_tok[lo + min(wave + 4 * k, n - 1)];
  }
  const int rbase = (blockIdx.x * 4 + wave) * RPW;
  // the first chunk's activations go out before the weight rows: loads
  // complete in order, so they are staged while the weights are in flight
  const int nc0 = min(kSbTok, n);
  XGroup<QF, MOE_ACT_BF16> x0[2];
#pragma unroll
  for (int k = 0; k < 2; ++k)
    if (wave + 4 * k < nc0) load_x1<QF>(reinterpret_cast<const uint16_t*>(a.x) + (size_t)tok0[k] * a.H, a.H, lane, x0[k]);
  RowTile<QF, RPW, 1> tg, tu;
  const bool keep = hot_expert(a, shared, e);
  tg.load(expert_view<QF>(shared ? a.sgate : a.gate, shared ? 0 : e, a.I, a.H, keep), rbase, 0, 1, a.I, lane, 64);
  tu.load(expert_view<QF>(shared ? a.sup : a.up, shared ? 0 : e, a.I, a.H, keep), rbase, 0, 1, a.I, lane, 64);
#pragma unroll
  for (int k = 0; k < 2; ++k)
    if (wave + 4 * k < nc0) put_x1<QF>(x0[k], lane, xs[wave + 4 * k]);
  __syncthreads();
  const bool gok = lane < a.H / kGroup;
  // the codes are unpacked once for all the expert's tokens (the block keeps
  // four waves per SIMD with them unpacked)
  uint32_t bg[RPW][16], bu[RPW][16];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    unpack_group<QF>(tg.c[rr][0], bg[rr]);
    unpack_group<QF>(tu.c[rr][0], bu[rr]);
  }
  void* out = shared ? a.hs : a.h;
  for (int c0 = 0; c0 < n; c0 += kSbTok) {
    const int nc = min(kSbTok, n - c0);
    if (c0 > 0) {
      __syncthreads();  // the previous chunk's readers are done
      for (int j = wave; j < nc; j += 4) stage_x1<QF>(reinterpret_cast<const uint16_t*>(a.x) +
                                                          (size_t)sb_token(a, shared, lo, c0 + j) * a.H, a.H, lane, xs[j]);
      __syncthreads();
    }
    for (int j = 0; j < nc; ++j) {
      XGroup<QF, MOE_ACT_BF16> xg;
      read_x1<QF>(xs[j], lane, xg);
      float v[2 * RPW];
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr) {
        __builtin_amdgcn_sched_barrier(0);
        const float gv = group_acc_unpacked<QF>(0.f, bg[rr], tg.s[rr][0], tg.m[rr][0], xg);
        const float uv = group_acc_unpacked<QF>(0.f, bu[rr], tu.s[rr][0], tu.m[rr][0], xg);
        v[rr] = gok ? gv : 0.f;
        v[RPW + rr] = gok ? uv : 0.f;
      }
      float g, u;
      reduce_gu1<RPW>(v, lane, &g, &u);
      constexpr int kStride = 32 / RPW;
      const int r = rbase + lane / kStride;
      if (lane < 32 && (lane & (kStride - 1)) == 0 && r < a.I)
        store_act<MOE_ACT_BF16>(out, (size_t)(lo + c0 + j) * a.I + r, silu(g) * u);
    }
  }
}

// down projection, fp32 out: 8 lanes per row (8 rows per wave, 32 per
// block), lane sub of a row owning the groups sub + 8 j (j < GPL, I <= 1024).
// h of each chunk of tokens is staged in LDS, prepared: [token][4][G] uint4
// pairs and [token][G] offset terms.
template <int QF, int GPL>
__global__ __launch_bounds__(256) void k_down_sb(FfnArgs a, int ny) {
  extern __shared__ __align__(16) uint32_t lds_sb[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int e, lo, n;
  if (!sb_work(a, ny, sb_row(ny), &e, &lo, &n)) return;
  const bool shared = e < 0;
  const int G = a.I / kGroup;
  uint4* hq = reinterpret_cast<uint4*>(lds_sb);             // [kSbTok][4][G]
  float* hc = reinterpret_cast<float*>(lds_sb + kSbTok * 16 * G);  // [kSbTok][G]
  const int rsub = lane >> 3, sub = lane & 7;
  const int rbase = (blockIdx.x * 4 + wave) * 8;
  const void* hin = shared ? a.hs : a.h;
  float* out = shared ? a.so : a.o;
  // one (token, group) item of h per thread and chunk (G <= 32, so a chunk
  // has at most 256 items); the first chunk's h goes out before the weight
  // rows, so it is staged while they are in flight
  auto put_h = [&](int it, XGroup<QF, MOE_ACT_BF16>& hg) {
    const int j = it / G, g = it - j * G;
    hg.prep();
#pragma unroll
    for (int i = 0; i < 4; ++i) hq[(j * 4 + i) * G + g] = make_uint4(hg.p[4 * i], hg.p[4 * i + 1], hg.p[4 * i + 2], hg.p[4 * i + 3]);
    hc[j * G + g] = hg.c;
  };
  const int it = threadIdx.x;
  XGroup<QF, MOE_ACT_BF16> h0;
  const bool item0 = it < min(kSbTok, n) * G;
  if (item0) h0.load_raw(hin, (size_t)(lo + it / G) * a.I + (size_t)(it % G) * kGroup);
  RowTile<QF, 1, GPL> tw;
  tw.load(expert_view<QF>(shared ? a.sdown : a.down, shared ? 0 : e, a.H, a.I, hot_expert(a, shared, e)), rbase,
          rsub, kSbLpr, a.H, sub, kSbLpr);
  if (item0) put_h(it, h0);
  __syncthreads();
  uint32_t b[GPL][16];
  bool unpacked = false;
  const int r = rbase + rsub;
  for (int c0 = 0; c0 < n; c0 += kSbTok) {
    const int nc = min(kSbTok, n - c0);
    if (c0 > 0) {
      __syncthreads();  // the previous chunk's readers are done
      if (it < nc * G) {
        XGroup<QF, MOE_ACT_BF16> hg;
        hg.load_raw(hin, (size_t)(lo + c0 + it / G) * a.I + (size_t)(it % G) * kGroup);
        put_h(it, hg);
      }
      __syncthreads();
    }
    if (!unpacked) {
#pragma unroll
      for (int gi = 0; gi < GPL; ++gi) unpack_group<QF>(tw.c[0][gi], b[gi]);
      unpacked = true;
    }
    for (int j = 0; j < nc; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int gi = 0; gi < GPL; ++gi) {
        const int g = min(sub + 8 * gi, G - 1);
        XGroup<QF, MOE_ACT_BF16> hg;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 v = hq[(j * 4 + i) * G + g];
          hg.p[4 * i] = v.x; hg.p[4 * i + 1] = v.y; hg.p[4 * i + 2] = v.z; hg.p[4 * i + 3] = v.w;
        }
        hg.c = hc[j * G + g];
        hg.sx = hg.c;
        const float v = group_acc_unpacked<QF>(acc, b[gi], tw.s[0][gi], tw.m[0][gi], hg);
        acc = sub + 8 * gi < G ? v : acc;
      }
      acc += dpp_f<kDppXor1>(acc);
      acc += dpp_f<kDppXor2>(acc);
      acc += dpp_f<kDppHalfMirror>(acc);
      if (sub == 0 && r < a.H) out[(size_t)(lo + c0 + j) * a.H + r] = acc;
    }
  }
}

// Layer forward with the small-batch routing's work list: down projection
// fused with the weighted combine.  A block owns 8 output rows of every
// distinct expert and of the shared expert, so each token's slots meet in the
// block and o never leaves it.  All h rows (the T K sorted rows, then the T
// shared rows) are staged in LDS, prepared, once per block, while the weight
// rows are in flight.  Wave w takes the work entries w + NW (kFdsEpb b + i)
// (entry 0: the shared expert, entry u + 1: the u-th distinct expert).  The
// products have the lane split and the arithmetic of k_down_sb, the combine
// the order of k_combine (shared first, then slots 0..K-1), so y has the same
// bits as the step-by-step calls.
constexpr int kFdsWaves = 16;
constexpr int kFdsEpb = 2;     // work entries per wave per batch
constexpr int kFdsRounds = 3;  // staged (row, group) items per thread
constexpr int kFdsTok = 8;     // tokens of an entry per pass over its groups
// At most 128 KiB of staged h (T (K + 1) <= 77 rows at I = 768): the block's
// products run after its h and weights have landed, and past about 80 rows
// (T = 8, K = 10) they cost what the saved combine launch gains.
constexpr size_t kFdsMaxLds = 128 * 1024;

// dynamic LDS bytes: prepared h (17 words per row and group), the block's
// o rows, and the pair -> sorted row map and combine weights
static size_t fds_lds_bytes(int n, int nh, int G) { return (size_t)nh * (68 * G + 32) + (size_t)n * 8; }

template <int QF, int GPL>
__global__ __launch_bounds__(64 * kFdsWaves) void k_fused_down_sb(FfnArgs a, CombineArgs c) {
  extern __shared__ __align__(16) uint32_t lds_fds[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool has_shared = a.so != nullptr;
  const int n = a.T * a.K, nh = n + (has_shared ? a.T : 0), ns = has_shared ? 1 : 0;
  const int G = a.I / kGroup;
  uint4* hq = reinterpret_cast<uint4*>(lds_fds);                   // [nh][4][G]
  float* hc = reinterpret_cast<float*>(lds_fds + nh * 16 * G);     // [nh][G]
  float* s_o = hc + nh * G;                                          // [nh][8]
  int32_t* s_pos = reinterpret_cast<int32_t*>(s_o + nh * 8);         // [n]
  float* s_w = reinterpret_cast<float*>(s_pos + n);                  // [n]
  const int rbase = blockIdx.x * 8;
  const int rsub = lane >> 3, sub = lane & 7;
  // this wave's work entries of a batch; then the combine's inputs and the
  // h rows are requested (neither waits on the work list; clamped indices
  // keep the loads out of conditionals), then the entries' weight rows
  int e[kFdsEpb], lo[kFdsEpb], cnt[kFdsEpb];
  bool ok[kFdsEpb];
  RowTile<QF, 1, GPL> tw[kFdsEpb];
  auto fetch_work = [&](int b) {
#pragma unroll
    for (int i = 0; i < kFdsEpb; ++i) {
      const int j = (kFdsEpb * b + i) * kFdsWaves + wave;
      const bool sh = has_shared && j == 0;
      const int4 wk = reinterpret_cast<const int4*>(a.work)[min(max(j - ns, 0), n - 1)];
      ok[i] = sh || (j - ns < n && wk.x >= 0);
      e[i] = sh ? -1 : wk.x;
      lo[i] = sh ? n : wk.y;
      cnt[i] = sh ? a.T : wk.z;
    }
  };
  auto fetch_weights = [&] {
#pragma unroll
    for (int i = 0; i < kFdsEpb; ++i) {
      const bool sh = e[i] < 0;
      if (ok[i])
        tw[i].load(expert_view<QF>(sh ? a.sdown : a.down, sh ? 0 : e[i], a.H, a.I, hot_expert(a, sh, e[i])), rbase,
                   rsub, kSbLpr, a.H, sub, kSbLpr);
    }
  };
  fetch_work(0);
  const int p = min((int)threadIdx.x, n - 1);
  const int32_t pos_v = c.pair_pos[p];
  const float w_v = c.w[p];
  XGroup<QF, MOE_ACT_BF16> hg[kFdsRounds];
#pragma unroll
  for (int r = 0; r < kFdsRounds; ++r) {
    const int it = min((int)threadIdx.x + 64 * kFdsWaves * r, nh * G - 1);
    const int row = it / G, g = it - row * G;
    const bool sh = row >= n;
    hg[r].load_raw(sh ? a.hs : a.h, (size_t)(sh ? row - n : row) * a.I + (size_t)g * kGroup);
  }
  fetch_weights();
#pragma unroll
  for (int r = 0; r < kFdsRounds; ++r) {
    const int it = (int)threadIdx.x + 64 * kFdsWaves * r;
    if (it < nh * G) {
      const int row = it / G, g = it - row * G;
      hg[r].prep();
#pragma unroll
      for (int i = 0; i < 4; ++i)
        hq[(row * 4 + i) * G + g] = make_uint4(hg[r].p[4 * i], hg[r].p[4 * i + 1], hg[r].p[4 * i + 2], hg[r].p[4 * i + 3]);
      hc[row * G + g] = hg[r].c;
    }
  }
  if ((int)threadIdx.x < n) {
    s_pos[threadIdx.x] = pos_v;
    s_w[threadIdx.x] = w_v;
  }
  __syncthreads();
  for (int b = 0;; ++b) {
    if (b > 0) {
      if (!ok[kFdsEpb - 1]) break;  // entries are dense: this wave has no more
      fetch_work(b);
      fetch_weights();
    }
    if (!ok[0]) break;
#pragma unroll
    for (int i = 0; i < kFdsEpb; ++i) {
      if (!ok[i]) continue;
      // up to kFdsTok tokens per pass: one group's codes unpacked at a time,
      // each token's sum still taken over the groups in order
      for (int j0 = 0; j0 < cnt[i]; j0 += kFdsTok) {
        const int nj = min(kFdsTok, cnt[i] - j0);
        float acc[kFdsTok];
#pragma unroll
        for (int jj = 0; jj < kFdsTok; ++jj) acc[jj] = 0.f;
#pragma unroll
        for (int gi = 0; gi < GPL; ++gi) {
          uint32_t bw[16];
          unpack_group<QF>(tw[i].c[0][gi], bw);
          const int g = min(sub + 8 * gi, G - 1);
#pragma unroll
          for (int jj = 0; jj < kFdsTok; ++jj) {
            if (jj < nj) {
              const int row = lo[i] + j0 + jj;
              XGroup<QF, MOE_ACT_BF16> xg;
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const uint4 v = hq[(row * 4 + q) * G + g];
                xg.p[4 * q] = v.x; xg.p[4 * q + 1] = v.y; xg.p[4 * q + 2] = v.z; xg.p[4 * q + 3] = v.w;
              }
              xg.c = hc[row * G + g];
              xg.sx = xg.c;
              const float v = group_acc_unpacked<QF>(acc[jj], bw, tw[i].s[0][gi], tw[i].m[0][gi], xg);
              acc[jj] = sub + 8 * gi < G ? v : acc[jj];
            }
          }
        }
#pragma unroll
        for (int jj = 0; jj < kFdsTok; ++jj) {
          if (jj < nj) {
            float v = acc[jj];
            v += dpp_f<kDppXor1>(v);
            v += dpp_f<kDppXor2>(v);
            v += dpp_f<kDppHalfMirror>(v);
            if (sub == 0) s_o[(lo[i] + j0 + jj) * 8 + rsub] = v;
          }
        }
      }
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < a.T * 8) {
    const int t = threadIdx.x >> 3, i = threadIdx.x & 7, r = rbase + i;
    float acc = has_shared ? s_o[(n + t) * 8 + i] : 0.f;
    for (int k = 0; k < a.K; ++k) acc = fmaf(s_w[t * a.K + k], s_o[s_pos[t * a.K + k] * 8 + i], acc);
    if (r < a.H) {
      const size_t idx = (size_t)t * a.H + r;
      c.y[idx] = acc;
      if (c.x_next) store_act<MOE_ACT_BF16>(c.x_next, idx, load_act<MOE_ACT_BF16>(c.x_resid, idx) + acc);
    }
  }
}

bool fused_down_sb_ok(const FfnArgs& a) {
  // I <= 24 groups: three groups per lane at most (registers of 16 waves)
  if (!a.work || a.T < 2 || a.act != MOE_ACT_BF16 || a.I % kGroup != 0 || a.I > 24 * kGroup) return false;
  if (mfma_split(a) != 0) return false;  // every expert on the GEMV kernels
  const int n = a.T * a.K, nh = n + (a.so ? a.T : 0), G = a.I / kGroup;
  return n <= 64 * kFdsWaves && a.T * 8 <= 64 * kFdsWaves && (int64_t)nh * G <= 64 * kFdsWaves * kFdsRounds &&
         fds_lds_bytes(n, nh, G) <= kFdsMaxLds;
}

hipError_t launch_fused_down_sb(const FfnArgs& a, const CombineArgs& c, hipStream_t s) {
  const int n = a.T * a.K, nh = n + (a.so ? a.T : 0), G = a.I / kGroup, gpl = (G + 7) / 8;
  const dim3 grid((a.H + 7) / 8);
  const size_t lds = fds_lds_bytes(n, nh, G);
  auto go = [&](auto kern) { kern<<<grid, 64 * kFdsWaves, lds, s>>>(a, c); };
  by_qfmt(a.qfmt, [&](auto q) {
    constexpr int QF = decltype(q)::value;
    if (gpl <= 1) go(k_fused_down_sb<QF, 1>); else if (gpl == 2) go(k_fused_down_sb<QF, 2>);
    else go(k_fused_down_sb<QF, 3>);
  });
  return hipGetLastError();
}

bool gateup_sb_ok(const FfnArgs& a) {
  return a.T > 1 && a.T * a.K <= kSbMaxPairs && a.act == MOE_ACT_BF16 && a.H <= 64 * kGroup;
}
// I <= 32 groups: k_down_sb stages one (token, group) item of h per thread
// and chunk (kSbTok tokens x 32 groups = its 256 threads)
static_assert(kSbTok * 32 <= 256, "one h item per thread and chunk");
bool down_sb_ok(const FfnArgs& a) {
  return a.T > 1 && a.T * a.K <= kSbMaxPairs && a.act == MOE_ACT_BF16 && a.I <= 32 * kGroup;
}

hipError_t launch_gateup_sb(const FfnArgs& a, hipStream_t s) {
  const int ny = a.T * a.K;
  const dim3 grid((a.I + 4 * kSbRpw - 1) / (4 * kSbRpw), ny + (a.n_shared && a.hs ? 1 : 0));
  by_qfmt(a.qfmt, [&](auto q) { k_gateup_sb<decltype(q)::value><<<grid, 256, 0, s>>>(a, ny); });
  return hipGetLastError();
}

hipError_t launch_down_sb(const FfnArgs& a, hipStream_t s) {
  const int ny = a.T * a.K;
  const int G = a.I / kGroup, gpl = (G + 7) / 8;
  const dim3 grid((a.H + 31) / 32, ny + (a.n_shared && a.so ? 1 : 0));
  const size_t lds = (size_t)kSbTok * 17 * G * 4;
  auto go = [&](auto kern) { kern<<<grid, 256, lds, s>>>(a, ny); };
  by_qfmt(a.qfmt, [&](auto q) {
    constexpr int QF = decltype(q)::value;
    if (gpl <= 1) go(k_down_sb<QF, 1>); else if (gpl == 2) go(k_down_sb<QF, 2>);
    else if (gpl == 3) go(k_down_sb<QF, 3>); else go(k_down_sb<QF, 4>);
  });
  return hipGetLastError();
}

}  // namespace moe
