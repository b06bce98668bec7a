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
