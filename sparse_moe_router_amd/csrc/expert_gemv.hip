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
//
// Inner product of one group (bf16 activations): each code u becomes the exact
// bf16 number 128 + u by OR-ing it into the mantissa of 0x4300 (=128), two
// codes per 32-bit word, and v_dot2_f32_bf16 multiplies the pair with a pair
// of activations in fp32 (products of an 8-bit code and a bf16 value are exact
// in fp32).  The offset is removed with a per-group constant computed once per
// token:  sum (u - 8) x = sum (128 + u) x - 136 sum x   (4-bit),
//         sum u x       = sum (128 + u) x - 128 sum x   (2-bit),
// and the group scale (and 2-bit minimum) is applied once per group:
//         acc += s * sum(q x)            (4-bit, w = s q)
//         acc += s * sum(u x) + m sum x  (2-bit, w = s u + m).
// Activation pairs are pre-arranged per token to match the code pairs a mask
// and a shift produce: 4-bit word i of a group yields pairs (8i+j, 8i+4+j) for
// j = 0..3 from nibbles j and j+4; 2-bit word i yields pairs (16i+j, 16i+8+j)
// for j = 0..7 from crumbs j and j+8.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

template <int QF> struct CodeOf;
template <> struct CodeOf<MOE_Q4_SYM_G32> { using T = uint4; static constexpr int kBytes = 16; };
template <> struct CodeOf<MOE_Q2_ASYM_G32> { using T = uint2; static constexpr int kBytes = 8; };

// Prepared activations of one 32-element group of one token.
template <int QF, int ACT> struct XGroup;

template <int QF> struct XGroup<QF, MOE_ACT_BF16> {
  uint32_t p[16];  // bf16 pairs matching the code pairs
  float c;         // 136 * sum x (4-bit) or 128 * sum x (2-bit)
  float sx;        // sum x (2-bit only)

  __device__ __forceinline__ void load(const void* base, size_t elem) {
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + elem);
    uint4 q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = src[i];
    if constexpr (QF == MOE_Q4_SYM_G32) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // elements 8i..8i+7 in q[i]
        p[4 * i + 0] = (q[i].x & 0xffffu) | (q[i].z << 16);
        p[4 * i + 1] = (q[i].x >> 16) | (q[i].z & 0xffff0000u);
        p[4 * i + 2] = (q[i].y & 0xffffu) | (q[i].w << 16);
        p[4 * i + 3] = (q[i].y >> 16) | (q[i].w & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {  // elements 16i..16i+7 in q[2i], 16i+8..16i+15 in q[2i+1]
        const uint32_t a[4] = {q[2 * i].x, q[2 * i].y, q[2 * i].z, q[2 * i].w};
        const uint32_t b[4] = {q[2 * i + 1].x, q[2 * i + 1].y, q[2 * i + 1].z, q[2 * i + 1].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          p[8 * i + 2 * m] = (a[m] & 0xffffu) | (b[m] << 16);
          p[8 * i + 2 * m + 1] = (a[m] >> 16) | (b[m] & 0xffff0000u);
        }
      }
    }
    constexpr uint32_t kOff = (QF == MOE_Q4_SYM_G32) ? 0x43084308u : 0x43004300u;  // (136,136) / (128,128)
    float c0 = 0.f, c1 = 0.f, s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      c0 = dot2_bf16(kOff, p[i], c0);
      c1 = dot2_bf16(kOff, p[i + 1], c1);
      if constexpr (QF == MOE_Q2_ASYM_G32) {
        s0 = dot2_bf16(0x3f803f80u, p[i], s0);
        s1 = dot2_bf16(0x3f803f80u, p[i + 1], s1);
      }
    }
    c = c0 + c1;
    sx = s0 + s1;
  }
};

template <int QF> struct XGroup<QF, MOE_ACT_F32> {
  float v[32];
  float sx;
  __device__ __forceinline__ void load(const void* base, size_t elem) {
    const float4* src = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + elem);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 f = src[i];
      v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
      s += (f.x + f.y) + (f.z + f.w);
    }
    sx = s;
  }
};

// sum over the group of q*x (4-bit, q = u - 8) or u*x (2-bit).
template <int QF, int ACT>
__device__ __forceinline__ float group_dot(const typename CodeOf<QF>::T& cw, const XGroup<QF, ACT>& x) {
  if constexpr (ACT == MOE_ACT_BF16) {
    float d0 = 0.f, d1 = 0.f;
    if constexpr (QF == MOE_Q4_SYM_G32) {
      const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        d0 = dot2_bf16((w[i] & 0x000f000fu) | 0x43004300u, x.p[4 * i + 0], d0);
        d1 = dot2_bf16(((w[i] >> 4) & 0x000f000fu) | 0x43004300u, x.p[4 * i + 1], d1);
        d0 = dot2_bf16(((w[i] >> 8) & 0x000f000fu) | 0x43004300u, x.p[4 * i + 2], d0);
        d1 = dot2_bf16(((w[i] >> 12) & 0x000f000fu) | 0x43004300u, x.p[4 * i + 3], d1);
      }
    } else {
      const uint32_t w[2] = {cw.x, cw.y};
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          d0 = dot2_bf16(((w[i] >> (2 * j)) & 0x00030003u) | 0x43004300u, x.p[8 * i + j], d0);
          d1 = dot2_bf16(((w[i] >> (2 * j + 2)) & 0x00030003u) | 0x43004300u, x.p[8 * i + j + 1], d1);
        }
      }
    }
    return (d0 + d1) - x.c;
  } else {
    float d0 = 0.f, d1 = 0.f;
    if constexpr (QF == MOE_Q4_SYM_G32) {
      const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          d0 = fmaf((float)((int)((w[i] >> (4 * j)) & 15u) - 8), x.v[8 * i + j], d0);
          d1 = fmaf((float)((int)((w[i] >> (4 * j + 4)) & 15u) - 8), x.v[8 * i + j + 1], d1);
        }
      }
    } else {
      const uint32_t w[2] = {cw.x, cw.y};
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
          d0 = fmaf((float)((w[i] >> (2 * j)) & 3u), x.v[16 * i + j], d0);
          d1 = fmaf((float)((w[i] >> (2 * j + 2)) & 3u), x.v[16 * i + j + 1], d1);
        }
      }
    }
    return d0 + d1;
  }
}

template <int QF, int ACT>
__device__ __forceinline__ float group_acc(float acc, const typename CodeOf<QF>::T& cw, uint16_t s16, uint16_t m16,
                                           const XGroup<QF, ACT>& x) {
  const float d = group_dot<QF, ACT>(cw, x);
  acc = fmaf(f16_to_f32(s16), d, acc);
  if constexpr (QF == MOE_Q2_ASYM_G32) acc = fmaf(f16_to_f32(m16), x.sx, acc);
  return acc;
}

struct MatView {
  const uint8_t* codes;
  const uint16_t* scales;
  const uint16_t* mins;
  size_t row_bytes;  // code bytes per row
  int groups;        // groups per row
};

template <int QF>
__device__ __forceinline__ MatView expert_view(const QMat& m, int e, int rows, int cols) {
  MatView v;
  v.row_bytes = (size_t)cols * (QF == MOE_Q4_SYM_G32 ? 4 : 2) / 8;
  v.groups = cols / kGroup;
  v.codes = m.codes + (size_t)e * rows * v.row_bytes;
  v.scales = m.scales + (size_t)e * rows * v.groups;
  v.mins = m.mins ? m.mins + (size_t)e * rows * v.groups : nullptr;
  return v;
}

// Which token list a block works on: a routed expert (its slice of the sorted
// pairs) or the shared expert (all tokens).  Routed blocks are found without a
// list of active experts: block y visits sorted positions y, y + ny, ... and
// takes the expert whose slice starts at that position (a binary search of
// expert_offsets gives the expert holding a position; an expert is visited by
// exactly one block, the one whose y matches its first position modulo ny).
struct Work {
  int expert;   // routed expert id, or -1 for the shared expert
  int lo, n;    // sorted positions [lo, lo + n) or tokens [0, n)
};

__device__ __forceinline__ int expert_at(const int32_t* offsets, int E, int pos) {
  int lo = 0, hi = E;  // largest e with offsets[e] <= pos
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= pos) lo = mid; else hi = mid;
  }
  return lo;
}

// Next routed expert for this block at or after sorted position *pos (step
// ny); returns false when the block has none left.
__device__ __forceinline__ bool next_routed(const FfnArgs& a, int ny, int* pos, Work* w) {
  const int n = a.T * a.K;
  for (; *pos < n; *pos += ny) {
    const int e = expert_at(a.offsets, a.E, *pos);
    if (a.offsets[e] == *pos) {
      w->expert = e;
      w->lo = *pos;
      w->n = a.offsets[e + 1] - *pos;
      *pos += ny;
      return true;
    }
  }
  return false;
}

// gate/up + SwiGLU:  h[j][r] = round_act(silu(Wg[r].x_t) * (Wu[r].x_t))
template <int QF, int ACT, int NT, int GPL, int RPW>
__global__ __launch_bounds__(256) void k_gateup(FfnArgs a, int ny, int lpr_log2) {
  using CT = typename CodeOf<QF>::T;
  const bool shared = (int)blockIdx.y == ny;  // the extra last row of blocks
  int pos = blockIdx.y;
  Work wk;
  if (shared) { wk.expert = -1; wk.lo = 0; wk.n = a.T; }
  else if (!next_routed(a, ny, &pos, &wk)) return;
 for (;;) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int LPR = 1 << lpr_log2, RPI = 64 >> lpr_log2;
  const int sub = lane & (LPR - 1), rsub = lane >> lpr_log2;
  const int G = a.H / kGroup;
  const MatView vg = expert_view<QF>(shared ? a.sgate : a.gate, shared ? 0 : wk.expert, a.I, a.H);
  const MatView vu = expert_view<QF>(shared ? a.sup : a.up, shared ? 0 : wk.expert, a.I, a.H);
  void* out = shared ? a.hs : a.h;
  const int r0 = (blockIdx.x * 4 + wave) * RPW * RPI + rsub;

  for (int c0 = 0; c0 < wk.n; c0 += NT) {
    const int nt = min(NT, wk.n - c0);
    XGroup<QF, ACT> xg[NT][GPL];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if (j < nt) {
        const int tok = shared ? c0 + j : a.sorted_pairs[wk.lo + c0 + j] / a.K;
#pragma unroll
        for (int gi = 0; gi < GPL; ++gi) {
          const int g = sub + gi * LPR;
          if (g < G) xg[j][gi].load(a.x, (size_t)tok * a.H + (size_t)g * kGroup);
        }
      }
    }
    // issue every row's loads before any arithmetic
    CT cg[RPW][GPL], cu[RPW][GPL];
    uint16_t sg[RPW][GPL], su[RPW][GPL], mg[RPW][GPL], mu[RPW][GPL];
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      const int r = r0 + rr * RPI;
#pragma unroll
      for (int gi = 0; gi < GPL; ++gi) {
        const int g = sub + gi * LPR;
        if (r < a.I && g < G) {
          cg[rr][gi] = *reinterpret_cast<const CT*>(vg.codes + (size_t)r * vg.row_bytes + (size_t)g * CodeOf<QF>::kBytes);
          cu[rr][gi] = *reinterpret_cast<const CT*>(vu.codes + (size_t)r * vu.row_bytes + (size_t)g * CodeOf<QF>::kBytes);
          sg[rr][gi] = vg.scales[(size_t)r * G + g];
          su[rr][gi] = vu.scales[(size_t)r * G + g];
          if constexpr (QF == MOE_Q2_ASYM_G32) {
            mg[rr][gi] = vg.mins[(size_t)r * G + g];
            mu[rr][gi] = vu.mins[(size_t)r * G + g];
          } else {
            mg[rr][gi] = 0; mu[rr][gi] = 0;
          }
        }
      }
    }
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      const int r = r0 + rr * RPI;
      float ga[NT], ua[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) { ga[j] = 0.f; ua[j] = 0.f; }
#pragma unroll
      for (int gi = 0; gi < GPL; ++gi) {
        const int g = sub + gi * LPR;
        if (r < a.I && g < G) {
#pragma unroll
          for (int j = 0; j < NT; ++j) {
            if (j < nt) {
              ga[j] = group_acc<QF, ACT>(ga[j], cg[rr][gi], sg[rr][gi], mg[rr][gi], xg[j][gi]);
              ua[j] = group_acc<QF, ACT>(ua[j], cu[rr][gi], su[rr][gi], mu[rr][gi], xg[j][gi]);
            }
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
  if (shared || !next_routed(a, ny, &pos, &wk)) return;
 }
}

// down projection:  o[j][r] = Wd[r] . h_j   (fp32 out)
template <int QF, int ACT, int NT, int GPL, int RPW>
__global__ __launch_bounds__(256) void k_down(FfnArgs a, int ny, int lpr_log2) {
  using CT = typename CodeOf<QF>::T;
  const bool shared = (int)blockIdx.y == ny;
  int pos = blockIdx.y;
  Work wk;
  if (shared) { wk.expert = -1; wk.lo = 0; wk.n = a.T; }
  else if (!next_routed(a, ny, &pos, &wk)) return;
 for (;;) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int LPR = 1 << lpr_log2, RPI = 64 >> lpr_log2;
  const int sub = lane & (LPR - 1), rsub = lane >> lpr_log2;
  const int G = a.I / kGroup;
  const MatView vd = expert_view<QF>(shared ? a.sdown : a.down, shared ? 0 : wk.expert, a.H, a.I);
  const void* hin = shared ? a.hs : a.h;
  float* out = shared ? a.so : a.o;
  const int r0 = (blockIdx.x * 4 + wave) * RPW * RPI + rsub;

  for (int c0 = 0; c0 < wk.n; c0 += NT) {
    const int nt = min(NT, wk.n - c0);
    XGroup<QF, ACT> hg[NT][GPL];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if (j < nt) {
        const size_t row = shared ? (size_t)(c0 + j) : (size_t)(wk.lo + c0 + j);
#pragma unroll
        for (int gi = 0; gi < GPL; ++gi) {
          const int g = sub + gi * LPR;
          if (g < G) hg[j][gi].load(hin, row * a.I + (size_t)g * kGroup);
        }
      }
    }
    CT cd[RPW][GPL];
    uint16_t sd[RPW][GPL], md[RPW][GPL];
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      const int r = r0 + rr * RPI;
#pragma unroll
      for (int gi = 0; gi < GPL; ++gi) {
        const int g = sub + gi * LPR;
        if (r < a.H && g < G) {
          cd[rr][gi] = *reinterpret_cast<const CT*>(vd.codes + (size_t)r * vd.row_bytes + (size_t)g * CodeOf<QF>::kBytes);
          sd[rr][gi] = vd.scales[(size_t)r * G + g];
          md[rr][gi] = (QF == MOE_Q2_ASYM_G32) ? vd.mins[(size_t)r * G + g] : (uint16_t)0;
        }
      }
    }
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      const int r = r0 + rr * RPI;
      float acc[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[j] = 0.f;
#pragma unroll
      for (int gi = 0; gi < GPL; ++gi) {
        const int g = sub + gi * LPR;
        if (r < a.H && g < G) {
#pragma unroll
          for (int j = 0; j < NT; ++j)
            if (j < nt) acc[j] = group_acc<QF, ACT>(acc[j], cd[rr][gi], sd[rr][gi], md[rr][gi], hg[j][gi]);
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

hipError_t launch_gateup(const FfnArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  return a.qfmt == MOE_Q4_SYM_G32 ? dispatch_act<MOE_Q4_SYM_G32>(a, true, s) : dispatch_act<MOE_Q2_ASYM_G32>(a, true, s);
}

hipError_t launch_down(const FfnArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  return a.qfmt == MOE_Q4_SYM_G32 ? dispatch_act<MOE_Q4_SYM_G32>(a, false, s) : dispatch_act<MOE_Q2_ASYM_G32>(a, false, s);
}

}  // namespace moe
