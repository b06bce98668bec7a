// Helpers of the few-token kernels (wave64, gfx950): one token's activations
// staged in LDS prepared for the group dot products, the transposed reduction
// of a wave's gate and up row sums, and the group dot product split into the
// unpacking of the codes and the products (so that several tokens share one
// unpacking).
#pragma once

#include "gemv_tile.h"

namespace moe {

// The token's activations staged once per block in LDS, prepared for
// group_acc: group g's 16 words of pairs in q[0..3][g], its offset term in
// c[g] (lane-contiguous: every read below is conflict-free).
struct XLds {
  uint4 q[4][64];
  float c[64];
};

// One wave's share of x: lane = group; groups past H / 32 repeat the last one.
template <int QF>
__device__ __forceinline__ void load_x1(const void* x, int H, int lane, XGroup<QF, MOE_ACT_BF16>& xg) {
  xg.load_raw(x, (size_t)min(lane, H / kGroup - 1) * kGroup);
}

// The loaded group prepared and stored in LDS.
template <int QF>
__device__ __forceinline__ void put_x1(XGroup<QF, MOE_ACT_BF16>& xg, int lane, XLds& xs) {
  xg.prep();
#pragma unroll
  for (int i = 0; i < 4; ++i) xs.q[i][lane] = make_uint4(xg.p[4 * i], xg.p[4 * i + 1], xg.p[4 * i + 2], xg.p[4 * i + 3]);
  xs.c[lane] = xg.c;
}

// One wave stages x.
template <int QF>
__device__ __forceinline__ void stage_x1(const void* x, int H, int lane, XLds& xs) {
  XGroup<QF, MOE_ACT_BF16> xg;
  load_x1<QF>(x, H, lane, xg);
  put_x1<QF>(xg, lane, xs);
}

template <int QF>
__device__ __forceinline__ void read_x1(const XLds& xs, int lane, XGroup<QF, MOE_ACT_BF16>& xg) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = xs.q[i][lane];
    xg.p[4 * i] = v.x; xg.p[4 * i + 1] = v.y; xg.p[4 * i + 2] = v.z; xg.p[4 * i + 3] = v.w;
  }
  xg.c = xs.c[lane];
  xg.sx = xg.c;
}

// The 2 RPW per-lane partial sums of a wave (gate rows 0..RPW-1, then up
// rows) reduced over the 64 lanes together: a permlane32 swap pairs gate row
// i with up row i (lanes < 32 keep the gate sum), a permlane16 swap halves
// the values again, one DPP rotate by 8 when RPW = 4, then DPP steps within
// the remaining 16 or 8 lanes.  Afterwards lane (32 / RPW) i (i < RPW) holds
// gate row i in *g and up row i in *u.
template <int RPW>
__device__ __forceinline__ void reduce_gu1(const float (&v)[2 * RPW], int lane, float* g, float* u) {
  static_assert(RPW == 1 || RPW == 2 || RPW == 4, "one, two or four rows per wave");
  auto f = [](uint32_t b) { return __uint_as_float(b); };
  auto b = [](float x) { return __float_as_uint(x); };
  if constexpr (RPW == 1) {
    const auto r0 = __builtin_amdgcn_permlane32_swap(b(v[0]), b(v[1]), false, false);
    float sum = f(r0[0]) + f(r0[1]);  // lanes < 32: gate, >= 32: up
    const auto r1 = __builtin_amdgcn_permlane16_swap(b(sum), b(sum), false, false);
    sum = f(r1[0]) + f(r1[1]);
    sum += dpp_f<kDppXor1>(sum);
    sum += dpp_f<kDppXor2>(sum);
    sum += dpp_f<kDppHalfMirror>(sum);
    sum += dpp_f<kDppMirror>(sum);
    const auto r = __builtin_amdgcn_permlane32_swap(b(sum), b(sum), false, false);
    *g = f(r[0]);
    *u = f(r[1]);
    return;
  }
  float w[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(b(v[i]), b(v[i + RPW]), false, false);
    w[i] = f(r[0]) + f(r[1]);
  }
  float x[RPW / 2 + (RPW == 1)];
#pragma unroll
  for (int i = 0; i < RPW / 2; ++i) {
    const auto r = __builtin_amdgcn_permlane16_swap(b(w[i]), b(w[i + RPW / 2]), false, false);
    x[i] = f(r[0]) + f(r[1]);
  }
  float sum;
  if constexpr (RPW == 4) {
    const bool hi = (lane & 8) != 0;
    const float keep = hi ? x[1] : x[0], give = hi ? x[0] : x[1];
    sum = keep + dpp_f<kDppRor8>(give);
    sum += dpp_f<kDppXor1>(sum);
    sum += dpp_f<kDppXor2>(sum);
    sum += dpp_f<kDppHalfMirror>(sum);
  } else {
    sum = x[0];
    sum += dpp_f<kDppXor1>(sum);
    sum += dpp_f<kDppXor2>(sum);
    sum += dpp_f<kDppHalfMirror>(sum);
    sum += dpp_f<kDppMirror>(sum);
  }
  const auto r = __builtin_amdgcn_permlane32_swap(b(sum), b(sum), false, false);  // gate half | up half
  *g = f(r[0]);
  *u = f(r[1]);
}

// The 16 bf16 code pairs of one group (matching the activation pairs of XGroup).
template <int QF>
__device__ __forceinline__ void unpack_group(const typename CodeOf<QF>::T& cw, uint32_t (&b)[16]) {
  if constexpr (QF == MOE_Q4_SYM_G32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // nibbles j, j + 4 -> bits 3..6, 19..22
      const uint32_t w = cw[i];
      b[4 * i + 0] = and_or(w << 3, 0x00780078u, 0x3f803f80u);
      b[4 * i + 1] = and_or(w >> 1, 0x00780078u, 0x3f803f80u);
      b[4 * i + 2] = and_or(w >> 5, 0x00780078u, 0x3f803f80u);
      b[4 * i + 3] = and_or(w >> 9, 0x00780078u, 0x3f803f80u);
    }
  } else if constexpr (QF == MOE_Q3_SYM_G32) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t hs = q3_high(cw[2], i);
#pragma unroll
      for (int j = 0; j < 8; ++j) b[8 * i + j] = q3_pair(cw[i], hs, j);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t w = cw[i];
#pragma unroll
      for (int j = 0; j < 8; ++j)  // crumbs j, j + 8 -> bits 5..6, 21..22
        b[8 * i + j] = and_or(shift_crumb(w, j), 0x00600060u, 0x3f803f80u);
    }
  }
}

// acc + the group's contribution from unpacked codes (the arithmetic of
// group_acc for bf16 activations, in the same order).
template <int QF>
__device__ __forceinline__ float group_acc_unpacked(float acc, const uint32_t (&b)[16], uint16_t s16, uint16_t m16,
                                                    const XGroup<QF, MOE_ACT_BF16>& x) {
  float d0 = 0.f, d1 = 0.f;
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    d0 = dot2_bf16(b[i], x.p[i], d0);
    d1 = dot2_bf16(b[i + 1], x.p[i + 1], d1);
  }
  const float d = (d0 + d1) - x.c;
  constexpr float kUnit = QF == MOE_Q4_SYM_G32 ? 16.f : QF == MOE_Q3_SYM_G32 ? 8.f : 4.f;
  acc = fmaf(f16_to_f32(s16) * kUnit, d, acc);
  if constexpr (QF == MOE_Q2_ASYM_G32) acc = fmaf(f16_to_f32(m16), x.sx, acc);
  return acc;
}

}  // namespace moe
