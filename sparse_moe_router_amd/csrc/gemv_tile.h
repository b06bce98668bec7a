// Dequantising dot products of packed group-32 rows with bf16 / fp32
// activations, shared by the expert kernels (wave64, gfx950).
//
// Inner product of one group (bf16 activations): each code u is OR-ed into the
// top mantissa bits of bf16 1.0, giving the exact bf16 number 1 + u/16 (4-bit)
// 1 + u/8 (3-bit) or 1 + u/4 (2-bit), two codes per 32-bit word, and
// v_dot2_f32_bf16 multiplies the pair with a pair of activations in fp32
// (every product is exact).  The offset is removed with a per-group constant
// computed once per token:
//   4-bit:  D = sum (1 + u/16) x - 1.5 sum x = sum (u - 8) x / 16,  acc += 16 s D
//   3-bit:  D = sum (1 + u/8) x - 1.5 sum x  = sum (u - 4) x / 8,   acc += 8 s D
//   2-bit:  D = sum (1 + u/4) x - sum x      = sum u x / 4,         acc += 4 s D + m sum x
// (w = s q with q = u - 8, or w = s u + m).  With the code in the top mantissa
// bits the cancelled offset stays within a few times the signal, so the fp32
// sums lose little to the cancellation.  Activation pairs are pre-arranged per
// token to match the code pairs a mask and a shift produce: 4-bit word i of a
// group yields pairs (8i+j, 8i+4+j) for j = 0..3 from nibbles j and j+4; 2-bit
// word i yields pairs (16i+j, 16i+8+j) for j = 0..7 from crumbs j and j+8, and
// so does 3-bit low-bit word i together with bits 16i+j, 16i+8+j of the
// third-bit word.
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

template <int QF> struct CodeOf;
template <> struct CodeOf<MOE_Q4_SYM_G32> { using T = u32x4; static constexpr int kBytes = 16; };
template <> struct CodeOf<MOE_Q2_ASYM_G32> { using T = u32x2; static constexpr int kBytes = 8; };
template <> struct CodeOf<MOE_Q3_SYM_G32> { using T = u32x3; static constexpr int kBytes = 12; };

// Prepared activations of one 32-element group of one token.
template <int QF, int ACT> struct XGroup;

template <int QF> struct XGroup<QF, MOE_ACT_BF16> {
  uint4 q[4];      // the group's 32 raw bf16 values
  uint32_t p[16];  // bf16 pairs matching the code pairs
  float c;         // 1.5 sum x (4-bit, 3-bit) or sum x (2-bit)
  float sx;        // sum x (2-bit only)

  __device__ __forceinline__ void load_raw(const void* base, size_t elem) {
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + elem);
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = src[i];
  }
  __device__ __forceinline__ void prep() {
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
    constexpr uint32_t kOff = (QF == MOE_Q2_ASYM_G32) ? 0x3f803f80u : 0x3fc03fc0u;  // (1, 1) / (1.5, 1.5)
    float c0 = 0.f, c1 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      c0 = dot2_bf16(kOff, p[i], c0);
      c1 = dot2_bf16(kOff, p[i + 1], c1);
    }
    c = c0 + c1;
    sx = c;  // used by the 2-bit format only, where c = sum x
  }
};

template <int QF> struct XGroup<QF, MOE_ACT_F32> {
  float4 r[8];  // the group's 32 fp32 values
  float sx;
  __device__ __forceinline__ void load_raw(const void* base, size_t elem) {
    const float4* src = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + elem);
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = src[i];
  }
  __device__ __forceinline__ void prep() {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += (r[i].x + r[i].y) + (r[i].z + r[i].w);
    sx = s;
  }
  __device__ __forceinline__ float at(int k) const {
    const float4 f = r[k >> 2];
    return (k & 3) == 0 ? f.x : (k & 3) == 1 ? f.y : (k & 3) == 2 ? f.z : f.w;
  }
};

// (a & m) | c in one instruction (the compiler otherwise emits an AND and an
// OR, since these constants need a literal and VOP3 takes none on gfx9; here
// the mask sits in a scalar register and the constant in a vector one: one
// scalar operand per instruction on gfx9).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(m), "v"(c));
  return d;
}

// Crumb j (bits 2j, 2j+1) moved to bits 5..6 (and crumb j + 8 to bits 21..22).
__device__ __forceinline__ uint32_t shift_crumb(uint32_t w, int j) { return j <= 2 ? w << (5 - 2 * j) : w >> (2 * j - 5); }

// The third bits of 3-bit low-bit word i (elements 16i .. 16i + 15 of the
// group: bits 16i .. 16i + 15 of the third-bit word t), spread so that
// element 16i + j sits at bit j and element 16i + 8 + j at bit 16 + j.
__device__ __forceinline__ uint32_t q3_high(uint32_t t, int i) {
  return __builtin_amdgcn_perm(t, t, i == 0 ? 0x0c010c00u : 0x0c030c02u);
}

// Codes j and j + 8 of 3-bit low-bit word w (crumbs at bits 2j and 2j + 16)
// with their third bits (bits j and 16 + j of the spread word hs) -> the bf16
// pair (1 + u/8): low bits to 4..5 and 20..21, third bit to 6 and 22.
__device__ __forceinline__ uint32_t q3_pair(uint32_t w, uint32_t hs, int j) {
  const uint32_t lo = j <= 2 ? w << (4 - 2 * j) : w >> (2 * j - 4);
  const uint32_t hi = j <= 6 ? hs << (6 - j) : hs >> (j - 6);
  return and_or(hi, 0x00400040u, and_or(lo, 0x00300030u, 0x3f803f80u));
}

// bf16 activations: sum q x / 16 (4-bit, q = u - 8) or sum u x / 4 (2-bit);
// fp32 activations: sum q x or sum u x.
template <int QF, int ACT>
__device__ __forceinline__ float group_dot(const typename CodeOf<QF>::T& cw, const XGroup<QF, ACT>& x) {
  if constexpr (ACT == MOE_ACT_BF16) {
    float d0 = 0.f, d1 = 0.f;
    if constexpr (QF == MOE_Q4_SYM_G32) {
      uint32_t w[4] = {cw[0], cw[1], cw[2], cw[3]};
      // unpack at the point of use (an empty asm that "updates" the words keeps
      // the compiler from hoisting every row's shifted copies at once)
#pragma unroll
      for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(w[i]));
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // nibbles j, j + 4 -> bits 3..6, 19..22
        d0 = dot2_bf16(and_or(w[i] << 3, 0x00780078u, 0x3f803f80u), x.p[4 * i + 0], d0);
        d1 = dot2_bf16(and_or(w[i] >> 1, 0x00780078u, 0x3f803f80u), x.p[4 * i + 1], d1);
        d0 = dot2_bf16(and_or(w[i] >> 5, 0x00780078u, 0x3f803f80u), x.p[4 * i + 2], d0);
        d1 = dot2_bf16(and_or(w[i] >> 9, 0x00780078u, 0x3f803f80u), x.p[4 * i + 3], d1);
      }
    } else if constexpr (QF == MOE_Q3_SYM_G32) {
      uint32_t w[3] = {cw[0], cw[1], cw[2]};
#pragma unroll
      for (int i = 0; i < 3; ++i) asm volatile("" : "+v"(w[i]));
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t hs = q3_high(w[2], i);
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          d0 = dot2_bf16(q3_pair(w[i], hs, j), x.p[8 * i + j], d0);
          d1 = dot2_bf16(q3_pair(w[i], hs, j + 1), x.p[8 * i + j + 1], d1);
        }
      }
    } else {
      uint32_t w[2] = {cw[0], cw[1]};
#pragma unroll
      for (int i = 0; i < 2; ++i) asm volatile("" : "+v"(w[i]));
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 8; j += 2) {  // crumbs j, j + 8 -> bits 5..6, 21..22
          d0 = dot2_bf16(and_or(shift_crumb(w[i], j), 0x00600060u, 0x3f803f80u), x.p[8 * i + j], d0);
          d1 = dot2_bf16(and_or(shift_crumb(w[i], j + 1), 0x00600060u, 0x3f803f80u), x.p[8 * i + j + 1], d1);
        }
      }
    }
    return (d0 + d1) - x.c;
  } else {
    float d0 = 0.f, d1 = 0.f;
    if constexpr (QF == MOE_Q4_SYM_G32) {
      const uint32_t w[4] = {cw[0], cw[1], cw[2], cw[3]};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          d0 = fmaf((float)((int)((w[i] >> (4 * j)) & 15u) - 8), x.at(8 * i + j), d0);
          d1 = fmaf((float)((int)((w[i] >> (4 * j + 4)) & 15u) - 8), x.at(8 * i + j + 1), d1);
        }
      }
    } else if constexpr (QF == MOE_Q3_SYM_G32) {
      const uint32_t w[3] = {cw[0], cw[1], cw[2]};
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
          const int e = 16 * i + j;
          const int u0 = (int)(((w[i] >> (2 * j)) & 3u) | (((w[2] >> e) & 1u) << 2));
          const int u1 = (int)(((w[i] >> (2 * j + 2)) & 3u) | (((w[2] >> (e + 1)) & 1u) << 2));
          d0 = fmaf((float)(u0 - 4), x.at(e), d0);
          d1 = fmaf((float)(u1 - 4), x.at(e + 1), d1);
        }
      }
    } else {
      const uint32_t w[2] = {cw[0], cw[1]};
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
          d0 = fmaf((float)((w[i] >> (2 * j)) & 3u), x.at(16 * i + j), d0);
          d1 = fmaf((float)((w[i] >> (2 * j + 2)) & 3u), x.at(16 * i + j + 1), d1);
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
  // the bf16 path's sums carry a factor 1/16, 1/8 or 1/4, folded into the scale (exactly)
  constexpr float kUnit = ACT == MOE_ACT_BF16 ? (QF == MOE_Q4_SYM_G32 ? 16.f : QF == MOE_Q3_SYM_G32 ? 8.f : 4.f) : 1.f;
  acc = fmaf(f16_to_f32(s16) * kUnit, d, acc);
  if constexpr (QF == MOE_Q2_ASYM_G32) acc = fmaf(f16_to_f32(m16), x.sx, acc);
  return acc;
}

struct MatView {
  const uint8_t* codes;
  const uint16_t* scales;
  const uint16_t* mins;
  size_t row_bytes;  // code bytes per row
  int groups;        // groups per row
  bool keep;         // load the codes with the default cache policy (a hot expert), else non-temporally
};

// Whether an expert's weights are kept in the caches: with hot > 0 the
// experts numbered below hot (the layer's most popular, when the caller has
// numbered its experts by popularity) and the shared expert; every other
// expert streams past the caches.
__device__ __forceinline__ bool hot_expert(const FfnArgs& a, bool shared, int e) {
  return a.hot > 0 && (shared || e < a.hot);
}

template <int QF>
__device__ __forceinline__ MatView expert_view(const QMat& m, int e, int rows, int cols, bool keep) {
  MatView v;
  v.keep = keep;
  v.row_bytes = (size_t)cols * code_bits(QF) / 8;
  v.groups = cols / kGroup;
  v.codes = m.codes + (size_t)e * rows * v.row_bytes;
  v.scales = m.scales + (size_t)e * rows * v.groups;
  v.mins = m.mins ? m.mins + (size_t)e * rows * v.groups : nullptr;
  return v;
}

// Packed codes, scales (and minima) of RPW rows x GPL groups for one lane.
template <int QF, int RPW, int GPL>
struct RowTile {
  using CT = typename CodeOf<QF>::T;
  CT c[RPW][GPL];
  uint16_t s[RPW][GPL];
  uint16_t m[RPW][GPL];

  // Branch-free: out-of-range rows / groups load a clamped in-range address
  // (their results are dropped later), so that no load sits in a conditional
  // block and all of them are in flight together.  Addresses are a
  // wave-uniform row base plus a 32-bit lane offset (scalar-base loads).
  // rbase: first row of the wave (uniform); the lane's row is rbase + rsub +
  // rr * rpi.
  __device__ __forceinline__ void load(const MatView& v, int rbase, int rsub, int rpi, int rows, int sub, int lpr) {
    if (v.keep) load_as<false>(v, rbase, rsub, rpi, rows, sub, lpr);  // uniform branch
    else load_as<true>(v, rbase, rsub, rpi, rows, sub, lpr);
  }

  template <bool NT>
  __device__ __forceinline__ void load_as(const MatView& v, int rbase, int rsub, int rpi, int rows, int sub,
                                          int lpr) {
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      const int ru = min(rbase + rr * rpi, rows - 1);          // uniform
      const int rc = min(ru + rsub, rows - 1);                 // this lane's row, >= ru
      const uint8_t* cb = v.codes + (size_t)ru * v.row_bytes;  // uniform bases
      const uint16_t* sb = v.scales + (size_t)ru * v.groups;
#pragma unroll
      for (int gi = 0; gi < GPL; ++gi) {
        const int gc = min(sub + gi * lpr, v.groups - 1);
        const uint32_t co = (uint32_t)(rc - ru) * (uint32_t)v.row_bytes + (uint32_t)gc * CodeOf<QF>::kBytes;
        const uint32_t so = (uint32_t)(rc - ru) * (uint32_t)v.groups + (uint32_t)gc;
        if constexpr (NT) c[rr][gi] = __builtin_nontemporal_load(reinterpret_cast<const CT*>(cb + co));
        else c[rr][gi] = *reinterpret_cast<const CT*>(cb + co);
        s[rr][gi] = sb[so];
        m[rr][gi] = (QF == MOE_Q2_ASYM_G32) ? (v.mins + (size_t)ru * v.groups)[so] : (uint16_t)0;
      }
    }
  }
};

}  // namespace moe
