// Top-K selection of router logits by one wave (wave64, gfx950): keys, the
// register-resident selection and its renormalised softmax weights.
#pragma once

#include "moe_device.h"

namespace moe {

constexpr int kRegLogits = 16;  // logits per lane held in registers: E <= 1024

// Order-preserving map of a float to uint32 (NaN treated as -inf); every real
// value maps to >= 0x007fffff, so 0 marks "taken / empty".
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f != f) f = -INFINITY;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// 64-bit selection key: larger logit first, then smaller expert id.
__device__ __forceinline__ uint64_t sel_key(float l, int e) {
  return ((uint64_t)order_key(l) << 32) | (uint32_t)(0xffffffffu - (uint32_t)e);
}
__device__ __forceinline__ int key_id(uint64_t k) { return (int)(0xffffffffu - (uint32_t)k); }

// A lane's candidates: the logits of experts lane + 64 i (i < PL) as 64-bit
// selection keys, sorted in descending order in registers (0 = empty).
template <int PL>
__device__ __forceinline__ void lane_candidates(const float* lg, int E, int lane, uint64_t (&c)[PL]) {
  float v[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) v[i] = lg[min(lane + 64 * i, E - 1)];  // clamped: no conditional loads
#pragma unroll
  for (int i = 0; i < PL; ++i) c[i] = (lane + 64 * i < E) ? sel_key(v[i], lane + 64 * i) : 0ull;
  // odd-even transposition sort (PL is small; every step is independent compare-swaps)
#pragma unroll
  for (int pass = 0; pass < PL; ++pass) {
#pragma unroll
    for (int i = pass & 1; i + 1 < PL; i += 2) {
      const uint64_t hi = c[i] > c[i + 1] ? c[i] : c[i + 1];
      const uint64_t lo = c[i] > c[i + 1] ? c[i + 1] : c[i];
      c[i] = hi;
      c[i + 1] = lo;
    }
  }
}

// One selection round over the lanes' sorted candidates: the wave maximum of
// the heads (32-bit logit keys, one DPP max per step), the lowest id among
// lanes tied at it; the winning lane drops its head.  Returns the expert id
// (wave-uniform) and its logit key in *key.
template <int PL>
__device__ __forceinline__ int select_round(uint64_t (&c)[PL], int lane, uint32_t* key) {
  const uint32_t bk = (uint32_t)(c[0] >> 32);
  const uint32_t m = wave_max_u32(bk);
  const uint64_t tied = __ballot(bk == m);
  int winner;  // lane
  if (__popcll(tied) == 1) {
    winner = (int)__ffsll((unsigned long long)tied) - 1;
  } else {  // several lanes hold an equal key: the lowest id wins
    const int id_min = wave_min_i32(bk == m ? key_id(c[0]) : 0x7fffffff);
    winner = id_min & 63;
  }
  const int id = (int)(0xffffffffu - (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)c[0], winner));
  if (lane == winner) {
#pragma unroll
    for (int i = 0; i + 1 < PL; ++i) c[i] = c[i + 1];
    c[PL - 1] = 0ull;
  }
  *key = m;
  return id;
}

// ids[k] and the renormalised softmax weight of the pick of round k (k < K <=
// 64), from lane k's (key, id) of that round and the first round's key.
__device__ __forceinline__ void write_topk(uint32_t mine, int mine_id, uint32_t top, int K, int lane, int32_t* ids,
                                           float* wts) {
  const float ex = lane < K ? expf(key_value(mine) - key_value(top)) : 0.f;
  const float total = wave_sum(ex);
  if (lane < K) {
    ids[lane] = mine_id;
    wts[lane] = ex / total;
  }
}

// Top-K of one token by one wave with the token's logits in registers
// (expert e = lane + 64 i, PL per lane): K selection rounds.
// Writes ids and the renormalised softmax weights of the K selected logits
// (unless ids is null; then only lds_ids, which requires K <= 64).
template <int PL>
__device__ __forceinline__ void wave_topk_regs(const float* lg, int E, int K, int lane, int32_t* ids, float* wts,
                                               int32_t* lds_ids) {
  uint64_t c[PL];
  lane_candidates<PL>(lg, E, lane, c);
  uint32_t mine = 0;   // lane k keeps the key and id picked in round k (k < 64)
  int mine_id = 0;
  uint32_t top = 0;
  for (int k = 0; k < K; ++k) {
    uint32_t m;
    const int id = select_round<PL>(c, lane, &m);
    if (k == 0) top = m;
    if (lane == (k & 63)) { mine = m; mine_id = id; }
    if (K > 64 && ids && lane == 0) ids[k] = id;
    if (lds_ids && lane == 0) lds_ids[k] = id;
  }
  if (K <= 64) {
    if (ids) write_topk(mine, mine_id, top, K, lane, ids, wts);  // ids / wts may be null: selection into LDS only
  } else {  // rare: more than 64 slots, weights from the stored logits
    const float l0 = key_value(top);
    __builtin_amdgcn_s_waitcnt(0);
    float part = 0.f;
    for (int k = lane; k < K; k += 64) part += expf(lg[ids[k]] - l0);
    const float total = wave_sum(part);
    for (int k = lane; k < K; k += 64) wts[k] = expf(lg[ids[k]] - l0) / total;
  }
}

// logits per lane held in registers for E experts: 1, 2, 4, 8 or 16
inline int regs_per_lane(int E) {
  int pl = 1;
  while (64 * pl < E) pl <<= 1;
  return pl;
}

}  // namespace moe
