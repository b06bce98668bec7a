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

// Selection state of one wave for E <= 64 PL experts (PL <= 8): lane l holds
// the logits of the consecutive experts PL l + i (i < PL) as 32-bit keys sorted
// in descending order (larger logit first, then lower expert id; 0 = empty),
// with each key's position i in a 4-bit field of pos (field j: the lane's j-th
// key).  Since a lower lane holds lower ids, the lowest lane among lanes whose
// heads tie holds the lowest id, so a round needs one wave maximum and one
// ballot; the picks come out in the same order as from wave_topk_regs.
template <int PL>
struct LaneSorted {
  static_assert(PL <= 8, "positions are packed in one 32-bit register");
  uint32_t k[PL];
  uint32_t pos;

  // lg: 16-byte aligned when E == 64 PL (the lane's PL logits are then read
  // as 16-byte vectors)
  __device__ __forceinline__ void load(const float* lg, int E, int lane) {
    float v[PL];
    if (PL >= 4 && E == 64 * PL) {
#pragma unroll
      for (int q = 0; q < PL / 4; ++q) {
        const float4 f = reinterpret_cast<const float4*>(lg + PL * lane)[q];
        v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < PL; ++i) v[i] = lg[min(PL * lane + i, E - 1)];  // clamped: no conditional loads
    }
    uint64_t c[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int e = PL * lane + i;
      c[i] = e < E ? sel_key(v[i], e) : 0ull;
    }
    auto cx = [&](int a, int b) {  // c[a] >= c[b] afterwards
      const uint64_t hi = c[a] > c[b] ? c[a] : c[b];
      const uint64_t lo = c[a] > c[b] ? c[b] : c[a];
      c[a] = hi;
      c[b] = lo;
    };
    if constexpr (PL == 2) {
      cx(0, 1);
    } else if constexpr (PL == 4) {
      cx(0, 1); cx(2, 3); cx(0, 2); cx(1, 3); cx(1, 2);
    } else if constexpr (PL == 8) {  // 19 comparators, depth 6
      cx(0, 2); cx(1, 3); cx(4, 6); cx(5, 7);
      cx(0, 4); cx(1, 5); cx(2, 6); cx(3, 7);
      cx(0, 1); cx(2, 3); cx(4, 5); cx(6, 7);
      cx(2, 4); cx(3, 5);
      cx(1, 4); cx(3, 6);
      cx(1, 2); cx(3, 4); cx(5, 6);
    }
    pos = 0;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      k[i] = (uint32_t)(c[i] >> 32);
      pos |= ((uint32_t)(key_id(c[i]) - PL * lane) & 15u) << (4 * i);
    }
  }

  // One round: the largest remaining key of the wave (returned, uniform); the
  // lowest lane holding it (the lowest id) drops it and writes its expert id
  // to ids_lds[round].  The winner is found from the ballot with mbcnt, so the
  // round has no scalar step between the maximum and the shift.
  __device__ __forceinline__ uint32_t round(int lane, int rnd, int32_t* ids_lds) {
    const uint32_t m = wave_max_u32(k[0]);
    const uint64_t tied = __ballot(k[0] == m);
    const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(tied >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)tied, 0u));
    const bool win = k[0] == m && below == 0;
    if (win) ids_lds[rnd] = PL * lane + (int)(pos & 15u);
#pragma unroll
    for (int i = 0; i + 1 < PL; ++i) k[i] = win ? k[i + 1] : k[i];  // selects, not a branch
    k[PL - 1] = win ? 0u : k[PL - 1];
    pos = win ? pos >> 4 : pos;
    return m;
  }
};

// logits per lane held in registers for E experts: 1, 2, 4, 8 or 16
inline int regs_per_lane(int E) {
  int pl = 1;
  while (64 * pl < E) pl <<= 1;
  return pl;
}

}  // namespace moe
