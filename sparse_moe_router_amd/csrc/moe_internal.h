// Internal launch interface between the C ABI (moe_abi.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

#include "moe.h"

namespace moe {

constexpr int kGroup = 32;

// Code bits per weight of a format.
__host__ __device__ constexpr int code_bits(int qfmt) {
  return qfmt == MOE_Q4_SYM_G32 ? 4 : qfmt == MOE_Q3_SYM_G32 ? 3 : 2;
}

// f(std::integral_constant<int, QF>{}) for the layer's format (one template
// instance per format).
template <typename F>
inline auto by_qfmt(int qfmt, F&& f) {
  if (qfmt == MOE_Q4_SYM_G32) return f(std::integral_constant<int, MOE_Q4_SYM_G32>{});
  if (qfmt == MOE_Q3_SYM_G32) return f(std::integral_constant<int, MOE_Q3_SYM_G32>{});
  return f(std::integral_constant<int, MOE_Q2_ASYM_G32>{});
}

struct QMat {
  const uint8_t* codes;
  const uint16_t* scales;
  const uint16_t* mins;
};

inline QMat qmat(const moe_qmat& m) { return QMat{m.codes, m.scales, m.mins}; }

// ---------------------------------------------------------------- router
struct RouterArgs {
  const void* x;        // [T][H] act
  const float* w;       // [E][H]
  const float* b;       // [E] or null
  float* logits;        // [T][E]
  int32_t* ids;         // [T][K]
  float* wts;           // [T][K]
  int T, H, E, K, act;
};
hipError_t launch_router_logits(const RouterArgs& a, hipStream_t s);
hipError_t launch_topk(const RouterArgs& a, hipStream_t s);

// ---------------------------------------------------------------- permutation
struct PermuteArgs {
  const int32_t* ids;   // [T*K]
  int32_t* offsets;     // [E+1]
  int32_t* sorted_pairs;
  int32_t* pair_pos;
  int32_t* chunk_base;  // [n_chunks][E] scratch
  int T, K, E;
  // written by the small-batch routing only (else null): work[u] = (expert,
  // first sorted position, token count, 0) of the u-th distinct expert in
  // sorted order and (-1, 0, 0, 0) past the last, for u < T K; sorted_tok[y]
  // = the token of sorted position y
  int32_t* work = nullptr;
  int32_t* sorted_tok = nullptr;
};
size_t permute_scratch_ints(int T, int K, int E);
hipError_t launch_permute(const PermuteArgs& a, hipStream_t s);
// top-K and permutation in one block for small batches (T*K <= 256, E <= 1024)
bool route_small_ok(int T, int K, int E);
hipError_t launch_route_small(const RouterArgs& a, const PermuteArgs& p, hipStream_t s);

// debug library only: range checks of caller-provided routing arrays (null
// arrays are skipped); err receives the failed checks' bits, after a
// synchronisation of s
struct RoutingCheck {
  const int32_t* ids;
  const int32_t* offsets;
  const int32_t* sorted;
  const int32_t* pos;
  int T, K, E;
};
hipError_t check_routing(const RoutingCheck& c, hipStream_t s, uint32_t* err);

// ---------------------------------------------------------------- expert FFN
struct FfnArgs {
  QMat gate, up, down;     // routed, expert 0 base
  QMat sgate, sup, sdown;  // shared expert (n_shared == 1) or unused
  int n_shared;
  int T, H, I, E, K, qfmt, act;
  const void* x;               // [T][H] act
  const int32_t* ids;          // [T*K] expert of each pair
  const int32_t* offsets;      // [E+1]
  const int32_t* sorted_pairs; // [T*K]
  void* h;                     // [T*K][I] act, sorted order
  void* hs;                    // [T][I] act, shared
  float* o;                    // [T*K][H] fp32, sorted order
  float* so;                   // [T][H] fp32, shared (null: shared expert skipped)
  // Split of the experts between the kernel families: experts with at least
  // mfma_min tokens (and the shared expert when T >= mfma_min) run on the
  // matrix-core grouped GEMM, the others on the GEMV kernels.  0: no split
  // (the GEMV kernels take every expert; the grouped GEMM is not launched).
  int mfma_min;
  // experts numbered below hot (and the shared expert) are loaded with the
  // default cache policy so that they stay in the caches across calls; 0: every
  // expert streams past them (non-temporal loads)
  int hot;
  // the small-batch routing's work list and tokens by sorted position
  // (PermuteArgs), or null: the small-batch kernels then find their expert
  // from ids, sorted_pairs and offsets
  const int32_t* work = nullptr;
  const int32_t* sorted_tok = nullptr;
};
// the GEMV kernels skip an expert with n tokens that the grouped GEMM takes
__host__ __device__ inline bool on_mfma(const FfnArgs& a, int n) { return a.mfma_min > 0 && n >= a.mfma_min; }
hipError_t launch_gateup(const FfnArgs& a, hipStream_t s);
hipError_t launch_down(const FfnArgs& a, hipStream_t s);
// small batches (1 < T, T K <= 256, bf16; H <= 2048 for gate/up, I <= 1024 for
// down): one block row per sorted position, the expert's codes unpacked once
// for all its tokens (launch_gateup / launch_down pick them)
bool gateup_sb_ok(const FfnArgs& a);
bool down_sb_ok(const FfnArgs& a);
hipError_t launch_gateup_sb(const FfnArgs& a, hipStream_t s);
hipError_t launch_down_sb(const FfnArgs& a, hipStream_t s);
// matrix-core grouped GEMMs for many tokens per expert: launch_gateup and
// launch_down set FfnArgs::mfma_min = mfma_split(a) and run the grouped GEMM
// for the experts it assigns (all of them when it returns 1), then the GEMV
// kernels for the rest
int mfma_split(const FfnArgs& a);
hipError_t launch_mfma_gateup(const FfnArgs& a, hipStream_t s);
hipError_t launch_mfma_down(const FfnArgs& a, hipStream_t s);

// ---------------------------------------------------------------- combine
struct CombineArgs {
  const float* o;          // [T*K][H] sorted order
  const float* so;         // [T][H] or null
  const int32_t* pair_pos; // [T*K]
  const float* w;          // [T*K]
  const void* x_resid;     // [T][H] act or null
  void* x_next;            // [T][H] act or null
  float* y;                // [T][H]
  int T, H, K, act;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
// layer forward with the small-batch routing's work list (FfnArgs::work): the
// down projection fused with the combine, all h rows staged in one block's
// LDS (T (K + 1) rows up to 128 KiB), no expert on the grouped GEMM
bool fused_down_sb_ok(const FfnArgs& a);
hipError_t launch_fused_down_sb(const FfnArgs& a, const CombineArgs& c, hipStream_t s);

// ---------------------------------------------------------------- fused decode path
// one token: gate/up with the routing (top-K, permutation) recomputed per
// block: K <= 64, E <= 1024, H, I <= 2048, bf16 activations
bool fused_decode_ok(int T, int K, int E, int H, int I, int act);
hipError_t launch_fused_gateup(const RouterArgs& r, const PermuteArgs& pm, const FfnArgs& a, hipStream_t s);
// one token: down projection fused with the combine (K <= 16, E <= 512, I <= 1024);
// h in slot order, as the one-token fused gate/up writes it
bool fused_down1_ok(int T, int K, int E, int I);
hipError_t launch_fused_down1(const FfnArgs& a, const CombineArgs& c, hipStream_t s);

// ---------------------------------------------------------------- test hook
hipError_t launch_dequant(const QMat& m, int qfmt, int rows, int cols, float* out, hipStream_t s);

}  // namespace moe
