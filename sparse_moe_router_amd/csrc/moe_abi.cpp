// C ABI of the routed MoE FFN layer: host-side validation, workspace layout
// and kernel dispatch.  No allocation, no host synchronisation, no state.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "moe.h"
#include "moe_internal.h"

namespace {

using namespace moe;

constexpr int kMaxDim = 4096;
constexpr int kMaxExperts = 8192;
constexpr int32_t kAbiVersion = 4;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t act_size(int act) { return act == MOE_ACT_BF16 ? 2 : 4; }

bool qmat_ok(const moe_qmat& m, int qfmt) {
  if (!m.codes || !m.scales) return false;
  if (!aligned(m.codes, 16) || !aligned(m.scales, 2)) return false;
  if (qfmt == MOE_Q2_ASYM_G32) return m.mins != nullptr && aligned(m.mins, 2);
  return true;
}

moe_status check_layer(const moe_layer* L) {
  if (!L) return MOE_E_ARG;
  if (L->hidden <= 0 || L->inter <= 0 || L->hidden % kGroup || L->inter % kGroup) return MOE_E_ARG;
  if (L->hidden > kMaxDim || L->inter > kMaxDim) return MOE_E_UNSUPPORTED;
  if (L->n_experts < 1 || L->top_k < 1 || L->top_k > L->n_experts) return MOE_E_ARG;
  if (L->n_experts > kMaxExperts) return MOE_E_UNSUPPORTED;
  if (L->qfmt != MOE_Q4_SYM_G32 && L->qfmt != MOE_Q2_ASYM_G32 && L->qfmt != MOE_Q3_SYM_G32) return MOE_E_UNSUPPORTED;
  if (L->act != MOE_ACT_F32 && L->act != MOE_ACT_BF16) return MOE_E_UNSUPPORTED;
  if (!L->router_w || !aligned(L->router_w, 16)) return MOE_E_ARG;
  if (L->routed.n != L->n_experts) return MOE_E_ARG;
  if (!qmat_ok(L->routed.gate, L->qfmt) || !qmat_ok(L->routed.up, L->qfmt) || !qmat_ok(L->routed.down, L->qfmt))
    return MOE_E_ARG;
  if (L->shared.n < 0 || L->hot_experts < 0) return MOE_E_ARG;
  if (L->shared.n > 1) return MOE_E_UNSUPPORTED;
  if (L->shared.n == 1 &&
      (!qmat_ok(L->shared.gate, L->qfmt) || !qmat_ok(L->shared.up, L->qfmt) || !qmat_ok(L->shared.down, L->qfmt)))
    return MOE_E_ARG;
  return MOE_OK;
}

moe_status check_tokens(const moe_layer* L, int32_t T) {
  if (T < 0) return MOE_E_ARG;
  const int64_t pairs = (int64_t)T * L->top_k;
  const int64_t wide = L->hidden > L->inter ? L->hidden : L->inter;
  if (pairs * wide >= ((int64_t)1 << 31) || (int64_t)T * L->n_experts >= ((int64_t)1 << 31)) return MOE_E_UNSUPPORTED;
  return MOE_OK;
}

// Workspace regions (byte offsets), each 256-byte aligned.
struct Ws {
  size_t logits, ids, w, offsets, sorted, pos, chunk, work, stok, h, hs, o, so, y, total;
};

Ws ws_layout(const moe_layer& L, int32_t T) {
  Ws w{};
  size_t off = 0;
  auto take = [&off](size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) & ~(size_t)255;
    return at;
  };
  const size_t t = (size_t)T, k = (size_t)L.top_k, e = (size_t)L.n_experts;
  const size_t a = act_size(L.act);
  w.logits = take(t * e * 4);
  w.ids = take(t * k * 4);
  w.w = take(t * k * 4);
  w.offsets = take((e + 1) * 4);
  w.sorted = take(t * k * 4);
  w.pos = take(t * k * 4);
  w.chunk = take(permute_scratch_ints(T, L.top_k, L.n_experts) * 4);
  w.work = take(t * k * 16);
  w.stok = take(t * k * 4);
  w.h = take(t * k * L.inter * a);
  w.hs = take(t * L.inter * a);
  w.o = take(t * k * L.hidden * 4);
  w.so = take(t * L.hidden * 4);
  w.y = take(t * L.hidden * 4);
  w.total = off;
  return w;
}

template <typename P>
P* at(void* ws, size_t off) { return reinterpret_cast<P*>(reinterpret_cast<char*>(ws) + off); }

moe_status ws_check(const moe_layer& L, int32_t T, void* ws, size_t ws_bytes) {
  if (!ws) return MOE_E_WORKSPACE;
  if (!aligned(ws, 256)) return MOE_E_ARG;
  if (ws_bytes < ws_layout(L, T).total) return MOE_E_WORKSPACE;
  return MOE_OK;
}

moe_status dev(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_E_DEVICE; }

#define MOE_TRY(expr)                         \
  do {                                        \
    const moe_status st_ = (expr);            \
    if (st_ != MOE_OK) return st_;            \
  } while (0)

RouterArgs router_args(const moe_layer& L, const void* x, int32_t T, float* logits, int32_t* ids, float* w) {
  return RouterArgs{x, L.router_w, L.router_b, logits, ids, w, T, L.hidden, L.n_experts, L.top_k, L.act};
}

// The shared expert runs only if the layer has one and its output (hs for
// gate/up, so for down) is given.
FfnArgs ffn_args(const moe_layer& L, const void* x, int32_t T, const int32_t* ids, const int32_t* offsets,
                 const int32_t* sorted, void* h, void* hs, float* o, float* so) {
  FfnArgs f{};
  f.gate = qmat(L.routed.gate); f.up = qmat(L.routed.up); f.down = qmat(L.routed.down);
  if (L.shared.n == 1) { f.sgate = qmat(L.shared.gate); f.sup = qmat(L.shared.up); f.sdown = qmat(L.shared.down); }
  f.n_shared = L.shared.n == 1 ? 1 : 0;
  f.T = T; f.H = L.hidden; f.I = L.inter; f.E = L.n_experts; f.K = L.top_k; f.qfmt = L.qfmt; f.act = L.act;
  f.x = x; f.ids = ids; f.offsets = offsets; f.sorted_pairs = sorted;
  f.h = h; f.hs = f.n_shared ? hs : nullptr; f.o = o; f.so = f.n_shared ? so : nullptr;
  f.hot = L.hot_experts;
  return f;
}

moe_status layer_forward_impl(const moe_layer& L, const void* x, int32_t T, float* y, void* x_next,
                              int32_t* ids_opt, float* w_opt, void* ws, hipStream_t s) {
  const Ws W = ws_layout(L, T);
  int32_t* ids = ids_opt ? ids_opt : at<int32_t>(ws, W.ids);
  float* wts = w_opt ? w_opt : at<float>(ws, W.w);
  const RouterArgs ra = router_args(L, x, T, at<float>(ws, W.logits), ids, wts);
  PermuteArgs pa{ids, at<int32_t>(ws, W.offsets), at<int32_t>(ws, W.sorted), at<int32_t>(ws, W.pos),
                 at<int32_t>(ws, W.chunk), T, L.top_k, L.n_experts};
  FfnArgs fa = ffn_args(L, x, T, ids, pa.offsets, pa.sorted_pairs, at<void>(ws, W.h), at<void>(ws, W.hs),
                        at<float>(ws, W.o), at<float>(ws, W.so));
  const CombineArgs ca{fa.o, fa.so, pa.pair_pos, wts, x_next ? x : nullptr, x_next, y, T, L.hidden, L.top_k, L.act};
  MOE_TRY(dev(launch_router_logits(ra, s)));
  if (fused_decode_ok(T, L.top_k, L.n_experts, L.hidden, L.inter, L.act)) {
    // few tokens: routing recomputed inside the gate/up kernel; one token: down + combine fused
    MOE_TRY(dev(launch_fused_gateup(ra, pa, fa, s)));
    if (fused_down1_ok(T, L.top_k, L.n_experts, L.inter)) return dev(launch_fused_down1(fa, ca, s));
    MOE_TRY(dev(launch_down(fa, s)));
    return dev(launch_combine(ca, s));
  }
  if (route_small_ok(T, L.top_k, L.n_experts)) {
    // with the work list: the small-batch kernels find their expert in one load
    pa.work = at<int32_t>(ws, W.work);
    pa.sorted_tok = at<int32_t>(ws, W.stok);
    fa.work = pa.work;
    fa.sorted_tok = pa.sorted_tok;
    MOE_TRY(dev(launch_route_small(ra, pa, s)));
  } else {
    MOE_TRY(dev(launch_topk(ra, s)));
    MOE_TRY(dev(launch_permute(pa, s)));
  }
  MOE_TRY(dev(launch_gateup(fa, s)));
  if (fused_down_sb_ok(fa)) return dev(launch_fused_down_sb(fa, ca, s));  // with the work list only
  MOE_TRY(dev(launch_down(fa, s)));
  return dev(launch_combine(ca, s));
}

// The debug library checks caller-provided routing arrays on the device
// before anything indexes with them; the release library takes them as given.
moe_status range_check(const moe_layer* L, int32_t T, const int32_t* ids, const int32_t* offsets,
                       const int32_t* sorted, const int32_t* pos, void* stream) {
#ifdef MOE_RANGE_CHECKS
  uint32_t err = 0;
  const RoutingCheck c{ids, offsets, sorted, pos, T, L->top_k, L->n_experts};
  MOE_TRY(dev(check_routing(c, reinterpret_cast<hipStream_t>(stream), &err)));
  return err ? MOE_E_ARG : MOE_OK;
#else
  (void)L; (void)T; (void)ids; (void)offsets; (void)sorted; (void)pos; (void)stream;
  return MOE_OK;
#endif
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return kAbiVersion; }

int32_t moe_range_checks(void) {
#ifdef MOE_RANGE_CHECKS
  return 1;
#else
  return 0;
#endif
}

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_E_ARG: return "MOE_E_ARG: invalid argument";
    case MOE_E_UNSUPPORTED: return "MOE_E_UNSUPPORTED: valid but unsupported size or format";
    case MOE_E_WORKSPACE: return "MOE_E_WORKSPACE: workspace missing or too small";
    case MOE_E_DEVICE: return "MOE_E_DEVICE: HIP launch error";
  }
  return "unknown moe_status";
}

size_t moe_workspace_bytes(const moe_layer* layer, int32_t T_max) {
  if (check_layer(layer) != MOE_OK || check_tokens(layer, T_max) != MOE_OK) return 0;
  return ws_layout(*layer, T_max).total;
}

moe_status moe_router_topk(const moe_layer* layer, const void* x, int32_t T, int32_t* topk_ids, float* topk_w,
                           float* logits_opt, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_layer(layer));
  MOE_TRY(check_tokens(layer, T));
  if (T == 0) return MOE_OK;
  if (!x || !topk_ids || !topk_w || !aligned(x, 16)) return MOE_E_ARG;
  float* logits = logits_opt;
  if (!logits) {
    MOE_TRY(ws_check(*layer, T, ws, ws_bytes));
    logits = at<float>(ws, ws_layout(*layer, T).logits);
  }
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const RouterArgs ra = router_args(*layer, x, T, logits, topk_ids, topk_w);
  MOE_TRY(dev(launch_router_logits(ra, s)));
  return dev(launch_topk(ra, s));
}

moe_status moe_permute(const moe_layer* layer, const int32_t* topk_ids, int32_t T, int32_t* expert_offsets,
                       int32_t* sorted_pairs, int32_t* pair_pos, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_layer(layer));
  MOE_TRY(check_tokens(layer, T));
  if (!topk_ids || !expert_offsets || !sorted_pairs || !pair_pos) return MOE_E_ARG;
  MOE_TRY(ws_check(*layer, T, ws, ws_bytes));
  MOE_TRY(range_check(layer, T, topk_ids, nullptr, nullptr, nullptr, stream));
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const Ws W = ws_layout(*layer, T);
  PermuteArgs pa{topk_ids, expert_offsets, sorted_pairs, pair_pos, at<int32_t>(ws, W.chunk), T, layer->top_k,
                 layer->n_experts};
  return dev(launch_permute(pa, s));  // T == 0 still writes the all-zero offsets
}

moe_status moe_expert_ffn_q(const moe_layer* layer, const void* x, int32_t T, const int32_t* topk_ids,
                            const int32_t* expert_offsets, const int32_t* sorted_pairs, float* expert_out,
                            float* shared_out_opt, void* h_opt, void* shared_h_opt, void* ws, size_t ws_bytes,
                            void* stream) {
  MOE_TRY(check_layer(layer));
  MOE_TRY(check_tokens(layer, T));
  if (T == 0) return MOE_OK;
  if (!x || !topk_ids || !expert_offsets || !sorted_pairs || !expert_out || !aligned(x, 16) ||
      !aligned(expert_out, 16))
    return MOE_E_ARG;
  if ((h_opt && !aligned(h_opt, 16)) || (shared_h_opt && !aligned(shared_h_opt, 16))) return MOE_E_ARG;
  if (shared_out_opt && !aligned(shared_out_opt, 16)) return MOE_E_ARG;
  void* h = h_opt;
  void* hs = shared_h_opt;
  if (!h || (!hs && shared_out_opt)) {
    MOE_TRY(ws_check(*layer, T, ws, ws_bytes));
    const Ws W = ws_layout(*layer, T);
    if (!h) h = at<void>(ws, W.h);
    if (!hs) hs = at<void>(ws, W.hs);
  }
  MOE_TRY(range_check(layer, T, topk_ids, expert_offsets, sorted_pairs, nullptr, stream));
  const bool shared = layer->shared.n == 1 && shared_out_opt != nullptr;
  const FfnArgs fa = ffn_args(*layer, x, T, topk_ids, expert_offsets, sorted_pairs, h, shared ? hs : nullptr,
                              expert_out, shared ? shared_out_opt : nullptr);
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  MOE_TRY(dev(launch_gateup(fa, s)));
  return dev(launch_down(fa, s));
}

moe_status moe_expert_gate_up_q(const moe_layer* layer, const void* x, int32_t T, const int32_t* topk_ids,
                                const int32_t* expert_offsets, const int32_t* sorted_pairs, void* h,
                                void* shared_h_opt, void* stream) {
  MOE_TRY(check_layer(layer));
  MOE_TRY(check_tokens(layer, T));
  if (T == 0) return MOE_OK;
  if (!x || !topk_ids || !expert_offsets || !sorted_pairs || !h || !aligned(x, 16) || !aligned(h, 16))
    return MOE_E_ARG;
  if (shared_h_opt && !aligned(shared_h_opt, 16)) return MOE_E_ARG;
  MOE_TRY(range_check(layer, T, topk_ids, expert_offsets, sorted_pairs, nullptr, stream));
  const bool shared = layer->shared.n == 1 && shared_h_opt != nullptr;
  const FfnArgs fa = ffn_args(*layer, x, T, topk_ids, expert_offsets, sorted_pairs, h,
                              shared ? shared_h_opt : nullptr, nullptr, nullptr);
  return dev(launch_gateup(fa, reinterpret_cast<hipStream_t>(stream)));
}

moe_status moe_expert_down_q(const moe_layer* layer, const void* h, const void* shared_h_opt, int32_t T,
                             const int32_t* topk_ids, const int32_t* expert_offsets, const int32_t* sorted_pairs,
                             float* expert_out, float* shared_out_opt, void* stream) {
  MOE_TRY(check_layer(layer));
  MOE_TRY(check_tokens(layer, T));
  if (T == 0) return MOE_OK;
  if (!h || !topk_ids || !expert_offsets || !sorted_pairs || !expert_out || !aligned(h, 16) ||
      !aligned(expert_out, 16))
    return MOE_E_ARG;
  if ((shared_h_opt && !aligned(shared_h_opt, 16)) || (shared_out_opt && !aligned(shared_out_opt, 16)))
    return MOE_E_ARG;
  if (shared_out_opt && layer->shared.n == 1 && !shared_h_opt) return MOE_E_ARG;
  MOE_TRY(range_check(layer, T, topk_ids, expert_offsets, sorted_pairs, nullptr, stream));
  const bool shared = layer->shared.n == 1 && shared_out_opt != nullptr;
  FfnArgs fa = ffn_args(*layer, nullptr, T, topk_ids, expert_offsets, sorted_pairs, const_cast<void*>(h),
                        shared ? const_cast<void*>(shared_h_opt) : nullptr, expert_out,
                        shared ? shared_out_opt : nullptr);
  return dev(launch_down(fa, reinterpret_cast<hipStream_t>(stream)));
}

moe_status moe_combine(const moe_layer* layer, const float* expert_out, const float* shared_out_opt,
                       const int32_t* pair_pos, const float* topk_w, int32_t T, float* y, const void* x_resid,
                       void* x_next_opt, void* stream) {
  MOE_TRY(check_layer(layer));
  MOE_TRY(check_tokens(layer, T));
  if (T == 0) return MOE_OK;
  if (!expert_out || !pair_pos || !topk_w || !y) return MOE_E_ARG;
  if (!aligned(expert_out, 16) || !aligned(y, 16) || (shared_out_opt && !aligned(shared_out_opt, 16))) return MOE_E_ARG;
  if (x_next_opt && !x_resid) return MOE_E_ARG;
  MOE_TRY(range_check(layer, T, nullptr, nullptr, nullptr, pair_pos, stream));
  const CombineArgs ca{expert_out, shared_out_opt, pair_pos, topk_w, x_resid, x_next_opt, y,
                       T, layer->hidden, layer->top_k, layer->act};
  return dev(launch_combine(ca, reinterpret_cast<hipStream_t>(stream)));
}

moe_status moe_layer_forward(const moe_layer* layer, const void* x, int32_t T, float* y, void* x_next_opt,
                             int32_t* topk_ids_opt, float* topk_w_opt, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_layer(layer));
  MOE_TRY(check_tokens(layer, T));
  if (T == 0) return MOE_OK;
  if (!x || !y || !aligned(x, 16) || !aligned(y, 16)) return MOE_E_ARG;
  MOE_TRY(ws_check(*layer, T, ws, ws_bytes));
  return layer_forward_impl(*layer, x, T, y, x_next_opt, topk_ids_opt, topk_w_opt, ws,
                            reinterpret_cast<hipStream_t>(stream));
}

moe_status moe_stack_forward(const moe_layer* layers, int32_t n_layers, void* x_inout, int32_t T, float* y_last_opt,
                             void* ws, size_t ws_bytes, void* stream) {
  if (!layers || n_layers < 0) return MOE_E_ARG;
  for (int32_t l = 0; l < n_layers; ++l) {
    MOE_TRY(check_layer(&layers[l]));
    MOE_TRY(check_tokens(&layers[l], T));
    if (layers[l].hidden != layers[0].hidden || layers[l].act != layers[0].act) return MOE_E_ARG;
  }
  if (T == 0 || n_layers == 0) return MOE_OK;
  if (!x_inout || !aligned(x_inout, 16) || (y_last_opt && !aligned(y_last_opt, 16))) return MOE_E_ARG;
  for (int32_t l = 0; l < n_layers; ++l) MOE_TRY(ws_check(layers[l], T, ws, ws_bytes));
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  for (int32_t l = 0; l < n_layers; ++l) {
    const Ws W = ws_layout(layers[l], T);
    float* y = (l == n_layers - 1 && y_last_opt) ? y_last_opt : at<float>(ws, W.y);
    MOE_TRY(layer_forward_impl(layers[l], x_inout, T, y, x_inout, nullptr, nullptr, ws, s));
  }
  return MOE_OK;
}

moe_status moe_dequant(const moe_qmat* m, int32_t qfmt, int32_t rows, int32_t cols, float* out, void* stream) {
  if (!m || !out || rows < 0 || cols < 0 || cols % kGroup) return MOE_E_ARG;
  if (qfmt != MOE_Q4_SYM_G32 && qfmt != MOE_Q2_ASYM_G32 && qfmt != MOE_Q3_SYM_G32) return MOE_E_UNSUPPORTED;
  if (!m->codes || !m->scales || (qfmt == MOE_Q2_ASYM_G32 && !m->mins)) return MOE_E_ARG;
  return dev(launch_dequant(qmat(*m), qfmt, rows, cols, out, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
