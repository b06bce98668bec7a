/*
 * moe.h -- C ABI of the routed Mixture-of-Experts FFN layer on MI355X (gfx950).
 *
 * The layer (page 2 "Layer 1: On-Demand MoE Expert Scheduling"; page 3 "How
 * Strata Makes Your Entire PC Work Together" and "The 'Doorbell' Mechanism";
 * page 5 "The model is large on paper, sparse in practice"): a router scores
 * every expert for each token, the top-K experts are selected (10 of 512 on
 * the pages), each selected expert -- a SwiGLU FFN with low-bit group-quantized
 * weights (page 1 "How Strata Makes the Impossible Possible", page 3 "A Few
 * Things to Keep in Perspective": 4-bit or 2-bit) -- processes the token, an
 * always-active shared expert processes every token, and the expert outputs
 * are summed with the renormalised router weights.  Selected expert ids stay in
 * device memory and are consumed there; nothing returns to the host.
 *
 * Conventions for every call:
 *   - All array pointers are DEVICE pointers unless stated otherwise.  The
 *     caller owns every buffer (weights, activations, outputs, workspace); the
 *     library allocates nothing and keeps no pointer after the call returns.
 *     Buffers must stay valid until the work enqueued on `stream` completes.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls validate their
 *     arguments on the host, enqueue kernels on `stream` and return without
 *     synchronising.  On an argument error nothing is enqueued.
 *   - Return codes: MOE_OK; MOE_E_ARG (NULL required pointer, T < 0, K < 1 or
 *     K > E, a size that is not a multiple of 32, inconsistent descriptor);
 *     MOE_E_UNSUPPORTED (a valid but unsupported size or format);
 *     MOE_E_WORKSPACE (workspace smaller than moe_workspace_bytes);
 *     MOE_E_DEVICE (a HIP launch error, read from hipGetLastError).  Faults
 *     inside kernels surface at the caller's next synchronisation.
 *   - T == 0 is a valid no-op.  Expert ids handed to moe_permute /
 *     moe_expert_ffn_q must lie in [0, E); others are undefined behaviour in
 *     the release library and MOE_E_ARG in the debug library
 *     (moe_range_checks).
 *   - Activations: x and the intermediate h are stored in the layer's
 *     activation type (bf16 bits or fp32); router weights, combine weights and
 *     outputs are fp32.  Accumulation is fp32.
 *   - Thread safety: the only global state is the per-device address of the
 *     array behind moe_layer_forward_noalloc, looked up once under a lock;
 *     other calls on distinct streams with distinct outputs and workspaces may
 *     run concurrently.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_E_ARG = 1,
  MOE_E_UNSUPPORTED = 2,
  MOE_E_WORKSPACE = 3,
  MOE_E_DEVICE = 4
} moe_status;

/* Packed weight formats.  Groups of 32 consecutive elements run along the
 * last (reduction) dimension of each row-major matrix.
 *   MOE_Q4_SYM_G32: byte j of a row holds element 2j in bits 3..0 and element
 *     2j+1 in bits 7..4 as u = q + 8 (u in 0..15); w = s * (u - 8) with s the
 *     group's fp16 scale.  (Symmetric grouped 4-bit: page 1 "Quantization
 *     Configuration Example".)
 *   MOE_Q2_ASYM_G32: byte j holds elements 4j..4j+3 in bits 1..0, 3..2, 5..4,
 *     7..6 (u in 0..3); w = fp32(s * u + m) with the group's fp16 scale s and
 *     fp16 minimum m.  (2-bit weights: page 3 "A Few Things to Keep in
 *     Perspective".)
 *   MOE_Q3_SYM_G32: each group of 32 elements is 12 consecutive bytes: bytes
 *     0..7 hold the two low bits of the codes in the 2-bit layout (element
 *     4j+i at bits 2i+1..2i of byte j), bytes 8..11 the third bit (element i
 *     at bit i mod 8 of byte 8 + i div 8); u = low + 4 high (0..7) and
 *     w = s * (u - 4) with the group's fp16 scale s.  (The pages' 3-bit
 *     quality tier, page 4 "In brief -- 5 key takeaways" and page 5 "A
 *     sensible 4090 setup", uses codebook formats the pages do not give; this
 *     plain symmetric format stands in for it.) */
typedef enum moe_qfmt { MOE_Q4_SYM_G32 = 1, MOE_Q2_ASYM_G32 = 2, MOE_Q3_SYM_G32 = 3 } moe_qfmt;

/* Storage type of activations x and of the expert intermediate h. */
typedef enum moe_act { MOE_ACT_F32 = 0, MOE_ACT_BF16 = 1 } moe_act;

/* One packed matrix kind for n experts, rows x cols each, expert e at a fixed
 * stride: codes  [n][rows][cols*bits/8] uint8,
 *         scales [n][rows][cols/32]     fp16 bits,
 *         mins   [n][rows][cols/32]     fp16 bits (2-bit format only, else NULL).
 * (bits = 4, 3 or 2; a 3-bit row is cols/32 groups of 12 bytes.) */
typedef struct moe_qmat {
  const uint8_t *codes;
  const uint16_t *scales;
  const uint16_t *mins;
} moe_qmat;

/* n SwiGLU experts: gate, up [n][inter][hidden]; down [n][hidden][inter]. */
typedef struct moe_experts {
  moe_qmat gate, up, down;
  int32_t n;
} moe_experts;

/* Host descriptor of one layer; read during each call, not retained. */
typedef struct moe_layer {
  int32_t hidden;      /* H, multiple of 32, <= 4096                        */
  int32_t inter;       /* I, expert intermediate size, multiple of 32, <= 4096 */
  int32_t n_experts;   /* E routed experts, 1..8192                         */
  int32_t top_k;       /* K, 1..E                                           */
  int32_t qfmt;        /* moe_qfmt                                          */
  int32_t act;         /* moe_act                                           */
  const float *router_w; /* [E][H] fp32, row-major                          */
  const float *router_b; /* [E] fp32 added to the logits, or NULL           */
  moe_experts routed;  /* n == E                                            */
  moe_experts shared;  /* n == 1 (always-active shared expert) or 0 (none)  */
  int32_t hot_experts; /* >= 0: cache policy of the expert weights (results  */
                       /* do not depend on it).  The pages keep the most     */
                       /* used experts resident near the GPU (page 2 "Layer */
                       /* 1: On-Demand MoE Expert Scheduling"; page 5 "The  */
                       /* desktop becomes a memory system").  With the       */
                       /* experts numbered by decreasing popularity, experts */
                       /* 0 .. hot_experts-1 and the shared expert are read  */
                       /* with the default (cache-allocating) policy, so     */
                       /* that they can stay in the last-level cache across  */
                       /* calls, and the others non-temporally.  0: every    */
                       /* expert streams (non-temporal).                     */
} moe_layer;

/* Router + top-K + weights (page 2 "Layer 1": the gating network picks the
 * top-K experts of each token; page 3 "The 'Doorbell' Mechanism": the device
 * decides the 10 expert ids of a token).
 *   logits[t][e] = sum_i router_w[e][i] * x[t][i] + router_b[e]   (fp32)
 *   topk_ids[t][0..K-1] = experts by logit descending, equal logits -> lower id
 *   topk_w[t][k] = exp(l_k - l_0) / sum_j exp(l_j - l_0)  (softmax over all E
 *                  logits renormalised over the K selected; sums to 1)
 * x [T][H] act type; topk_ids [T][K] int32; topk_w [T][K] fp32;
 * logits_opt [T][E] fp32 or NULL (then the logits live in the workspace).
 * Workspace: at least moe_workspace_bytes(layer, T). */
moe_status moe_router_topk(const moe_layer *layer, const void *x, int32_t T,
                           int32_t *topk_ids, float *topk_w, float *logits_opt,
                           void *ws, size_t ws_bytes, void *stream);

/* Token -> expert permutation: stable counting sort of the T*K (token, slot)
 * pairs p = t*K + k by expert id (dispatch of each token to its experts,
 * page 3 "The 'Doorbell' Mechanism").
 *   expert_offsets [E+1]: exclusive prefix sum of per-expert pair counts,
 *                         expert_offsets[E] = T*K
 *   sorted_pairs   [T*K]: pairs ordered by (expert, p)
 *   pair_pos       [T*K]: pair_pos[p] = index of p in sorted_pairs
 * All int32.  Workspace: at least moe_workspace_bytes(layer, T). */
moe_status moe_permute(const moe_layer *layer, const int32_t *topk_ids, int32_t T,
                       int32_t *expert_offsets, int32_t *sorted_pairs, int32_t *pair_pos,
                       void *ws, size_t ws_bytes, void *stream);

/* Expert FFNs on the permuted pairs: for sorted position j with pair
 * p = sorted_pairs[j], token t = p / K and expert e = topk_ids[p]
 * (expert_offsets[e] <= j < expert_offsets[e+1]), i.e. the outputs of
 * moe_router_topk and moe_permute:
 *   h = round_act(silu(W_g[e] x_t) * (W_u[e] x_t)),  silu(z) = z / (1 + exp(-z))
 *   expert_out[j] = W_d[e] h                         (fp32, [T*K][H])
 * and, if the layer has a shared expert and shared_out_opt != NULL, the same
 * FFN with the shared weights for every token: shared_out_opt[t] ([T][H] fp32).
 * (SwiGLU expert sub-networks, page 2 "Layer 1"; shared expert, page 5.)
 * Weights are dequantised in registers; x and h are consumed in the act type.
 * h_opt ([T*K][I] act type, sorted order) and shared_h_opt ([T][I] act type)
 * receive the intermediate activations h if non-NULL (otherwise they live in
 * the workspace); shared_h_opt is only written when shared_out_opt is given.
 * Workspace: at least moe_workspace_bytes(layer, T). */
moe_status moe_expert_ffn_q(const moe_layer *layer, const void *x, int32_t T, const int32_t *topk_ids,
                            const int32_t *expert_offsets, const int32_t *sorted_pairs,
                            float *expert_out, float *shared_out_opt,
                            void *h_opt, void *shared_h_opt,
                            void *ws, size_t ws_bytes, void *stream);

/* The two halves of moe_expert_ffn_q, one kernel each.
 * moe_expert_gate_up_q: h[j] = round_act(silu(W_g[e] x_t) * (W_u[e] x_t)) for
 *   every sorted position j (h [T*K][I] act type), and for the shared expert
 *   shared_h_opt[t] ([T][I]) if non-NULL and the layer has one.
 * moe_expert_down_q: expert_out[j] = W_d[e] h[j] ([T*K][H] fp32), and
 *   shared_out_opt[t] = W_d^shared shared_h_opt[t] if shared_out_opt is given
 *   (then shared_h_opt is required).
 * Both read topk_ids, expert_offsets and sorted_pairs as moe_expert_ffn_q does.
 * No workspace.  (Rows "fused dequant gate/up + SwiGLU" and "fused dequant down
 * projection" of the expert sub-network, page 2 "Layer 1".) */
moe_status moe_expert_gate_up_q(const moe_layer *layer, const void *x, int32_t T, const int32_t *topk_ids,
                                const int32_t *expert_offsets, const int32_t *sorted_pairs,
                                void *h, void *shared_h_opt, void *stream);
moe_status moe_expert_down_q(const moe_layer *layer, const void *h, const void *shared_h_opt, int32_t T,
                             const int32_t *topk_ids, const int32_t *expert_offsets,
                             const int32_t *sorted_pairs, float *expert_out, float *shared_out_opt,
                             void *stream);

/* Weighted combine:
 *   y[t] = shared_out[t] + sum_{k=0..K-1} topk_w[t][k] * expert_out[pair_pos[t*K+k]]
 * accumulated in fp32 in exactly that order (shared first, then slot 0..K-1),
 * so results are bitwise reproducible.  shared_out_opt may be NULL (term
 * omitted).  If x_next_opt != NULL it receives round_act(fp32(x_resid[t] + y[t]))
 * -- the residual stream into the next layer -- and x_resid (act type [T][H])
 * must be given; x_next_opt may alias x_resid.  y [T][H] fp32. */
moe_status moe_combine(const moe_layer *layer, const float *expert_out, const float *shared_out_opt,
                       const int32_t *pair_pos, const float *topk_w, int32_t T,
                       float *y, const void *x_resid, void *x_next_opt, void *stream);

/* The whole layer: router/top-K, permutation, expert FFNs, shared expert and
 * combine, all on `stream` with no host synchronisation.  y [T][H] fp32.
 * x_next_opt (act type [T][H], may alias x) receives round_act(fp32(x + y)) if
 * non-NULL.  topk_ids_opt / topk_w_opt ([T][K]) receive the routing if
 * non-NULL.  Workspace: at least moe_workspace_bytes(layer, T). */
moe_status moe_layer_forward(const moe_layer *layer, const void *x, int32_t T,
                             float *y, void *x_next_opt,
                             int32_t *topk_ids_opt, float *topk_w_opt,
                             void *ws, size_t ws_bytes, void *stream);

/* Size of the device array moe_layer_forward_noalloc uses in place of a
 * workspace: 16 MiB, enough for about 145 tokens of the 512-expert layer
 * (hidden 2048, intermediate 768, top-10 + shared, bf16). */
#define MOE_NOALLOC_SCRATCH_BYTES (16u << 20)

/* moe_layer_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops or
 * harnesses that must not call the allocator).  Same arguments and results as
 * moe_layer_forward (the same kernels run); the intermediate buffers live in a
 * library-owned device array of MOE_NOALLOC_SCRATCH_BYTES, one per GPU, held
 * until the process ends.  The call allocates nothing: the first call on a
 * device looks the array's address up (with that device current) and keeps
 * it.  Returns MOE_E_WORKSPACE when the layer needs more than the array at T
 * tokens (moe_workspace_bytes(layer, T) > MOE_NOALLOC_SCRATCH_BYTES), and
 * MOE_E_DEVICE if the address lookup fails.  Every call on a GPU shares that
 * GPU's array: calls that overlap on one device (concurrent streams, threads)
 * race and must be serialised by the caller. */
moe_status moe_layer_forward_noalloc(const moe_layer *layer, const void *x, int32_t T,
                                     float *y, void *x_next_opt,
                                     int32_t *topk_ids_opt, float *topk_w_opt, void *stream);

/* Bytes of workspace the calls above need for up to T_max tokens (host-only,
 * pure function of the shapes; returns 0 for an invalid descriptor). */
size_t moe_workspace_bytes(const moe_layer *layer, int32_t T_max);

/* n_layers MoE layers applied in sequence to a residual stream held in the act
 * type: x <- round_act(fp32(x + layer_l(x))) for l = 0..n_layers-1, x_inout
 * [T][H] updated in place.  `layers` is a HOST array of n_layers descriptors
 * (all with the same H, act).  y_last_opt [T][H] fp32 receives the last
 * layer's y if non-NULL.  Workspace: max over layers of moe_workspace_bytes. */
moe_status moe_stack_forward(const moe_layer *layers, int32_t n_layers, void *x_inout, int32_t T,
                             float *y_last_opt, void *ws, size_t ws_bytes, void *stream);

/* Test hook: dequantise rows x cols of one packed matrix (expert 0 of `m`)
 * into out [rows][cols] fp32, with the format's definition (Q4: s*(u-8);
 * Q2: fmaf(s, u, m), one rounding). */
moe_status moe_dequant(const moe_qmat *m, int32_t qfmt, int32_t rows, int32_t cols,
                       float *out, void *stream);

/* Human-readable name of a status code (static string). */
const char *moe_status_str(moe_status s);

/* ABI version, bumped on any change of the structs or signatures above. */
int32_t moe_abi_version(void);

/* 1 in the debug library (libmoe_debug.so), 0 in the release library.  The
 * debug library range-checks, on the device, the routing arrays a caller
 * hands to moe_permute (ids in [0, E)), moe_expert_ffn_q /
 * moe_expert_gate_up_q / moe_expert_down_q (ids; offsets a non-decreasing
 * run from 0 to T*K; sorted pairs in [0, T*K)) and moe_combine (pair
 * positions in [0, T*K)) before any kernel indexes with them, and returns
 * MOE_E_ARG with nothing else enqueued when one is out of range.  The check
 * synchronises the stream (the call then returns after the check has run), so
 * those calls cannot be captured in a HIP graph in the debug library.  (The
 * ids pick among the E experts, page 2 "Layer 1".) */
int32_t moe_range_checks(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
