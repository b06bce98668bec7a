"""CPU oracle of the routed MoE FFN layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path never calls it and it
shares no code with the HIP library.

It is the plain definition of the layer, evaluated in float64 with NumPy, with
the rounding points of the definition written out explicitly:

* the router is a linear gate over the token's hidden state that picks the
  top-K experts of each token; all other experts are skipped (page 2, "Layer 1:
  On-Demand MoE Expert Scheduling"; page 3, "The 'Doorbell' Mechanism": the
  GPU decides which 10 experts a token needs);
* 512 experts per layer, 10 routed plus one always-active shared expert per
  token (page 3, "How Strata Makes Your Entire PC Work Together"; page 5, "The
  model is large on paper, sparse in practice");
* expert weights are stored with 4 or 2 bits per weight in groups (page 1,
  "How Strata Makes the Impossible Possible" and "Quantization Configuration
  Example", symmetric grouping; page 3, "A Few Things to Keep in Perspective").

Where the pages are silent this oracle takes these readings (each is listed
with its reason in the design notes of the repository):
  gate scores = softmax over the selected logits (softmax, top-k, renormalise);
  ties go to the lower expert index; the router bias enters before selection;
  experts are SwiGLU FFNs without biases; the intermediate activation h is
  rounded to the activation storage type; the shared expert enters with
  weight 1; y is summed shared-first then slot 0..K-1.

Every function below cites what it follows.  All arrays are float64 unless
stated; integer outputs are int64.
"""
from __future__ import annotations

import numpy as np

GROUP = 32
Q4 = "q4_sym_g32"
Q2 = "q2_asym_g32"
Q3 = "q3_sym_g32"
ACT_F32 = "f32"
ACT_BF16 = "bf16"


# ----------------------------------------------------------------------------
# rounding points

def round_f32(a):
    """Round float64 values to the nearest float32 (ties to even); return float64."""
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_bf16(a):
    """Round to bfloat16 through float32, nearest-even at each step; return float64."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    bits = f.view(np.uint32).astype(np.uint64)
    keep = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) << 16
    return keep.astype(np.uint32).view(np.float32).astype(np.float64)


def round_act(a, act):
    """Storage rounding of an activation (x or h): bf16 or fp32."""
    if act == ACT_BF16:
        return round_bf16(a)
    if act == ACT_F32:
        return round_f32(a)
    raise ValueError(act)


def fp16_to_f64(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


# ----------------------------------------------------------------------------
# dequantisation of the group-32 formats (page 1 "Quantization Configuration
# Example": symmetric grouped 4-bit; page 3: 2-bit; page 4 "In brief -- 5 key
# takeaways" and page 5 "A sensible 4090 setup": a 3-bit quality tier, whose
# codebook formats the pages do not give -- a plain symmetric 3-bit group-32
# format stands in for it)

def unpack_q4(codes):
    """uint8 [..., C/2] -> codes u in 0..15, [..., C]; element 2j is the low nibble of byte j."""
    c = np.asarray(codes, dtype=np.uint8)
    u = np.empty(c.shape[:-1] + (2 * c.shape[-1],), dtype=np.int64)
    u[..., 0::2] = c & 0x0F
    u[..., 1::2] = c >> 4
    return u


def unpack_q2(codes):
    """uint8 [..., C/4] -> codes u in 0..3, [..., C]; element 4j+i sits in bits 2i+1..2i of byte j."""
    c = np.asarray(codes, dtype=np.uint8)
    u = np.empty(c.shape[:-1] + (4 * c.shape[-1],), dtype=np.int64)
    for i in range(4):
        u[..., i::4] = (c >> (2 * i)) & 3
    return u


def unpack_q3(codes):
    """uint8 [..., 3C/8] -> codes u in 0..7, [..., C].

    Each 32-element group occupies 12 consecutive bytes: bytes 0..7 hold the
    low two bits of the codes in the 2-bit layout (element 4j+i at bits
    2i+1..2i of byte j), bytes 8..11 the third bit (element i at bit i mod 8
    of byte 8 + i div 8); u = low + 4 high.
    """
    c = np.asarray(codes, dtype=np.uint8)
    g = c.reshape(c.shape[:-1] + (c.shape[-1] // 12, 12))
    low = unpack_q2(g[..., :8])                    # [..., G, 32]
    high = np.empty_like(low)
    for i in range(32):
        high[..., i] = (g[..., 8 + i // 8] >> (i % 8)) & 1
    u = low + 4 * high
    return u.reshape(c.shape[:-1] + (u.shape[-2] * 32,))


def _per_group(plane, cols):
    """fp16 plane [..., cols/32] -> float64 [..., cols], each value repeated over its group."""
    return np.repeat(fp16_to_f64(plane), GROUP, axis=-1)[..., :cols]


def dequant_q4(codes, scales):
    """w = s * (u - 8): exact in float64 and representable in float32 (11-bit x 4-bit)."""
    u = unpack_q4(codes)
    return _per_group(scales, u.shape[-1]) * (u - 8).astype(np.float64)


def dequant_q2(codes, scales, mins):
    """w = fp32(s * u + m): the exact value s*u + m (float64 holds it) rounded once to float32."""
    u = unpack_q2(codes)
    cols = u.shape[-1]
    return round_f32(_per_group(scales, cols) * u.astype(np.float64) + _per_group(mins, cols))


def dequant_q3(codes, scales):
    """w = s * (u - 4): exact in float64 and representable in float32 (11-bit x 3-bit)."""
    u = unpack_q3(codes)
    return _per_group(scales, u.shape[-1]) * (u - 4).astype(np.float64)


def dequant(codes, scales, mins, qfmt):
    if qfmt == Q4:
        return dequant_q4(codes, scales)
    if qfmt == Q3:
        return dequant_q3(codes, scales)
    if qfmt == Q2:
        return dequant_q2(codes, scales, mins)
    raise ValueError(qfmt)


# ----------------------------------------------------------------------------
# router (page 2 "Layer 1": a light gating network picks the top-K experts per
# token; page 3 "Doorbell": the ids of the chosen experts are the router's output)

def router_logits(x, w_r, b):
    """l[t,e] = sum_i W_r[e,i] x[t,i] + b[e] in float64."""
    l = np.asarray(x, np.float64) @ np.asarray(w_r, np.float64).T
    if b is not None:
        l = l + np.asarray(b, np.float64)[None, :]
    return l


def select_topk(logits, k):
    """ids[t, 0..K-1]: experts ordered by logit descending, ties to the lower index.

    A stable sort of -l keeps equal logits in index order, which is the key
    (-l, e) ascending.
    """
    l = np.asarray(logits, np.float64)
    order = np.argsort(-l, axis=-1, kind="stable")
    return order[..., :k].astype(np.int64)


def topk_weights(logits, ids):
    """w[t,k] = exp(l_k - l_0) / sum_j exp(l_j - l_0) over the K selected logits.

    Equal to the full softmax over all E logits renormalised over the K
    selected experts (the full denominator cancels).
    """
    sel = np.take_along_axis(np.asarray(logits, np.float64), np.asarray(ids), axis=-1)
    z = np.exp(sel - sel[..., :1])
    return z / z.sum(axis=-1, keepdims=True)


# ----------------------------------------------------------------------------
# token -> expert permutation (per-expert dispatch: page 3 "Doorbell", experts
# are dispatched by id)

def permute(ids, n_experts):
    """Stable counting sort of the pairs p = t*K + k by expert.

    Returns expert_offsets [E+1] (exclusive prefix sum of per-expert counts),
    sorted_pairs [T*K] (pairs by (expert, p) ascending) and pair_pos [T*K]
    (position of pair p in sorted_pairs).
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=n_experts)[:n_experts]
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_pairs = np.argsort(flat, kind="stable").astype(np.int64)
    pair_pos = np.empty_like(sorted_pairs)
    pair_pos[sorted_pairs] = np.arange(flat.size, dtype=np.int64)
    return offsets, sorted_pairs, pair_pos


# ----------------------------------------------------------------------------
# expert FFN (SwiGLU: h = silu(W_g x) * (W_u x), o = W_d h)

def silu(z):
    z = np.asarray(z, np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(xrows, wg, wu, wd, act, h=None):
    """o = W_d round_act(silu(W_g x) * (W_u x)) for each row of ``xrows`` [n][H].

    Returns (o, h, v) with v the value of silu(g) * u before rounding.  If ``h``
    is given it replaces the rounded intermediate (teacher forcing at the
    rounding point); v is still computed.
    """
    g = np.asarray(xrows, np.float64) @ wg.T
    u = np.asarray(xrows, np.float64) @ wu.T
    v = silu(g) * u
    if h is None:
        h = round_act(v, act)
    return np.asarray(h, np.float64) @ wd.T, np.asarray(h, np.float64), v


# ----------------------------------------------------------------------------
# the layer

def expert_weights(es, e, qfmt):
    """Dequantised (gate, up, down) of expert id ``e`` of an ExpertSet (by id if the set is indexed)."""
    j = int(e)
    if len(es.index):
        j = int(np.nonzero(es.index == e)[0][0])
    return tuple(dequant(m.codes[j], m.scales[j], None if m.mins is None else m.mins[j], qfmt)
                 for m in (es.gate, es.up, es.down))


def layer_forward(layer, x, ids=None, keep_expert_out=True, h=None, shared_h=None):
    """The routed MoE FFN layer on the exact activations ``x`` [T][H].

    ``layer`` is a synth.LayerData (router, routed experts -- all, or a subset
    covering every id that is used -- and the shared expert).  ``ids`` (T x K)
    overrides the selection for the downstream steps; logits and weights are
    still computed from the oracle's logits at those ids.

    ``h`` ([T*K][I], sorted order) and ``shared_h`` ([T][I]) replace the
    rounded intermediate activations of the routed and shared experts if given.

    Returns a dict with logits, ids, w, offsets, sorted_pairs, pair_pos,
    expert_out (o rows in sorted order), h and h_pre (sorted order, after and
    before rounding), shared_out, shared_h, shared_h_pre and y, all float64 /
    int64.
    """
    spec = layer.spec
    act, k, e_n = spec.act, spec.top_k, spec.n_experts
    x = np.asarray(x, np.float64)
    t_n, hdim = x.shape
    logits = router_logits(x, layer.router_w, layer.router_b)
    sel = select_topk(logits, k) if ids is None else np.asarray(ids, np.int64).reshape(t_n, k)
    w = topk_weights(logits, sel)
    offsets, sorted_pairs, pair_pos = permute(sel, e_n)

    o = np.zeros((t_n * k, hdim)) if keep_expert_out else None
    hs = np.zeros((t_n * k, spec.inter)) if keep_expert_out else None
    hv = np.zeros((t_n * k, spec.inter)) if keep_expert_out else None
    o_by_pair = np.zeros((t_n * k, hdim))
    for e in range(e_n):
        lo, hi = offsets[e], offsets[e + 1]
        if lo == hi:
            continue
        pairs = sorted_pairs[lo:hi]
        wg, wu, wd = expert_weights(layer.routed, e, spec.qfmt)
        oe, he, ve = expert_ffn(x[pairs // k], wg, wu, wd, act, None if h is None else h[lo:hi])
        o_by_pair[pairs] = oe
        if keep_expert_out:
            o[lo:hi] = oe
            hs[lo:hi] = he
            hv[lo:hi] = ve

    shared_out = np.zeros((t_n, hdim))
    sh, shv = [], []
    for j in range(layer.shared.n):
        wg, wu, wd = expert_weights(layer.shared, layer.shared.index[j] if len(layer.shared.index) else j,
                                    spec.qfmt)
        sj, hj, vj = expert_ffn(x, wg, wu, wd, act, None if shared_h is None else shared_h)
        shared_out = shared_out + sj
        sh.append(hj)
        shv.append(vj)

    y = combine(shared_out, o_by_pair.reshape(t_n, k, hdim), w)
    return dict(logits=logits, ids=sel, w=w, offsets=offsets, sorted_pairs=sorted_pairs,
                pair_pos=pair_pos, expert_out=o, h=hs, h_pre=hv, shared_out=shared_out,
                shared_h=sh, shared_h_pre=shv, y=y)


def combine(shared_out, o_tk, w):
    """y_t = s_t + sum_{k=0}^{K-1} w[t,k] o[t,k], accumulated in that order."""
    y = np.array(shared_out, dtype=np.float64, copy=True)
    for kk in range(o_tk.shape[1]):
        y = y + w[:, kk:kk + 1] * o_tk[:, kk, :]
    return y


def residual_step(x, y):
    """Stack wiring between MoE layers: x_next = bf16(fp32(x + y))."""
    return round_bf16(round_f32(np.asarray(x, np.float64) + np.asarray(y, np.float64)))


# ----------------------------------------------------------------------------
# helpers for comparing against an fp32 implementation of the router

def router_error_bound(x, w_r, b, parts=1):
    """beta[t,e] = gamma_n (c sum_i |W_r[e,i] x[t,i]| + |b_e|), gamma_n = n u / (1 - n u), u = 2^-24.

    Worst-case bound on the error of an fp32 evaluation of the logit with exact
    (float64-representable) inputs, in any summation order, for two forms of
    the evaluation:

    * ``parts=1``: an fp32 dot product of length H plus the bias: n = H + 1,
      c = 1 (each product is exact in fp32 or rounded once, each of the H
      additions rounds once);
    * ``parts=3``: each fp32 weight split exactly into three bf16 parts
      (hi + mid + lo = w, |hi| + |mid| + |lo| <= (1 + 2^-6) |w|), the 3 H exact
      products of x with the parts summed in fp32, plus the bias:
      n = 3 H + 1, c = 1 + 2^-6.
    """
    if parts not in (1, 3):
        raise ValueError(parts)
    hdim = np.asarray(x).shape[-1]
    n = parts * hdim + 1
    u = 2.0 ** -24
    gamma = n * u / (1 - n * u)
    c = 1.0 if parts == 1 else 1.0 + 2.0 ** -6
    mag = c * (np.abs(np.asarray(x, np.float64)) @ np.abs(np.asarray(w_r, np.float64)).T)
    if b is not None:
        mag = mag + np.abs(np.asarray(b, np.float64))[None, :]
    return gamma * mag


def certify_ids(logits, beta, ids_a, ids_b):
    """Are two top-K id lists both consistent with the exact logits, up to the error bound?

    Returns (ok, differs): ``differs`` marks tokens whose id lists are not
    identical; ``ok`` is False if some difference is not a near-tie, i.e.
    if for a position where the lists differ the exact logit gap exceeds the
    combined bound of the two experts involved.
    """
    ids_a = np.asarray(ids_a, np.int64)
    ids_b = np.asarray(ids_b, np.int64)
    differs = np.any(ids_a != ids_b, axis=-1)
    ok = True
    for t in np.nonzero(differs)[0]:
        la, lb = logits[t, ids_a[t]], logits[t, ids_b[t]]
        ba, bb = beta[t, ids_a[t]], beta[t, ids_b[t]]
        # slot by slot, the two choices must be interchangeable within the bound
        if np.any(np.abs(la - lb) > ba + bb):
            ok = False
    return ok, differs
