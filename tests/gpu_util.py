"""Helpers for the GPU parity tests: drive the C ABI on device tensors and
compare every step with the CPU oracle.  Imported by tests only."""
from __future__ import annotations

import sys

import numpy as np
import torch

import synth
from oracle import moe_oracle as mo
from sparse_moe_router_amd import api
from synth import torch_io

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device_layer(ld: synth.LayerData, device=DEV) -> api.Layer:
    return api.Layer(**torch_io.layer_kwargs(ld, device))


def x_dev(x: synth.Activations, act: str, device=DEV):
    return torch_io.x_tensor(x.storage, act, device)


def run_steps(L: api.Layer, x: torch.Tensor, T: int, with_shared=True):
    """The five ABI calls one after the other; returns host numpy results."""
    dev = x.device
    E, K, H = L.n_experts, L.top_k, L.hidden
    ws = api.workspace(L, max(T, 1), dev)
    ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    w = torch.empty((T, K), dtype=torch.float32, device=dev)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    api.moe_router_topk(L, x, T, ids, w, logits, ws)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sp = torch.empty(T * K, dtype=torch.int32, device=dev)
    pp = torch.empty(T * K, dtype=torch.int32, device=dev)
    api.moe_permute(L, ids, T, off, sp, pp, ws)
    o = torch.empty((T * K, H), dtype=torch.float32, device=dev)
    so = torch.empty((T, H), dtype=torch.float32, device=dev) if with_shared else None
    hh = torch.empty((T * K, L.inter), dtype=L.act_dtype, device=dev)
    hs = torch.empty((T, L.inter), dtype=L.act_dtype, device=dev) if with_shared else None
    api.moe_expert_ffn_q(L, x, T, ids, off, sp, o, so, hh, hs, ws)
    y = torch.empty((T, H), dtype=torch.float32, device=dev)
    api.moe_combine(L, o, so, pp, w, T, y)
    torch.cuda.synchronize()
    h = lambda t: None if t is None else t.cpu().numpy()
    f = lambda t: None if t is None else t.float().cpu().numpy().astype(np.float64)
    return dict(ids=h(ids).astype(np.int64), w=h(w), logits=h(logits), offsets=h(off), sorted_pairs=h(sp),
                pair_pos=h(pp), expert_out=h(o), shared_out=h(so), y=h(y), h=f(hh), shared_h=f(hs))


def run_forward(L: api.Layer, x: torch.Tensor, T: int, x_next=False):
    dev = x.device
    ws = api.workspace(L, max(T, 1), dev)
    y = torch.empty((T, L.hidden), dtype=torch.float32, device=dev)
    ids = torch.empty((T, L.top_k), dtype=torch.int32, device=dev)
    w = torch.empty((T, L.top_k), dtype=torch.float32, device=dev)
    xn = torch.empty_like(x[:T]) if x_next else None
    api.moe_layer_forward(L, x, T, y, xn, ids, w, ws)
    torch.cuda.synchronize()
    return dict(y=y.cpu().numpy(), ids=ids.cpu().numpy().astype(np.int64), w=w.cpu().numpy(),
                x_next=None if xn is None else xn.cpu())


# bf16 activations and at least this many tokens: the library evaluates the
# logits on the matrix cores with each fp32 weight split into three bf16 parts
ROUTER_MFMA_MIN_TOKENS = 64


def router_parts(spec, T):
    """Parts per weight of the library's logit evaluation for a call of T tokens:
    3 on the matrix-core path (bf16 x, T >= 64, H a multiple of 64), else 1
    (an fp32 dot product)."""
    return 3 if spec.act == synth.ACT_BF16 and T >= ROUTER_MFMA_MIN_TOKENS and spec.hidden % 64 == 0 else 1


def check_routing(ld: synth.LayerData, xv: np.ndarray, gpu: dict, tokens=None):
    """Router logits within the fp32 bound, ids identical to the oracle's
    selection on the GPU's own fp32 logits, and identical (or a certified
    near-tie) to the selection on exact logits.  Returns the number of tokens
    whose ids differ from the exact-logit selection."""
    spec = ld.spec
    tok = np.arange(xv.shape[0]) if tokens is None else np.asarray(tokens)
    exact = mo.router_logits(xv[tok], ld.router_w, ld.router_b)
    beta = mo.router_error_bound(xv[tok], ld.router_w, ld.router_b, parts=router_parts(spec, xv.shape[0]))
    lg = gpu["logits"][tok].astype(np.float64)
    assert np.all(np.abs(lg - exact) <= beta), "router logits outside the fp32 error bound"
    ids_gpu = gpu["ids"][tok]
    assert np.array_equal(mo.select_topk(lg, spec.top_k), ids_gpu), "top-k differs from selection on the same logits"
    w_same = mo.topk_weights(lg, ids_gpu)
    assert np.abs(gpu["w"][tok] - w_same).max() <= 1e-6
    assert np.all(np.abs(gpu["w"][tok].astype(np.float64).sum(-1) - 1) <= spec.top_k * 2.0 ** -23)
    ok, differs = mo.certify_ids(exact, beta, ids_gpu, mo.select_topk(exact, spec.top_k))
    assert ok, "GPU ids differ from the exact selection beyond a near-tie"
    return int(differs.sum())


def check_permutation(gpu: dict, E: int):
    off, sp, pp = mo.permute(gpu["ids"], E)
    assert np.array_equal(gpu["offsets"], off)
    assert np.array_equal(gpu["sorted_pairs"], sp)
    assert np.array_equal(gpu["pair_pos"], pp)


def rel_err(got, want):
    want = np.asarray(want, np.float64)
    rms = np.sqrt(np.mean(want * want))
    err = np.abs(np.asarray(got, np.float64) - want).max()
    return err / rms if rms > 0 else err, rms


def check_y(ld, xv, gpu, tol=2e-3, tokens=None):
    """y against the oracle evaluated with the GPU's (certified) ids."""
    tok = np.arange(xv.shape[0]) if tokens is None else np.asarray(tokens)
    ref = mo.layer_forward(ld, xv[tok], ids=gpu["ids"][tok], keep_expert_out=tokens is None)
    r, rms = rel_err(gpu["y"][tok], ref["y"])
    assert rms > 0
    assert r <= tol, f"max|dy| = {r:.3e} x RMS(y) exceeds {tol}"
    return ref, r


def _half_step(v, act):
    """Half the spacing of the storage type at |v| (bf16: 8 significant bits, fp32: 24)."""
    e = np.floor(np.log2(np.maximum(np.abs(v), 1e-38)))
    return 2.0 ** (e - (8 if act == synth.ACT_BF16 else 24))


def _silu_prime(g):
    s = 1.0 / (1.0 + np.exp(-g))
    return s * (1.0 + g * (1.0 - s))


def certify_h(ld, xv, gpu, tokens_of_rows, experts_of_rows, h_gpu, h_ref, v_ref, es):
    """Check every element where the GPU's rounded intermediate h differs from
    the oracle's: it must be the storage rounding of a value within the fp32
    evaluation error of the exact pre-rounding value v, i.e.
    |h_gpu - v| <= dv + half a storage step at h_gpu.

    Error model of the GPU's fp32 evaluation of v = silu(g) u:
    dv <= |silu'(g) u| e_g + |silu(g)| e_u + 2^-20 |v|, with the dot-product
    error e_g <= 2^-12 sum_i |W_g[r,i] x_i| (a generous multiple of the
    2^-24-per-operation bound that also covers the offset code encoding,
    whose cancelled offset is up to 1.5 sum |x|), likewise e_u.  Near-cancelling g or u make v small and its relative error
    large, so several storage steps can separate the two roundings there.
    Returns the number of differing elements."""
    act = ld.spec.act
    rows, cols = np.nonzero(h_gpu != h_ref)
    if rows.size == 0:
        return 0
    cache = {}
    for j, r in zip(rows.tolist(), cols.tolist()):
        e = int(experts_of_rows[j])
        if e not in cache:
            cache[e] = mo.expert_weights(es, e, ld.spec.qfmt)
        wg, wu, _ = cache[e]
        x = np.asarray(xv[int(tokens_of_rows[j])], np.float64)
        g, u = wg[r] @ x, wu[r] @ x
        sg, su = np.abs(wg[r] * x).sum(), np.abs(wu[r] * x).sum()
        sig = 1.0 / (1.0 + np.exp(-g))
        dv = abs(_silu_prime(g) * u) * 2.0 ** -12 * sg + abs(g * sig) * 2.0 ** -12 * su + 2.0 ** -20 * abs(v_ref[j, r])
        hg = h_gpu[j, r]
        assert abs(hg - v_ref[j, r]) <= dv + _half_step(hg, act), \
            f"h[{j},{r}] = {hg!r} vs exact {v_ref[j, r]!r}: beyond fp32 error + rounding"
    return int(rows.size)


def check_y_teacher_forced(ld, xv, gpu, tol=2e-3):
    """y against the oracle fed the GPU's ids and, after certifying each
    rounding-boundary flip, the GPU's rounded intermediate h.  Returns
    (max|dy|/RMS, flips)."""
    spec = ld.spec
    ref = mo.layer_forward(ld, xv, ids=gpu["ids"])
    k = spec.top_k
    pairs = gpu["sorted_pairs"]
    flips = certify_h(ld, xv, gpu, pairs // k, gpu["ids"].reshape(-1)[pairs], gpu["h"], ref["h"], ref["h_pre"],
                      ld.routed)
    shared_h = None
    if gpu.get("shared_h") is not None and ld.shared.n:
        sid = int(ld.shared.index[0]) if len(ld.shared.index) else 0
        flips += certify_h(ld, xv, gpu, np.arange(xv.shape[0]), np.full(xv.shape[0], sid), gpu["shared_h"],
                           ref["shared_h"][0], ref["shared_h_pre"][0], ld.shared)
        shared_h = gpu["shared_h"]
    forced = mo.layer_forward(ld, xv, ids=gpu["ids"], h=gpu["h"], shared_h=shared_h)
    r, rms = rel_err(gpu["y"], forced["y"])
    assert rms > 0
    assert r <= tol, f"teacher-forced max|dy| = {r:.3e} x RMS(y) exceeds {tol}"
    # the expert outputs themselves, per routed pair and for the shared expert
    ro, _ = rel_err(gpu["expert_out"], forced["expert_out"])
    assert ro <= tol, f"teacher-forced expert_out max|do| = {ro:.3e} x RMS exceeds {tol}"
    if shared_h is not None and gpu.get("shared_out") is not None:
        rs, _ = rel_err(gpu["shared_out"], forced["shared_out"])
        assert rs <= tol, f"teacher-forced shared_out max|do| = {rs:.3e} x RMS exceeds {tol}"
    direct, _ = rel_err(gpu["y"], ref["y"])
    return r, direct, flips


def pairs_direct(ld, xv, gpu, tol=2e-3, bar=False):
    """The routed expert outputs (one row per pair, sorted order) and the shared
    expert's output against the oracle evaluated with the GPU's ids and its own
    rounding of h (no teacher forcing): max|do| / RMS(o) over all pairs.  With
    ``bar`` both must be within tol.  Returns (routed, shared) ratios."""
    ref = mo.layer_forward(ld, xv, ids=gpu["ids"])
    ro, _ = rel_err(gpu["expert_out"], ref["expert_out"])
    rs = 0.0
    if gpu.get("shared_out") is not None and ld.shared.n:
        rs, _ = rel_err(gpu["shared_out"], ref["shared_out"])
    if bar:
        assert ro <= tol, f"expert_out max|do| = {ro:.3e} x RMS exceeds {tol}"
        assert rs <= tol, f"shared_out max|do| = {rs:.3e} x RMS exceeds {tol}"
    return ro, rs
