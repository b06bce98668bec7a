"""Seeded synthetic inputs for the routed MoE FFN layer.

This module only *makes inputs*: activations, router weights and biases, and
expert weights in the packed group-32 formats.  It holds none of the layer's
arithmetic (no router products, no top-k, no dequantisation, no expert FFN, no
combine).  Both the CPU oracle (``oracle/``) and the HIP path (through the
tests and ``bench.py``) take their inputs from here and from nowhere else.

Shapes and value distributions follow the workloads the pages describe for
Qwen3.8-Flash-Next (512 experts per layer, 10 routed + 1 shared expert per
token, 24,576 experts in total, hence 48 MoE layers: page 3 "How Strata Makes
Your Entire PC Work Together", page 5 "The model is large on paper, sparse in
practice"), with hidden 2048 and intermediate 768, 4-bit and 2-bit weights
("4-bit or even 2-bit precision": page 1 "How Strata Makes the Impossible
Possible"; page 3 "A Few Things to Keep in Perspective").

Random streams: ``numpy.random.Generator(PCG64(SeedSequence(key)))`` with
``key = [seed, family, layer, tensor_id, index]``.  Expert weights are drawn
per expert, so any subset of experts can be regenerated without the rest.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import numpy as np

Q4 = "q4_sym_g32"
Q2 = "q2_asym_g32"
Q3 = "q3_sym_g32"
ACT_F32 = "f32"
ACT_BF16 = "bf16"
GROUP = 32

# tensor ids inside a seed key
_T_X, _T_ROUTER_W, _T_ROUTER_RANK, _T_GATE, _T_UP, _T_DOWN = range(6)


@dataclass(frozen=True)
class LayerSpec:
    """One workload: the shape of a routed MoE FFN layer and its inputs."""

    name: str
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    tokens: int
    qfmt: str
    act: str
    router_std: float
    zipf_s: Optional[float]       # None: no router bias
    family: int                   # seed family of the weights (same shape + format share it)
    n_shared: int = 1
    n_layers: int = 1
    weight_std: float = 0.02
    ordered: bool = False         # experts numbered by decreasing popularity (Zipf rank e + 1)

    def with_tokens(self, t: int) -> "LayerSpec":
        return replace(self, tokens=t)


def _spec_table() -> dict:
    h, e, k, i = 2048, 512, 10, 768
    rstd = math.sqrt(1.0 / h)
    return {
        "tiny": LayerSpec("tiny", 64, 8, 2, 128, 4, Q4, ACT_F32, 0.02, None, family=0),
        "decode": LayerSpec("decode", h, e, k, i, 1, Q4, ACT_BF16, rstd, 1.1, family=1),
        "verify": LayerSpec("verify", h, e, k, i, 5, Q2, ACT_BF16, rstd, 1.1, family=2),
        "decode_q3": LayerSpec("decode_q3", h, e, k, i, 1, Q3, ACT_BF16, rstd, 1.1, family=5),
        "prefill": LayerSpec("prefill", h, e, k, i, 4096, Q4, ACT_BF16, rstd, 1.1, family=1),
        "stack_t1": LayerSpec("stack_t1", h, e, k, i, 1, Q2, ACT_BF16, rstd, 1.1, family=4, n_layers=48),
        "stack_t8": LayerSpec("stack_t8", h, e, k, i, 8, Q2, ACT_BF16, rstd, 1.1, family=4, n_layers=48),
    }


SPECS = _spec_table()


def rng(seed: int, family: int, layer: int, tensor: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, family, layer, tensor, index])))


# ----------------------------------------------------------------------------
# storage-type helpers (input encoding only)

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the bit patterns."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f64_to_f16_bits(a: np.ndarray) -> np.ndarray:
    """Round float64 values to IEEE half (numpy rounds to nearest even); return bits."""
    return np.asarray(a, dtype=np.float64).astype(np.float16).view(np.uint16)


# ----------------------------------------------------------------------------
# packed formats (the byte layout both sides must read)
#
# Groups of 32 consecutive elements run along each matrix's last (reduction)
# dimension.  Q4: byte j of a row holds element 2j in its low nibble and 2j+1
# in its high nibble, stored as u = q + 8.  Q2: byte j holds elements
# 4j..4j+3 in bits [1:0], [3:2], [5:4], [7:6].  Q3: 12 bytes per group, the
# low two bits of the codes in the Q2 layout (8 bytes), then the third bit of
# element i at bit i % 8 of byte 8 + i // 8, stored as u = q + 4.  Scales and
# minima are fp16 planes [rows][cols/32].

def pack_q4(u: np.ndarray) -> np.ndarray:
    u = np.asarray(u, dtype=np.uint8)
    return (u[..., 0::2] & 0xF) | ((u[..., 1::2] & 0xF) << 4)


def pack_q2(u: np.ndarray) -> np.ndarray:
    u = np.asarray(u, dtype=np.uint8)
    return ((u[..., 0::4] & 3) | ((u[..., 1::4] & 3) << 2)
            | ((u[..., 2::4] & 3) << 4) | ((u[..., 3::4] & 3) << 6)).astype(np.uint8)


def pack_q3(u: np.ndarray) -> np.ndarray:
    """Codes u in 0..7 [..., C] -> [..., 3C/8]: per 32-element group 12 bytes, the
    low two bits in the 2-bit layout (bytes 0..7), then the third bit of
    element i at bit i % 8 of byte 8 + i // 8."""
    u = np.asarray(u, dtype=np.uint8)
    g = u.reshape(*u.shape[:-1], u.shape[-1] // GROUP, GROUP)
    low = pack_q2(g & 3)                                       # [..., G, 8]
    hb = (g >> 2) & 1
    high = np.zeros(g.shape[:-1] + (4,), np.uint8)
    for i in range(GROUP):
        high[..., i // 8] |= (hb[..., i] << (i % 8)).astype(np.uint8)
    return np.concatenate([low, high], axis=-1).reshape(*u.shape[:-1], u.shape[-1] * 3 // 8)


def quantize_q4(w: np.ndarray):
    """Symmetric round-to-nearest 4-bit, group 32: s = fp16(amax/7), q = clamp(rint(w/s), -8, 7).

    Returns (codes uint8 [..., cols/2], scales fp16 bits [..., cols/32]).
    """
    w = np.asarray(w, dtype=np.float32)
    g = w.reshape(*w.shape[:-1], w.shape[-1] // GROUP, GROUP).astype(np.float64)
    amax = np.abs(g).max(axis=-1)
    s16 = (amax / 7.0).astype(np.float16)
    s = s16.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint(g / np.where(s > 0, s, 1.0)), 0.0)
    q = np.clip(q, -8, 7).astype(np.int16)
    u = (q + 8).astype(np.uint8).reshape(w.shape)
    return pack_q4(u), s16.view(np.uint16)


def quantize_q3(w: np.ndarray):
    """Symmetric round-to-nearest 3-bit, group 32: s = fp16(amax/3), q = clamp(rint(w/s), -4, 3).

    Returns (codes uint8 [..., 3 cols/8], scales fp16 bits [..., cols/32]).
    """
    w = np.asarray(w, dtype=np.float32)
    g = w.reshape(*w.shape[:-1], w.shape[-1] // GROUP, GROUP).astype(np.float64)
    amax = np.abs(g).max(axis=-1)
    s16 = (amax / 3.0).astype(np.float16)
    s = s16.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint(g / np.where(s > 0, s, 1.0)), 0.0)
    q = np.clip(q, -4, 3).astype(np.int16)
    u = (q + 4).astype(np.uint8).reshape(w.shape)
    return pack_q3(u), s16.view(np.uint16)


def quantize_q2(w: np.ndarray):
    """Asymmetric round-to-nearest 2-bit, group 32: m = fp16(min), s = fp16((max-min)/3),
    u = clamp(rint((w-m)/s), 0, 3).

    Returns (codes uint8 [..., cols/4], scales fp16 bits, mins fp16 bits).
    """
    w = np.asarray(w, dtype=np.float32)
    g = w.reshape(*w.shape[:-1], w.shape[-1] // GROUP, GROUP).astype(np.float64)
    mn = g.min(axis=-1)
    mx = g.max(axis=-1)
    m16 = mn.astype(np.float16)
    s16 = ((mx - mn) / 3.0).astype(np.float16)
    s = s16.astype(np.float64)[..., None]
    m = m16.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.where(s > 0, np.rint((g - m) / np.where(s > 0, s, 1.0)), 0.0)
    u = np.clip(u, 0, 3).astype(np.uint8).reshape(w.shape)
    return pack_q2(u), s16.view(np.uint16), m16.view(np.uint16)


def requantize_codes_q4(w: np.ndarray, scales_bits: np.ndarray) -> np.ndarray:
    """Codes u in [0,15] that the quantizer picks for weights w under given fp16 scales."""
    g = np.asarray(w, dtype=np.float64).reshape(*w.shape[:-1], w.shape[-1] // GROUP, GROUP)
    s = np.asarray(scales_bits, dtype=np.uint16).view(np.float16).astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s != 0, np.rint(g / np.where(s != 0, s, 1.0)), 0.0)
    return (np.clip(q, -8, 7) + 8).astype(np.uint8).reshape(w.shape)


def requantize_codes_q3(w: np.ndarray, scales_bits: np.ndarray) -> np.ndarray:
    """Codes u in [0,7] that the quantizer picks for weights w under given fp16 scales."""
    g = np.asarray(w, dtype=np.float64).reshape(*w.shape[:-1], w.shape[-1] // GROUP, GROUP)
    s = np.asarray(scales_bits, dtype=np.uint16).view(np.float16).astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s != 0, np.rint(g / np.where(s != 0, s, 1.0)), 0.0)
    return (np.clip(q, -4, 3) + 4).astype(np.uint8).reshape(w.shape)


def requantize_codes_q2(w: np.ndarray, scales_bits: np.ndarray, mins_bits: np.ndarray) -> np.ndarray:
    g = np.asarray(w, dtype=np.float64).reshape(*w.shape[:-1], w.shape[-1] // GROUP, GROUP)
    s = np.asarray(scales_bits, dtype=np.uint16).view(np.float16).astype(np.float64)[..., None]
    m = np.asarray(mins_bits, dtype=np.uint16).view(np.float16).astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.where(s != 0, np.rint((g - m) / np.where(s != 0, s, 1.0)), 0.0)
    return np.clip(u, 0, 3).astype(np.uint8).reshape(w.shape)


# ----------------------------------------------------------------------------
# containers

@dataclass
class PackedMat:
    """[n][rows][...] planes of one matrix kind (gate, up or down) for n experts."""

    codes: np.ndarray
    scales: np.ndarray
    mins: Optional[np.ndarray] = None


@dataclass
class ExpertSet:
    gate: PackedMat
    up: PackedMat
    down: PackedMat
    index: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))  # expert ids held

    @property
    def n(self) -> int:
        return int(self.gate.codes.shape[0])


@dataclass
class LayerData:
    spec: LayerSpec
    layer: int
    router_w: np.ndarray              # [E][H] float32
    router_b: Optional[np.ndarray]    # [E] float32 or None
    routed: ExpertSet                 # all E experts, or the subset in routed.index
    shared: ExpertSet                 # n_shared experts


@dataclass
class Activations:
    values: np.ndarray    # [T][H] float32 (exact values of the stored activations)
    storage: np.ndarray   # float32 [T][H] (act f32) or uint16 bf16 bits [T][H]


# ----------------------------------------------------------------------------
# generators

def gen_x(spec: LayerSpec, seed: int = 0, layer: int = 0, tokens: Optional[int] = None) -> Activations:
    t = spec.tokens if tokens is None else tokens
    v = rng(seed, spec.family, layer, _T_X, t).standard_normal((t, spec.hidden), dtype=np.float32)
    if spec.act == ACT_BF16:
        bits = f32_to_bf16_bits(v)
        return Activations(bf16_bits_to_f32(bits), bits)
    return Activations(v.copy(), v)


def gen_router(spec: LayerSpec, seed: int = 0, layer: int = 0):
    w = rng(seed, spec.family, layer, _T_ROUTER_W).standard_normal(
        (spec.n_experts, spec.hidden), dtype=np.float32) * np.float32(spec.router_std)
    w = w.astype(np.float32)
    if spec.zipf_s is None:
        return w, None
    # Zipf(s) prior over a random ranking of the experts, as a logit offset:
    # b_e = -s * ln(rank_e) with ranks 1..E (the normaliser cancels in top-k and softmax);
    # with spec.ordered the experts are numbered by popularity (rank_e = e + 1)
    if spec.ordered:
        ranks = 1 + np.arange(spec.n_experts)
    else:
        ranks = 1 + rng(seed, spec.family, layer, _T_ROUTER_RANK).permutation(spec.n_experts)
    b = (-spec.zipf_s * np.log(ranks.astype(np.float64))).astype(np.float32)
    return w, b


def _quantize(spec: LayerSpec, w: np.ndarray):
    if spec.qfmt == Q4:
        c, s = quantize_q4(w)
        return c, s, None
    if spec.qfmt == Q2:
        return quantize_q2(w)
    if spec.qfmt == Q3:
        c, s = quantize_q3(w)
        return c, s, None
    raise ValueError(spec.qfmt)


def gen_expert_dense(spec: LayerSpec, seed: int, layer: int, e: int):
    """Unquantized float32 weights of expert e (e == n_experts: the shared expert)."""
    sd = np.float32(spec.weight_std)
    g = rng(seed, spec.family, layer, _T_GATE, e).standard_normal((spec.inter, spec.hidden), dtype=np.float32) * sd
    u = rng(seed, spec.family, layer, _T_UP, e).standard_normal((spec.inter, spec.hidden), dtype=np.float32) * sd
    d = rng(seed, spec.family, layer, _T_DOWN, e).standard_normal((spec.hidden, spec.inter), dtype=np.float32) * sd
    return g, u, d


def _gen_one(spec: LayerSpec, seed: int, layer: int, e: int):
    return tuple(_quantize(spec, m) for m in gen_expert_dense(spec, seed, layer, e))


def code_bytes_per_row(qfmt: str, cols: int) -> int:
    return {Q4: cols // 2, Q3: cols * 3 // 8, Q2: cols // 4}[qfmt]


def _alloc_set(spec: LayerSpec, n: int) -> ExpertSet:
    def mat(rows, cols):
        return PackedMat(np.empty((n, rows, code_bytes_per_row(spec.qfmt, cols)), np.uint8),
                         np.empty((n, rows, cols // GROUP), np.uint16),
                         np.empty((n, rows, cols // GROUP), np.uint16) if spec.qfmt == Q2 else None)
    return ExpertSet(mat(spec.inter, spec.hidden), mat(spec.inter, spec.hidden), mat(spec.hidden, spec.inter))


def gen_experts(spec: LayerSpec, ids: Sequence[int], seed: int = 0, layer: int = 0,
                threads: Optional[int] = None) -> ExpertSet:
    """Packed weights of the listed experts (id n_experts is the shared expert), in list order."""
    ids = [int(i) for i in ids]
    out = _alloc_set(spec, len(ids))
    out.index = np.asarray(ids, dtype=np.int64)

    def work(j):
        parts = _gen_one(spec, seed, layer, ids[j])
        for mat, (c, s, m) in zip((out.gate, out.up, out.down), parts):
            mat.codes[j] = c
            mat.scales[j] = s
            if m is not None:
                mat.mins[j] = m

    nthreads = threads or min(16, os.cpu_count() or 1)
    if len(ids) <= 2 or nthreads <= 1:
        for j in range(len(ids)):
            work(j)
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(work, range(len(ids))))
    return out


def gen_layer(spec: LayerSpec, seed: int = 0, layer: int = 0, routed_ids: Optional[Sequence[int]] = None,
              threads: Optional[int] = None) -> LayerData:
    """One layer's router and packed experts.  ``routed_ids`` limits the routed experts generated."""
    w, b = gen_router(spec, seed, layer)
    ids = range(spec.n_experts) if routed_ids is None else routed_ids
    routed = gen_experts(spec, ids, seed, layer, threads)
    shared = gen_experts(spec, [spec.n_experts + j for j in range(spec.n_shared)], seed, layer, threads)
    return LayerData(spec, layer, w, b, routed, shared)


def subset(es: ExpertSet, rows: Sequence[int]) -> ExpertSet:
    """The experts at positions ``rows`` of a set (positions, not expert ids)."""
    rows = np.asarray(rows, dtype=np.int64)

    def m(p: PackedMat) -> PackedMat:
        return PackedMat(p.codes[rows], p.scales[rows], None if p.mins is None else p.mins[rows])

    return ExpertSet(m(es.gate), m(es.up), m(es.down), es.index[rows] if len(es.index) else rows)
