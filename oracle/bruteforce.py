"""Scalar brute-force oracle of the routed MoE FFN layer -- TEST INFRASTRUCTURE ONLY.

Pure Python loops and the ``math``/``struct`` modules, no NumPy arithmetic.
It restates the same layer definition as ``oracle.moe_oracle`` element by
element, written independently, for tiny inputs, so that the two can pin each
other: a dropped term, a wrong sign, a transposed operand or a wrong packing
order in one of them shows up as a mismatch.

Sources of the definition are the same as in ``oracle.moe_oracle`` (page 2
"Layer 1: On-Demand MoE Expert Scheduling"; page 3 "How Strata Makes Your
Entire PC Work Together" and "The 'Doorbell' Mechanism"; page 5 "The model
is large on paper, sparse in practice"; page 1 "Quantization Configuration
Example").
"""
from __future__ import annotations

import math
import struct


def f16(bits: int) -> float:
    """IEEE half bits -> float (struct's 'e' codec)."""
    return struct.unpack("<e", struct.pack("<H", int(bits) & 0xFFFF))[0]


def to_f32(v: float) -> float:
    """Nearest float32 (the C double->float conversion struct uses rounds to nearest even)."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


def to_bf16(v: float) -> float:
    """bfloat16 via float32, nearest-even at both steps."""
    b = struct.unpack("<I", struct.pack("<f", v))[0]
    lsb = (b >> 16) & 1
    b = ((b + 0x7FFF + lsb) >> 16) << 16
    return struct.unpack("<f", struct.pack("<I", b & 0xFFFFFFFF))[0]


def round_act(v: float, act: str) -> float:
    return to_bf16(v) if act == "bf16" else to_f32(v)


def code3(codes_row, col: int) -> int:
    """3-bit code of column ``col``: group col // 32 is 12 bytes, 8 of two-bit
    fields (element 4j+i of the group at bits 2i, 2i+1 of byte j) then 4 of
    single bits (element i at bit i % 8 of byte 8 + i // 8)."""
    base = 12 * (col // 32)
    i = col % 32
    low = (int(codes_row[base + i // 4]) >> (2 * (i % 4))) & 3
    high = (int(codes_row[base + 8 + i // 8]) >> (i % 8)) & 1
    return low | (high << 2)


def weight(codes_row, scales_row, mins_row, qfmt: str, col: int) -> float:
    """Dequantised weight at column ``col`` of one packed row."""
    grp = col // 32
    s = f16(scales_row[grp])
    if qfmt == "q4_sym_g32":
        byte = int(codes_row[col // 2])
        u = (byte >> 4) if (col % 2) else (byte & 15)
        return s * (u - 8)
    if qfmt == "q3_sym_g32":
        return s * (code3(codes_row, col) - 4)
    byte = int(codes_row[col // 4])
    u = (byte >> (2 * (col % 4))) & 3
    return to_f32(s * u + f16(mins_row[grp]))


def row_weights(codes_row, scales_row, mins_row, qfmt: str, cols: int):
    """All dequantised weights of one packed row, group by group."""
    out = []
    for grp in range(cols // 32):
        s = f16(scales_row[grp])
        m = None if mins_row is None else f16(mins_row[grp])
        for col in range(32 * grp, 32 * grp + 32):
            if qfmt == "q4_sym_g32":
                byte = int(codes_row[col // 2])
                u = (byte >> 4) if (col % 2) else (byte & 15)
                out.append(s * (u - 8))
            elif qfmt == "q3_sym_g32":
                out.append(s * (code3(codes_row, col) - 4))
            else:
                byte = int(codes_row[col // 4])
                u = (byte >> (2 * (col % 4))) & 3
                out.append(to_f32(s * u + m))
    return out


def matvec(mat, j: int, qfmt: str, rows: int, cols: int, v):
    """sum_c W[j][r][c] v[c] for each r, with W the packed matrix of expert position j."""
    out = []
    for r in range(rows):
        wr = row_weights(mat.codes[j][r].tolist(), mat.scales[j][r].tolist(),
                         None if mat.mins is None else mat.mins[j][r].tolist(), qfmt, cols)
        acc = 0.0
        for c in range(cols):
            acc += wr[c] * v[c]
        out.append(acc)
    return out


def swiglu_expert(es, j: int, qfmt: str, act: str, hidden: int, inter: int, xv):
    g = matvec(es.gate, j, qfmt, inter, hidden, xv)
    u = matvec(es.up, j, qfmt, inter, hidden, xv)
    h = []
    for a, b in zip(g, u):
        sig = 1.0 / (1.0 + math.exp(-a)) if a > -700 else 0.0
        h.append(round_act(a * sig * b, act))
    return matvec(es.down, j, qfmt, hidden, inter, h)


def layer_forward(layer, x):
    """The layer on exact activations x (list of T lists of H floats).

    Returns dict(ids, w, offsets, sorted_pairs, pair_pos, y) as Python lists.
    """
    spec = layer.spec
    hdim, e_n, k, inter = spec.hidden, spec.n_experts, spec.top_k, spec.inter
    pos = {int(e): j for j, e in enumerate(layer.routed.index)} if len(layer.routed.index) else None
    t_n = len(x)
    rw = layer.router_w.tolist()
    rb = None if layer.router_b is None else layer.router_b.tolist()
    ids, ws, ys = [], [], []
    for t in range(t_n):
        logits = []
        for e in range(e_n):
            acc = 0.0
            for i in range(hdim):
                acc += rw[e][i] * x[t][i]
            if rb is not None:
                acc += rb[e]
            logits.append(acc)
        chosen = sorted(range(e_n), key=lambda e: (-logits[e], e))[:k]
        top = logits[chosen[0]]
        ex = [math.exp(logits[e] - top) for e in chosen]
        tot = sum(ex)
        wt = [v / tot for v in ex]
        ids.append(chosen)
        ws.append(wt)
        y = [0.0] * hdim
        for j in range(layer.shared.n):
            s = swiglu_expert(layer.shared, j, spec.qfmt, spec.act, hdim, inter, x[t])
            y = [a + b for a, b in zip(y, s)]
        for kk, e in enumerate(chosen):
            o = swiglu_expert(layer.routed, pos[e] if pos else e, spec.qfmt, spec.act, hdim, inter, x[t])
            y = [a + wt[kk] * b for a, b in zip(y, o)]
        ys.append(y)
    flat = [e for row in ids for e in row]
    counts = [0] * e_n
    for e in flat:
        counts[e] += 1
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    sorted_pairs = []
    for e in range(e_n):
        for p, pe in enumerate(flat):
            if pe == e:
                sorted_pairs.append(p)
    pair_pos = [0] * len(flat)
    for i, p in enumerate(sorted_pairs):
        pair_pos[p] = i
    return dict(ids=ids, w=ws, offsets=offsets, sorted_pairs=sorted_pairs, pair_pos=pair_pos, y=ys)
