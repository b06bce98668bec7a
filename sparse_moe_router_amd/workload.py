"""Algorithmic byte and flop counts of the routed MoE FFN layer.

These are the quantities the roofline figures divide by: what the method must
move (the packed weights of the experts actually selected, the router, the
activations in and the output out) and the multiply-adds it must do.  They
never count the dense work over all experts.
"""
from __future__ import annotations

GROUP = 32


def code_bits(qfmt: str) -> int:
    return {"q4_sym_g32": 4, "q3_sym_g32": 3, "q2_asym_g32": 2}[qfmt]


def matrix_bytes(qfmt: str, rows: int, cols: int) -> int:
    """Packed codes + fp16 scales (+ fp16 minima for the 2-bit format) of one matrix."""
    groups = rows * (cols // GROUP)
    planes = 2 if qfmt == "q2_asym_g32" else 1
    return rows * cols * code_bits(qfmt) // 8 + planes * 2 * groups


def expert_bytes(qfmt: str, hidden: int, inter: int) -> int:
    """gate [I][H] + up [I][H] + down [H][I]."""
    return 2 * matrix_bytes(qfmt, inter, hidden) + matrix_bytes(qfmt, hidden, inter)


def act_bytes(act: str) -> int:
    return 2 if act == "bf16" else 4


def router_bytes(hidden: int, n_experts: int, bias: bool = True) -> int:
    return 4 * n_experts * hidden + (4 * n_experts if bias else 0)


def layer_bytes(qfmt: str, act: str, hidden: int, inter: int, n_experts: int, tokens: int,
                distinct_experts: int, n_shared: int = 1, bias: bool = True) -> int:
    """Router + (U + shared) experts + x in + y (fp32) out."""
    return (router_bytes(hidden, n_experts, bias)
            + (distinct_experts + n_shared) * expert_bytes(qfmt, hidden, inter)
            + tokens * hidden * act_bytes(act) + tokens * hidden * 4)


def expert_weight_bytes(qfmt: str, hidden: int, inter: int, distinct_experts: int, n_shared: int = 1) -> int:
    return (distinct_experts + n_shared) * expert_bytes(qfmt, hidden, inter)


def layer_flops(hidden: int, inter: int, n_experts: int, top_k: int, tokens: int, n_shared: int = 1) -> int:
    """2 T E H (router) + 2 T (K + shared) 3 H I (expert SwiGLU)."""
    return 2 * tokens * n_experts * hidden + 2 * tokens * (top_k + n_shared) * 3 * hidden * inter


def spec_layer_bytes(spec, distinct_experts: int, tokens: int = None) -> int:
    t = spec.tokens if tokens is None else tokens
    return layer_bytes(spec.qfmt, spec.act, spec.hidden, spec.inter, spec.n_experts, t,
                       distinct_experts, spec.n_shared, spec.zipf_s is not None)
