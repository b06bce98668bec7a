"""Move generated inputs into torch tensors (device memory); no arithmetic."""
from __future__ import annotations

import numpy as np
import torch

from . import ACT_BF16, LayerData, PackedMat


def _t(a, device):
    if a is None:
        return None
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def _mat(p: PackedMat, device):
    return (_t(p.codes, device), _t(p.scales, device), _t(p.mins, device))


def experts_to(es, device):
    return dict(gate=_mat(es.gate, device), up=_mat(es.up, device), down=_mat(es.down, device))


def layer_kwargs(layer: LayerData, device) -> dict:
    """Keyword arguments describing one layer with device tensors (router, routed, shared)."""
    s = layer.spec
    return dict(hidden=s.hidden, inter=s.inter, n_experts=s.n_experts, top_k=s.top_k, qfmt=s.qfmt, act=s.act,
                router_w=_t(layer.router_w, device), router_b=_t(layer.router_b, device),
                routed=experts_to(layer.routed, device),
                shared=experts_to(layer.shared, device) if layer.shared.n else None)


def x_tensor(storage: np.ndarray, act: str, device) -> torch.Tensor:
    """Activations in their storage type: bf16 from bit patterns, or fp32."""
    if act == ACT_BF16:
        return torch.from_numpy(np.ascontiguousarray(storage).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(storage, dtype=np.float32)).to(device)


def device_filled_kwargs(spec, layer: int, device, seed: int = 0) -> dict:
    """Keyword arguments of one layer whose expert planes are filled on the
    device, for runs over many layers (the 48-layer stack): uniform random
    codes, fp16 scales s = 0.0096 U(0.85, 1.15) and, for the 2-bit format,
    minima m = -1.5 s; the router and its bias come from gen_router as for
    every other layer.  The scale is 0.35 x the 0.0274 that the 2-bit
    quantiser gives N(0, 0.02^2) weights: a SwiGLU layer's output grows with
    the square of its input, and with that larger scale (y about 1.1 x RMS of
    x at RMS 1) the residual stream of 48 layers without a norm overflows
    after about ten layers, leaving NaN logits and a degenerate routing; at
    0.35 x, y is about 4 % of x and the stream stays finite over 48 layers.
    The bytes per layer do not depend on the values."""
    from . import Q2, Q3, gen_router
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + spec.family * 10_007 + layer) & 0x7FFFFFFF)
    bits = {Q2: 2, Q3: 3}.get(spec.qfmt, 4)

    def mat(n, rows, cols):
        codes = torch.randint(0, 256, (n, rows, cols * bits // 8), dtype=torch.uint8, device=device, generator=g)
        s = (0.0096 * (0.85 + 0.3 * torch.rand((n, rows, cols // 32), device=device, generator=g))).half()
        mins = (-1.5 * s.float()).half().view(torch.int16) if bits == 2 else None
        return codes, s.view(torch.int16), mins

    def experts(n):
        return dict(gate=mat(n, spec.inter, spec.hidden), up=mat(n, spec.inter, spec.hidden),
                    down=mat(n, spec.hidden, spec.inter))

    w, b = gen_router(spec, seed=seed, layer=layer)
    return dict(hidden=spec.hidden, inter=spec.inter, n_experts=spec.n_experts, top_k=spec.top_k, qfmt=spec.qfmt,
                act=spec.act, router_w=_t(w, device), router_b=_t(b, device), routed=experts(spec.n_experts),
                shared=experts(1) if spec.n_shared else None)
