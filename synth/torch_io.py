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
