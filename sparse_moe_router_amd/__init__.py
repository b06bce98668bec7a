"""Routed Mixture-of-Experts FFN layer for MI355X (gfx950).

The compute lives in ``libmoe.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/moe.h``); ``sparse_moe_router_amd.api`` is its Python
binding.  PyTorch provides device memory and streams only.
"""
from . import workload  # noqa: F401  (pure-Python byte/flop accounting)

__all__ = ["api", "workload"]
