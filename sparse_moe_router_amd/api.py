"""Python binding of libmoe.so -- argument marshalling only.

Each function has the name of the C entry point it calls and takes torch
tensors (device memory) instead of raw pointers.  Every step of the layer runs
in the HIP kernels behind the C ABI; nothing here computes.  If the library is
missing the binding raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")
# the same entry points with device range checks of caller-provided routing
# arrays (select it with use_debug_library)
DEBUG_LIB_PATH = os.path.join(_HERE, "libmoe_debug.so")

MOE_OK, MOE_E_ARG, MOE_E_UNSUPPORTED, MOE_E_WORKSPACE, MOE_E_DEVICE = range(5)
MOE_Q4_SYM_G32, MOE_Q2_ASYM_G32, MOE_Q3_SYM_G32 = 1, 2, 3
MOE_ACT_F32, MOE_ACT_BF16 = 0, 1
QFMT = {"q4_sym_g32": MOE_Q4_SYM_G32, "q2_asym_g32": MOE_Q2_ASYM_G32, "q3_sym_g32": MOE_Q3_SYM_G32}
CODE_BITS = {MOE_Q4_SYM_G32: 4, MOE_Q3_SYM_G32: 3, MOE_Q2_ASYM_G32: 2}
ACT = {"f32": MOE_ACT_F32, "bf16": MOE_ACT_BF16}

EXPORTS = ("moe_router_topk", "moe_permute", "moe_expert_ffn_q", "moe_expert_gate_up_q", "moe_expert_down_q",
           "moe_combine", "moe_layer_forward", "moe_layer_forward_noalloc",
           "moe_workspace_bytes", "moe_stack_forward", "moe_dequant", "moe_status_str", "moe_abi_version",
           "moe_range_checks")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {msg}")
        self.status = status


class c_qmat(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("mins", ctypes.c_void_p)]


class c_experts(ctypes.Structure):
    _fields_ = [("gate", c_qmat), ("up", c_qmat), ("down", c_qmat), ("n", ctypes.c_int32)]


class c_layer(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("qfmt", ctypes.c_int32), ("act", ctypes.c_int32),
                ("router_w", ctypes.c_void_p), ("router_b", ctypes.c_void_p),
                ("routed", c_experts), ("shared", c_experts), ("hot_experts", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m sparse_moe_router_amd.build` "
                               "(there is no non-HIP fallback)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        lp = ctypes.POINTER(c_layer)
        sigs = {
            "moe_router_topk": [lp, vp, i32, vp, vp, vp, vp, sz, vp],
            "moe_permute": [lp, vp, i32, vp, vp, vp, vp, sz, vp],
            "moe_expert_ffn_q": [lp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "moe_expert_gate_up_q": [lp, vp, i32, vp, vp, vp, vp, vp, vp],
            "moe_expert_down_q": [lp, vp, vp, i32, vp, vp, vp, vp, vp, vp],
            "moe_combine": [lp, vp, vp, vp, vp, i32, vp, vp, vp, vp],
            "moe_layer_forward": [lp, vp, i32, vp, vp, vp, vp, vp, sz, vp],
            "moe_layer_forward_noalloc": [lp, vp, i32, vp, vp, vp, vp, vp],
            "moe_stack_forward": [lp, i32, vp, i32, vp, vp, sz, vp],
            "moe_dequant": [ctypes.POINTER(c_qmat), i32, i32, i32, vp, vp],
        }
        for name, args in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.moe_workspace_bytes.argtypes = [lp, i32]
        L.moe_workspace_bytes.restype = sz
        L.moe_status_str.argtypes = [ctypes.c_int]
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_abi_version.argtypes = []
        L.moe_abi_version.restype = i32
        L.moe_range_checks.argtypes = []
        L.moe_range_checks.restype = i32
        _lib = L
    return _lib


def use_debug_library(debug: bool = True):
    """Route every later call to the debug library (or back to the release
    one).  Layer objects and workspaces stay valid across the switch."""
    global LIB_PATH, _lib
    path = DEBUG_LIB_PATH if debug else os.path.join(_HERE, "libmoe.so")
    if path != LIB_PATH:
        LIB_PATH, _lib = path, None


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoeError(fn, status, lib().moe_status_str(status).decode())


def _need(name: str, t: Optional[torch.Tensor], n: int, dtype=None):
    """Type, dtype and size of one argument: at least ``n`` elements.

    Checked for every buffer before anything is marshalled: the C ABI receives
    bare pointers, so a buffer that is too small would turn into a device
    access out of bounds."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.numel() < n:
        raise ValueError(f"{name}: {t.numel()} elements, at least {n} needed")


def _ptr(t: Optional[torch.Tensor], dtype=None, device=None) -> Optional[int]:
    """Device address of a contiguous tensor (on ``device`` when given)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"expected a torch.Tensor, got {type(t).__name__}")
    if not t.is_cuda:
        raise ValueError("tensor must live in device memory")
    if device is not None and t.device != device:
        raise ValueError(f"tensor on {t.device}, the layer's weights on {device}")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _act_dtype(act: int):
    return torch.bfloat16 if act == MOE_ACT_BF16 else torch.float32


class Layer:
    """A moe_layer descriptor over device tensors (kept alive by this object).

    routed / shared: dict(gate=(codes, scales, mins), up=(...), down=(...)) with
    codes uint8 [n][rows][...], scales and mins int16/uint16-bit fp16 planes
    [n][rows][cols/32] (mins None for the 4-bit format).
    """

    def __init__(self, *, hidden: int, inter: int, n_experts: int, top_k: int, qfmt, act,
                 router_w: torch.Tensor, router_b: Optional[torch.Tensor], routed: dict,
                 shared: Optional[dict] = None, hot_experts: int = 0):
        self.qfmt = QFMT.get(qfmt, qfmt)
        self.act = ACT.get(act, act)
        self.hidden, self.inter, self.n_experts, self.top_k = hidden, inter, n_experts, top_k
        self.act_dtype = _act_dtype(self.act)
        self.device = router_w.device
        self._keep = [router_w, router_b, routed, shared]
        if router_w.shape != (n_experts, hidden):
            raise ValueError("router_w must be [E][H]")
        if router_b is not None and router_b.shape != (n_experts,):
            raise ValueError("router_b must be [E]")
        if self.qfmt not in CODE_BITS:
            raise ValueError(f"unknown format {qfmt!r}")
        cb = CODE_BITS[self.qfmt]
        dev = self.device

        def qm(parts, n, rows, cols):
            codes, scales, mins = parts
            if codes.dtype != torch.uint8 or tuple(codes.shape) != (n, rows, cols * cb // 8):
                raise ValueError(f"codes must be uint8 [{n}][{rows}][{cols * cb // 8}], got {codes.dtype} {tuple(codes.shape)}")
            if scales.element_size() != 2 or tuple(scales.shape) != (n, rows, cols // 32):
                raise ValueError("scales must be 16-bit [n][rows][cols/32]")
            if (mins is None) != (self.qfmt != MOE_Q2_ASYM_G32):
                raise ValueError("mins are required for the 2-bit format only")
            if mins is not None and (mins.element_size() != 2 or tuple(mins.shape) != (n, rows, cols // 32)):
                raise ValueError("mins must be 16-bit [n][rows][cols/32]")
            return c_qmat(_ptr(codes, device=dev), _ptr(scales, device=dev), _ptr(mins, device=dev))

        def ex(d, n):
            if d is None:
                return c_experts(c_qmat(), c_qmat(), c_qmat(), 0)
            return c_experts(qm(d["gate"], n, inter, hidden), qm(d["up"], n, inter, hidden),
                             qm(d["down"], n, hidden, inter), n)

        self.c = c_layer(hidden, inter, n_experts, top_k, self.qfmt, self.act,
                         _ptr(router_w, torch.float32), _ptr(router_b, torch.float32, dev),
                         ex(routed, n_experts), ex(shared, 1), int(hot_experts))

    @property
    def ref(self):
        return ctypes.byref(self.c)


def moe_workspace_bytes(layer: Layer, T_max: int) -> int:
    return int(lib().moe_workspace_bytes(layer.ref, int(T_max)))


def workspace(layer: Layer, T_max: int, device=None) -> torch.Tensor:
    """A device workspace tensor of moe_workspace_bytes(layer, T_max) bytes."""
    n = moe_workspace_bytes(layer, T_max)
    if n == 0:
        raise MoeError("moe_workspace_bytes", MOE_E_ARG, "invalid layer descriptor or T")
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def _ws(layer: Layer, ws):
    return (None, 0) if ws is None else (_ptr(ws, torch.uint8, layer.device), ws.numel())


def _x(layer: Layer, x: torch.Tensor, T: int):
    if not isinstance(x, torch.Tensor) or x.dtype != layer.act_dtype or x.dim() != 2 or \
            x.shape[1] != layer.hidden or x.shape[0] < T:
        raise ValueError(f"x must be {layer.act_dtype} [>=T][{layer.hidden}]")
    return _ptr(x, device=layer.device)


def _p(layer: Layer, t, dtype=None):
    return _ptr(t, dtype, layer.device)


def moe_router_topk(layer: Layer, x, T, topk_ids, topk_w, logits=None, ws=None, stream=None):
    K, E = layer.top_k, layer.n_experts
    _need("topk_ids", topk_ids, T * K, torch.int32)
    _need("topk_w", topk_w, T * K, torch.float32)
    _need("logits", logits, T * E, torch.float32)
    w, wn = _ws(layer, ws)
    _check("moe_router_topk", lib().moe_router_topk(layer.ref, _x(layer, x, T), int(T), _p(layer, topk_ids),
                                                    _p(layer, topk_w), _p(layer, logits), w, wn, _stream(stream)))


def moe_permute(layer: Layer, topk_ids, T, expert_offsets, sorted_pairs, pair_pos, ws, stream=None):
    K, E = layer.top_k, layer.n_experts
    _need("topk_ids", topk_ids, T * K, torch.int32)
    _need("expert_offsets", expert_offsets, E + 1, torch.int32)
    _need("sorted_pairs", sorted_pairs, T * K, torch.int32)
    _need("pair_pos", pair_pos, T * K, torch.int32)
    w, wn = _ws(layer, ws)
    _check("moe_permute", lib().moe_permute(layer.ref, _p(layer, topk_ids), int(T), _p(layer, expert_offsets),
                                            _p(layer, sorted_pairs), _p(layer, pair_pos), w, wn, _stream(stream)))


def _routing_inputs(layer: Layer, T, topk_ids, expert_offsets, sorted_pairs):
    K, E = layer.top_k, layer.n_experts
    _need("topk_ids", topk_ids, T * K, torch.int32)
    _need("expert_offsets", expert_offsets, E + 1, torch.int32)
    _need("sorted_pairs", sorted_pairs, T * K, torch.int32)


def moe_expert_ffn_q(layer: Layer, x, T, topk_ids, expert_offsets, sorted_pairs, expert_out, shared_out=None,
                     h=None, shared_h=None, ws=None, stream=None):
    K, H, I = layer.top_k, layer.hidden, layer.inter
    _routing_inputs(layer, T, topk_ids, expert_offsets, sorted_pairs)
    _need("expert_out", expert_out, T * K * H, torch.float32)
    _need("shared_out", shared_out, T * H, torch.float32)
    _need("h", h, T * K * I, layer.act_dtype)
    _need("shared_h", shared_h, T * I, layer.act_dtype)
    w, wn = _ws(layer, ws)
    _check("moe_expert_ffn_q", lib().moe_expert_ffn_q(layer.ref, _x(layer, x, T), int(T), _p(layer, topk_ids),
                                                      _p(layer, expert_offsets), _p(layer, sorted_pairs),
                                                      _p(layer, expert_out), _p(layer, shared_out), _p(layer, h),
                                                      _p(layer, shared_h), w, wn, _stream(stream)))


def _gate_up_args(layer, x, T, topk_ids, expert_offsets, sorted_pairs, h, shared_h, stream):
    K, I = layer.top_k, layer.inter
    _routing_inputs(layer, T, topk_ids, expert_offsets, sorted_pairs)
    _need("h", h, T * K * I, layer.act_dtype)
    _need("shared_h", shared_h, T * I, layer.act_dtype)
    return (layer.ref, _x(layer, x, T), int(T), _p(layer, topk_ids), _p(layer, expert_offsets),
            _p(layer, sorted_pairs), _p(layer, h), _p(layer, shared_h), _stream(stream))


def moe_expert_gate_up_q(layer: Layer, x, T, topk_ids, expert_offsets, sorted_pairs, h, shared_h=None,
                         stream=None):
    _check("moe_expert_gate_up_q", lib().moe_expert_gate_up_q(
        *_gate_up_args(layer, x, T, topk_ids, expert_offsets, sorted_pairs, h, shared_h, stream)))


def moe_expert_down_q(layer: Layer, h, shared_h, T, topk_ids, expert_offsets, sorted_pairs, expert_out,
                      shared_out=None, stream=None):
    K, H, I = layer.top_k, layer.hidden, layer.inter
    _routing_inputs(layer, T, topk_ids, expert_offsets, sorted_pairs)
    _need("h", h, T * K * I, layer.act_dtype)
    _need("shared_h", shared_h, T * I, layer.act_dtype)
    _need("expert_out", expert_out, T * K * H, torch.float32)
    _need("shared_out", shared_out, T * H, torch.float32)
    _check("moe_expert_down_q", lib().moe_expert_down_q(layer.ref, _p(layer, h), _p(layer, shared_h), int(T),
                                                        _p(layer, topk_ids), _p(layer, expert_offsets),
                                                        _p(layer, sorted_pairs), _p(layer, expert_out),
                                                        _p(layer, shared_out), _stream(stream)))


def moe_combine(layer: Layer, expert_out, shared_out, pair_pos, topk_w, T, y, x_resid=None, x_next=None,
                stream=None):
    K, H = layer.top_k, layer.hidden
    _need("expert_out", expert_out, T * K * H, torch.float32)
    _need("shared_out", shared_out, T * H, torch.float32)
    _need("pair_pos", pair_pos, T * K, torch.int32)
    _need("topk_w", topk_w, T * K, torch.float32)
    _need("y", y, T * H, torch.float32)
    _need("x_resid", x_resid, T * H, layer.act_dtype)
    _need("x_next", x_next, T * H, layer.act_dtype)
    _check("moe_combine", lib().moe_combine(layer.ref, _p(layer, expert_out), _p(layer, shared_out),
                                            _p(layer, pair_pos), _p(layer, topk_w), int(T), _p(layer, y),
                                            _p(layer, x_resid), _p(layer, x_next), _stream(stream)))


def _layer_forward_args(layer, x, T, y, x_next, topk_ids, topk_w, ws, stream):
    K, H = layer.top_k, layer.hidden
    _need("y", y, T * H, torch.float32)
    _need("x_next", x_next, T * H, layer.act_dtype)
    _need("topk_ids", topk_ids, T * K, torch.int32)
    _need("topk_w", topk_w, T * K, torch.float32)
    w, wn = _ws(layer, ws)
    return (layer.ref, _x(layer, x, T), int(T), _p(layer, y), _p(layer, x_next), _p(layer, topk_ids),
            _p(layer, topk_w), w, wn, _stream(stream))


def moe_layer_forward(layer: Layer, x, T, y, x_next=None, topk_ids=None, topk_w=None, ws=None, stream=None):
    _check("moe_layer_forward", lib().moe_layer_forward(
        *_layer_forward_args(layer, x, T, y, x_next, topk_ids, topk_w, ws, stream)))


NOALLOC_SCRATCH_BYTES = 16 << 20  # MOE_NOALLOC_SCRATCH_BYTES


def moe_layer_forward_noalloc(layer: Layer, x, T, y, x_next=None, topk_ids=None, topk_w=None, stream=None):
    """moe_layer_forward with the library's own device array in place of a workspace."""
    K, H = layer.top_k, layer.hidden
    _need("y", y, T * H, torch.float32)
    _need("x_next", x_next, T * H, layer.act_dtype)
    _need("topk_ids", topk_ids, T * K, torch.int32)
    _need("topk_w", topk_w, T * K, torch.float32)
    _check("moe_layer_forward_noalloc", lib().moe_layer_forward_noalloc(
        layer.ref, _x(layer, x, T), int(T), _p(layer, y), _p(layer, x_next), _p(layer, topk_ids),
        _p(layer, topk_w), _stream(stream)))


class Bound:
    """One entry point with its arguments checked and marshalled once.

    Calling it enqueues the same call again (same buffers, same stream) through
    the C ABI with no per-call Python checks, for loops where the host would
    otherwise take as long as the kernels.  It keeps the tensors it was given
    alive.  A non-OK status still raises MoeError."""

    def __init__(self, name: str, args: tuple, keep: tuple):
        self.name, self.args, self._keep = name, args, keep
        self.fn = getattr(lib(), name)

    def __call__(self):
        st = self.fn(*self.args)
        if st != MOE_OK:
            _check(self.name, st)


def bind_layer_forward(layer: Layer, x, T, y, x_next=None, topk_ids=None, topk_w=None, ws=None,
                       stream=None) -> Bound:
    """moe_layer_forward(...) as a Bound call."""
    return Bound("moe_layer_forward", _layer_forward_args(layer, x, T, y, x_next, topk_ids, topk_w, ws, stream),
                 (layer, x, y, x_next, topk_ids, topk_w, ws, stream))


def bind_expert_gate_up_q(layer: Layer, x, T, topk_ids, expert_offsets, sorted_pairs, h, shared_h=None,
                          stream=None) -> Bound:
    """moe_expert_gate_up_q(...) as a Bound call."""
    return Bound("moe_expert_gate_up_q",
                 _gate_up_args(layer, x, T, topk_ids, expert_offsets, sorted_pairs, h, shared_h, stream),
                 (layer, x, topk_ids, expert_offsets, sorted_pairs, h, shared_h, stream))


def moe_stack_forward(layers, x_inout, T, y_last=None, ws=None, stream=None):
    arr = (c_layer * len(layers))(*[l.c for l in layers])
    if not layers:
        _check("moe_stack_forward", lib().moe_stack_forward(arr, 0, None, int(T), None, None, 0, _stream(stream)))
        return
    L0 = layers[0]
    if any(l.device != L0.device for l in layers):
        raise ValueError("every layer of a stack must live on one device")
    _need("y_last", y_last, T * L0.hidden, torch.float32)
    w, wn = _ws(L0, ws)
    _check("moe_stack_forward", lib().moe_stack_forward(arr, len(layers), _x(L0, x_inout, T), int(T),
                                                        _p(L0, y_last), w, wn, _stream(stream)))


def moe_dequant(codes, scales, mins, qfmt, rows, cols, out, stream=None):
    q = QFMT.get(qfmt, qfmt)
    if q not in CODE_BITS:
        raise ValueError(f"unknown format {qfmt!r}")
    _need("codes", codes, rows * cols * CODE_BITS[q] // 8, torch.uint8)
    _need("scales", scales, rows * (cols // 32))
    _need("mins", mins, rows * (cols // 32))
    _need("out", out, rows * cols, torch.float32)
    dev = out.device
    m = c_qmat(_ptr(codes, device=dev), _ptr(scales, device=dev), _ptr(mins, device=dev))
    _check("moe_dequant", lib().moe_dequant(ctypes.byref(m), q, int(rows), int(cols), _ptr(out, torch.float32),
                                            _stream(stream)))


def moe_abi_version() -> int:
    return int(lib().moe_abi_version())


def moe_range_checks() -> int:
    return int(lib().moe_range_checks())
