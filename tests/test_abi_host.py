"""The C ABI library loads, exports every declared symbol, and validates
arguments on the host before touching the device (CPU only: every call here
returns before any kernel launch)."""
import ctypes
import os
import re

import pytest

from sparse_moe_router_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(api.LIB_PATH), reason="libmoe.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("moe_router_topk", "moe_permute", "moe_expert_ffn_q", "moe_combine", "moe_layer_forward"):
        assert n in names
    assert set(names) == set(api.EXPORTS)


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(api.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_debug_library_exports_the_same_entry_points_with_range_checks():
    """libmoe_debug.so: the same symbols; moe_range_checks() tells the two apart."""
    assert os.path.exists(api.DEBUG_LIB_PATH), "libmoe_debug.so not built"
    dbg, rel = ctypes.CDLL(api.DEBUG_LIB_PATH), ctypes.CDLL(api.LIB_PATH)
    for n in declared_functions():
        assert hasattr(dbg, n), n
    dbg.moe_range_checks.restype = rel.moe_range_checks.restype = ctypes.c_int32
    assert rel.moe_range_checks() == 0 and dbg.moe_range_checks() == 1
    assert api.moe_range_checks() == 0  # the binding's default is the release library


def test_abi_version_and_status_strings():
    assert api.moe_abi_version() == 4
    for s in range(5):
        assert api.lib().moe_status_str(s).startswith(b"MOE_")


FAKE = 0x10000  # a non-null, aligned address that is never dereferenced here


def layer(**kw):
    d = dict(hidden=2048, inter=768, n_experts=512, top_k=10, qfmt=api.MOE_Q4_SYM_G32, act=api.MOE_ACT_BF16)
    d.update(kw)
    q = api.c_qmat(FAKE, FAKE, FAKE if d["qfmt"] == api.MOE_Q2_ASYM_G32 else None)
    ex = api.c_experts(q, q, q, d.pop("n_routed", d["n_experts"]))
    sh = api.c_experts(q, q, q, d.pop("n_shared", 1))
    return api.c_layer(d["hidden"], d["inter"], d["n_experts"], d["top_k"], d["qfmt"], d["act"],
                       d.pop("router_w", FAKE), None, ex, sh)


def ws_bytes(L, T):
    return api.lib().moe_workspace_bytes(ctypes.byref(L), T)


@pytest.mark.parametrize("kw,status", [
    (dict(top_k=0), api.MOE_E_ARG),
    (dict(top_k=513), api.MOE_E_ARG),
    (dict(hidden=2050), api.MOE_E_ARG),
    (dict(inter=100), api.MOE_E_ARG),
    (dict(hidden=8192), api.MOE_E_UNSUPPORTED),
    (dict(qfmt=7), api.MOE_E_UNSUPPORTED),
    (dict(act=5), api.MOE_E_UNSUPPORTED),
    (dict(n_routed=511), api.MOE_E_ARG),
    (dict(n_shared=2), api.MOE_E_UNSUPPORTED),
    (dict(router_w=None), api.MOE_E_ARG),
])
def test_bad_descriptor_rejected_before_launch(kw, status):
    L = layer(**kw)
    lib = api.lib()
    assert ws_bytes(L, 4) == 0
    got = lib.moe_layer_forward(ctypes.byref(L), FAKE, 4, FAKE, None, None, None, FAKE, 1 << 40, None)
    assert got == status


def test_q2_requires_mins():
    L = layer(qfmt=api.MOE_Q2_ASYM_G32)
    assert ws_bytes(L, 1) > 0
    L.routed.down.mins = None
    assert ws_bytes(L, 1) == 0


def test_negative_hot_experts_rejected():
    L = layer()
    L.hot_experts = -1
    assert ws_bytes(L, 1) == 0
    L.hot_experts = 10**6  # any count from 0 up is valid
    assert ws_bytes(L, 1) > 0


def test_q3_format_accepted_without_mins():
    L = layer(qfmt=api.MOE_Q3_SYM_G32)
    assert ws_bytes(L, 1) > 0
    q = api.c_qmat(FAKE, FAKE, None)
    assert api.lib().moe_dequant(ctypes.byref(q), api.MOE_Q3_SYM_G32, 4, 33, FAKE, None) == api.MOE_E_ARG


def test_token_count_rules():
    L = layer()
    lib = api.lib()
    r = ctypes.byref(L)
    assert lib.moe_layer_forward(r, FAKE, -1, FAKE, None, None, None, FAKE, 1 << 40, None) == api.MOE_E_ARG
    # T == 0 is a no-op that needs no buffers at all
    assert lib.moe_layer_forward(r, None, 0, None, None, None, None, None, 0, None) == api.MOE_OK
    assert lib.moe_router_topk(r, None, 0, None, None, None, None, 0, None) == api.MOE_OK
    assert lib.moe_expert_ffn_q(r, None, 0, None, None, None, None, None, None, None, None, 0, None) == api.MOE_OK
    assert lib.moe_combine(r, None, None, None, None, 0, None, None, None, None) == api.MOE_OK


def test_workspace_checks():
    L = layer()
    lib = api.lib()
    r = ctypes.byref(L)
    need = ws_bytes(L, 4)
    assert need > 0 and ws_bytes(L, 8) >= need  # monotone in T
    assert lib.moe_layer_forward(r, FAKE, 4, FAKE, None, None, None, FAKE, need - 1, None) == api.MOE_E_WORKSPACE
    assert lib.moe_layer_forward(r, FAKE, 4, FAKE, None, None, None, None, need, None) == api.MOE_E_WORKSPACE
    assert lib.moe_layer_forward(r, FAKE + 16, 4, FAKE, None, None, None, FAKE + 64, need, None) == api.MOE_E_ARG
    assert lib.moe_permute(r, FAKE, 4, FAKE, FAKE, FAKE, FAKE, need - 1, None) == api.MOE_E_WORKSPACE


def test_null_required_pointers():
    L = layer()
    lib = api.lib()
    r = ctypes.byref(L)
    need = ws_bytes(L, 2)
    assert lib.moe_layer_forward(None, FAKE, 2, FAKE, None, None, None, FAKE, need, None) == api.MOE_E_ARG
    assert lib.moe_layer_forward(r, None, 2, FAKE, None, None, None, FAKE, need, None) == api.MOE_E_ARG
    assert lib.moe_router_topk(r, FAKE, 2, None, FAKE, None, FAKE, need, None) == api.MOE_E_ARG
    assert lib.moe_combine(r, None, None, FAKE, FAKE, 2, FAKE, None, None, None) == api.MOE_E_ARG
    assert lib.moe_combine(r, FAKE, None, FAKE, FAKE, 2, FAKE, None, FAKE, None) == api.MOE_E_ARG  # x_next w/o x
    q = api.c_qmat(FAKE, FAKE, None)
    assert lib.moe_dequant(ctypes.byref(q), api.MOE_Q2_ASYM_G32, 4, 32, FAKE, None) == api.MOE_E_ARG
    assert lib.moe_dequant(ctypes.byref(q), 9, 4, 32, FAKE, None) == api.MOE_E_UNSUPPORTED
    assert lib.moe_dequant(ctypes.byref(q), api.MOE_Q4_SYM_G32, 4, 33, FAKE, None) == api.MOE_E_ARG


def test_stack_checks_every_layer():
    good, bad = layer(), layer(top_k=0)
    arr = (api.c_layer * 2)(good, bad)
    assert api.lib().moe_stack_forward(arr, 2, FAKE, 1, None, FAKE, 1 << 40, None) == api.MOE_E_ARG
    mixed = (api.c_layer * 2)(good, layer(hidden=1024))
    assert api.lib().moe_stack_forward(mixed, 2, FAKE, 1, None, FAKE, 1 << 40, None) == api.MOE_E_ARG


def test_binding_refuses_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(api, "_lib", None)
    monkeypatch.setattr(api, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no non-HIP fallback"):
        api.lib()


def test_bound_call_reports_the_status():
    """api.Bound re-issues one marshalled call: a rejected descriptor raises MoeError with the library's status
    (nothing is launched), and a T = 0 call is a no-op."""
    bad = layer(top_k=0)
    call = api.Bound("moe_layer_forward", (ctypes.byref(bad), FAKE, 4, FAKE, None, None, None, FAKE, 1 << 40, None),
                     keep=(bad,))
    for _ in range(2):
        with pytest.raises(api.MoeError) as e:
            call()
        assert e.value.status == api.MOE_E_ARG
    good = layer()
    api.Bound("moe_layer_forward", (ctypes.byref(good), None, 0, None, None, None, None, None, 0, None),
              keep=(good,))()


# ----------------------------------------------------------------------------- binding argument sizes

def fake_layer(T_hidden=64, inter=96, E=8, K=3, act=api.MOE_ACT_BF16):
    """A binding-level Layer without device tensors: only the fields the wrappers' checks read."""
    import torch
    L = object.__new__(api.Layer)
    L.hidden, L.inter, L.n_experts, L.top_k = T_hidden, inter, E, K
    L.act, L.qfmt = act, api.MOE_Q4_SYM_G32
    L.act_dtype = torch.bfloat16 if act == api.MOE_ACT_BF16 else torch.float32
    L.device = torch.device("cuda", 0)
    L.c = layer(hidden=T_hidden, inter=inter, n_experts=E, top_k=K)
    return L


def binding_calls(L, T):
    """(name, call(args), args) of every wrapper with correctly sized host tensors."""
    import torch
    K, E, H, I = L.top_k, L.n_experts, L.hidden, L.inter
    a, i32, f32 = L.act_dtype, torch.int32, torch.float32
    z = lambda n, d: torch.zeros(n, dtype=d)
    x = torch.zeros((T, H), dtype=a)
    return [
        ("moe_router_topk", lambda d: api.moe_router_topk(L, x, T, d["topk_ids"], d["topk_w"], d["logits"]),
         dict(topk_ids=z(T * K, i32), topk_w=z(T * K, f32), logits=z(T * E, f32))),
        ("moe_permute", lambda d: api.moe_permute(L, d["topk_ids"], T, d["expert_offsets"], d["sorted_pairs"],
                                                  d["pair_pos"], None),
         dict(topk_ids=z(T * K, i32), expert_offsets=z(E + 1, i32), sorted_pairs=z(T * K, i32),
              pair_pos=z(T * K, i32))),
        ("moe_expert_ffn_q", lambda d: api.moe_expert_ffn_q(L, x, T, d["topk_ids"], d["expert_offsets"],
                                                            d["sorted_pairs"], d["expert_out"], d["shared_out"],
                                                            d["h"], d["shared_h"]),
         dict(topk_ids=z(T * K, i32), expert_offsets=z(E + 1, i32), sorted_pairs=z(T * K, i32),
              expert_out=z(T * K * H, f32), shared_out=z(T * H, f32), h=z(T * K * I, a), shared_h=z(T * I, a))),
        ("moe_expert_gate_up_q", lambda d: api.moe_expert_gate_up_q(L, x, T, d["topk_ids"], d["expert_offsets"],
                                                                    d["sorted_pairs"], d["h"], d["shared_h"]),
         dict(topk_ids=z(T * K, i32), expert_offsets=z(E + 1, i32), sorted_pairs=z(T * K, i32),
              h=z(T * K * I, a), shared_h=z(T * I, a))),
        ("moe_expert_down_q", lambda d: api.moe_expert_down_q(L, d["h"], d["shared_h"], T, d["topk_ids"],
                                                              d["expert_offsets"], d["sorted_pairs"],
                                                              d["expert_out"], d["shared_out"]),
         dict(topk_ids=z(T * K, i32), expert_offsets=z(E + 1, i32), sorted_pairs=z(T * K, i32),
              h=z(T * K * I, a), shared_h=z(T * I, a), expert_out=z(T * K * H, f32), shared_out=z(T * H, f32))),
        ("moe_combine", lambda d: api.moe_combine(L, d["expert_out"], d["shared_out"], d["pair_pos"], d["topk_w"],
                                                  T, d["y"], d["x_resid"], d["x_next"]),
         dict(expert_out=z(T * K * H, f32), shared_out=z(T * H, f32), pair_pos=z(T * K, i32),
              topk_w=z(T * K, f32), y=z(T * H, f32), x_resid=z(T * H, a), x_next=z(T * H, a))),
        ("moe_layer_forward", lambda d: api.moe_layer_forward(L, x, T, d["y"], d["x_next"], d["topk_ids"],
                                                              d["topk_w"]),
         dict(y=z(T * H, f32), x_next=z(T * H, a), topk_ids=z(T * K, i32), topk_w=z(T * K, f32))),
        ("moe_stack_forward", lambda d: api.moe_stack_forward([L], x, T, d["y_last"]),
         dict(y_last=z(T * H, f32))),
    ]


CALLS = [c[0] for c in binding_calls(fake_layer(), 5)]


@pytest.mark.parametrize("name", CALLS)
def test_binding_rejects_every_undersized_buffer(name):
    """Each buffer one element short raises ValueError naming it, before any pointer is
    taken; with every buffer at its size the call gets past the size checks (and then
    stops at the device check, these being host tensors)."""
    L = fake_layer()
    call, args = {n: (c, a) for n, c, a in binding_calls(L, 5)}[name]
    for key, t in args.items():
        short = dict(args)
        short[key] = t[:-1]
        with pytest.raises(ValueError, match=f"{key}: .* at least {t.numel()} needed"):
            call(short)
    with pytest.raises(ValueError, match="device memory"):
        call(args)


def test_binding_checks_dequant_sizes():
    import torch
    out = torch.zeros(4 * 64, dtype=torch.float32)
    for qfmt, cb in (("q4_sym_g32", 4), ("q3_sym_g32", 3), ("q2_asym_g32", 2)):
        codes = torch.zeros(4 * 64 * cb // 8, dtype=torch.uint8)
        sc = torch.zeros(8, dtype=torch.int16)
        mins = sc if qfmt == "q2_asym_g32" else None
        with pytest.raises(ValueError, match="codes"):
            api.moe_dequant(codes[:-1], sc, mins, qfmt, 4, 64, out)
        with pytest.raises(ValueError, match="out"):
            api.moe_dequant(codes, sc, mins, qfmt, 4, 64, out[:-1])
        with pytest.raises(ValueError, match="device memory"):
            api.moe_dequant(codes, sc, mins, qfmt, 4, 64, out)
