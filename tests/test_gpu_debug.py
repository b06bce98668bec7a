"""The debug library (libmoe_debug.so) through the C ABI: the same results as
the release library for valid routing arrays, and MOE_E_ARG -- with nothing
else enqueued -- when a caller-provided id, offset, sorted pair or pair
position is out of range.  The bad values are only ever read by the range
check, inside their arrays' extents: no kernel indexes with them."""
import pytest
import torch

import synth
from sparse_moe_router_amd import api
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    api.use_debug_library(False)
    spec = synth.LayerSpec("debug", 256, 16, 4, 64, 6, "q4_sym_g32", "bf16", 256 ** -0.5, 1.1, family=97)
    ld = synth.gen_layer(spec)
    L = gu.device_layer(ld)
    x = gu.x_dev(synth.gen_x(spec), "bf16")
    yield spec, L, x
    api.use_debug_library(False)


def _run(spec, L, x, ws):
    """Router, permutation, expert FFNs and combine through the separate entry points."""
    T, K, E, H = spec.tokens, spec.top_k, spec.n_experts, spec.hidden
    i32 = dict(dtype=torch.int32, device=gu.DEV)
    ids, w = torch.empty((T, K), **i32), torch.empty((T, K), dtype=torch.float32, device=gu.DEV)
    off, srt, pos = torch.empty(E + 1, **i32), torch.empty(T * K, **i32), torch.empty(T * K, **i32)
    o = torch.empty((T * K, H), dtype=torch.float32, device=gu.DEV)
    so = torch.empty((T, H), dtype=torch.float32, device=gu.DEV)
    y = torch.empty((T, H), dtype=torch.float32, device=gu.DEV)
    api.moe_router_topk(L, x, T, ids, w, ws=ws)
    api.moe_permute(L, ids, T, off, srt, pos, ws)
    api.moe_expert_ffn_q(L, x, T, ids, off, srt, o, so, ws=ws)
    api.moe_combine(L, o, so, pos, w, T, y)
    torch.cuda.synchronize()
    return dict(ids=ids, w=w, off=off, srt=srt, pos=pos, o=o, so=so, y=y)


def test_debug_library_matches_the_release_library(setup):
    spec, L, x = setup
    ws = api.workspace(L, spec.tokens, gu.DEV)
    rel = _run(spec, L, x, ws)
    api.use_debug_library(True)
    try:
        assert api.moe_range_checks() == 1
        dbg = _run(spec, L, x, ws)
    finally:
        api.use_debug_library(False)
    for k in rel:
        assert torch.equal(rel[k], dbg[k]), k


@pytest.mark.parametrize("bad", ["id_E", "id_negative", "offsets_end", "offsets_order", "sorted", "pair_pos"])
def test_debug_library_rejects_out_of_range_routing(setup, bad):
    spec, L, x = setup
    T, K, E, H, I = spec.tokens, spec.top_k, spec.n_experts, spec.hidden, spec.inter
    ws = api.workspace(L, T, gu.DEV)
    r = _run(spec, L, x, ws)
    ids, off, srt, pos = (r[k].clone() for k in ("ids", "off", "srt", "pos"))
    if bad == "id_E":
        ids[2, 1] = E
    elif bad == "id_negative":
        ids[0, 0] = -3
    elif bad == "offsets_end":
        off[E] = T * K + 1
    elif bad == "offsets_order":
        off[1], off[2] = T * K, 0
    elif bad == "sorted":
        srt[3] = T * K
    elif bad == "pair_pos":
        pos[5] = -1
    gu.say(f"debug library, bad routing: {bad}")
    o = torch.full((T * K, H), float("nan"), dtype=torch.float32, device=gu.DEV)
    h = torch.full((T * K, I), float("nan"), dtype=torch.bfloat16, device=gu.DEV)
    y = torch.full((T, H), float("nan"), dtype=torch.float32, device=gu.DEV)
    api.use_debug_library(True)
    try:
        if bad.startswith("id"):
            o2, s2, p2 = torch.empty(E + 1, dtype=torch.int32, device=gu.DEV), torch.empty_like(srt), torch.empty_like(pos)
            with pytest.raises(api.MoeError) as ex:
                api.moe_permute(L, ids, T, o2, s2, p2, ws)
            assert ex.value.status == api.MOE_E_ARG
            with pytest.raises(api.MoeError) as ex:
                api.moe_expert_ffn_q(L, x, T, ids, r["off"], r["srt"], o, ws=ws)
            assert ex.value.status == api.MOE_E_ARG
        elif bad.startswith("offsets") or bad == "sorted":
            with pytest.raises(api.MoeError) as ex:
                api.moe_expert_gate_up_q(L, x, T, ids, off, srt, h)
            assert ex.value.status == api.MOE_E_ARG
            with pytest.raises(api.MoeError) as ex:
                api.moe_expert_down_q(L, torch.zeros((T * K, I), dtype=torch.bfloat16, device=gu.DEV), None, T,
                                      ids, off, srt, o)
            assert ex.value.status == api.MOE_E_ARG
        else:
            with pytest.raises(api.MoeError) as ex:
                api.moe_combine(L, r["o"], r["so"], pos, r["w"], T, y)
            assert ex.value.status == api.MOE_E_ARG
        torch.cuda.synchronize()
    finally:
        api.use_debug_library(False)
    # nothing was enqueued after the check: the outputs keep their fill
    assert torch.isnan(o).all() and torch.isnan(h.float()).all() and torch.isnan(y).all()
