"""moe_layer_forward_noalloc (the layer with the library's own device array in
place of a workspace) gives the bits of moe_layer_forward with a caller
workspace, through the C ABI: two calls in a row on one layer, the second with
fewer tokens (the array keeps the first call's contents), each compared with
the workspace call on the same input; a token count whose workspace exceeds
the array is refused before anything runs."""
import numpy as np
import pytest
import torch

import synth
from sparse_moe_router_amd import api
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    api.lib()


def _both(L, xd, T):
    """(noalloc, workspace) results of one call each: y, x_next, ids, weights."""
    out = []
    for noalloc in (True, False):
        y = torch.full((T, L.hidden), float("nan"), dtype=torch.float32, device=gu.DEV)
        xn = torch.zeros((T, L.hidden), dtype=L.act_dtype, device=gu.DEV)
        ids = torch.full((T, L.top_k), -1, dtype=torch.int32, device=gu.DEV)
        w = torch.zeros((T, L.top_k), dtype=torch.float32, device=gu.DEV)
        if noalloc:
            api.moe_layer_forward_noalloc(L, xd[:T], T, y, xn, ids, w)
        else:
            api.moe_layer_forward(L, xd[:T], T, y, xn, ids, w, ws=api.workspace(L, T, gu.DEV))
        torch.cuda.synchronize()
        out.append((y.cpu().numpy(), xn.view(torch.int16).cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()))
    return out


@pytest.mark.parametrize("qfmt,sizes", [("q2_asym_g32", (64, 5)), ("q4_sym_g32", (8, 1))],
                         ids=["q2_T64_then_T5", "q4_T8_then_T1"])
def test_noalloc_matches_workspace_call(qfmt, sizes):
    spec = synth.LayerSpec("noalloc", 2048, 512, 10, 768, max(sizes), qfmt, "bf16", 2048 ** -0.5, 1.1, family=97)
    ld = synth.gen_layer(spec)
    L = gu.device_layer(ld)
    xd = gu.x_dev(synth.gen_x(spec), spec.act)
    for T in sizes:
        assert api.moe_workspace_bytes(L, T) <= api.NOALLOC_SCRATCH_BYTES
        a, b = _both(L, xd, T)
        gu.say(f"noalloc {qfmt} T={T}: max|dy| {np.abs(a[0] - b[0]).max():.1e}")
        for got, want in zip(a, b):
            assert np.array_equal(got, want)


def test_noalloc_refuses_more_than_its_array():
    spec = synth.LayerSpec("noalloc_big", 2048, 16, 10, 768, 1, "q4_sym_g32", "bf16", 2048 ** -0.5, 1.1, family=98)
    L = gu.device_layer(synth.gen_layer(spec))
    T = 1
    while api.moe_workspace_bytes(L, T) <= api.NOALLOC_SCRATCH_BYTES:
        T *= 2
    x = torch.zeros((T, 2048), dtype=torch.bfloat16, device=gu.DEV)
    y = torch.full((T, 2048), 7.0, dtype=torch.float32, device=gu.DEV)
    with pytest.raises(api.MoeError) as e:
        api.moe_layer_forward_noalloc(L, x, T, y)
    assert e.value.status == api.MOE_E_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
