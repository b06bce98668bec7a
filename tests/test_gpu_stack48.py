"""The 48-layer stack of 512-expert MoE layers at its full shape (hidden 2048,
intermediate 768, top-10 + shared, 2-bit weights; 24,576 routed experts,
page 3 "How Strata Makes Your Entire PC Work Together") at batch 1 and 8,
through moe_stack_forward, checked layer by layer against the oracle.

The layers' expert planes are filled on the device (uniform codes, fp16 scales
and minima of the stack recipe); the routers come from the seeded generator.
moe_stack_forward must equal the layers run one after another with
moe_layer_forward bit for bit.  For every layer the test reads back the layer's
input x_l and the experts its tokens touched, and the oracle, fed x_l (teacher
forcing across layers), must agree: ids identical or a certified near-tie,
logits within the bound, the permutation bit-exact, every rounding-boundary
flip of h certified, y and the per-pair outputs within 2e-3 x RMS against the
oracle fed the GPU's certified h (the direct figure, against the oracle's own
rounding of h, is reported), and x_{l+1} exactly bf16(fp32(x_l + y_l)) of the
GPU's own y.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import synth
from oracle import moe_oracle as mo
from sparse_moe_router_amd import api
from synth import torch_io
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
N_LAYERS = 48
CHUNK = 12
_RUNS = {}


@pytest.fixture(scope="module")
def stack():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    spec = synth.SPECS["stack_t1"]
    assert spec.n_layers == N_LAYERS
    gu.say(f"filling the {N_LAYERS}-layer 2-bit stack on the device")
    kw = [torch_io.device_filled_kwargs(spec, l, gu.DEV) for l in range(N_LAYERS)]
    layers = [api.Layer(**k) for k in kw]
    yield spec, kw, layers
    _RUNS.clear()


def _run(stack, T):
    """The stack at T tokens: moe_stack_forward, and the layers one by one (inputs,
    routing, logits, y and x_next of every layer), on the host."""
    if T in _RUNS:
        return _RUNS[T]
    spec, _, layers = stack
    tspec = synth.SPECS["stack_t1" if T == 1 else "stack_t8"]
    assert tspec.tokens == T
    x0 = gu.x_dev(synth.gen_x(tspec), tspec.act)
    ws = api.workspace(layers[0], T, gu.DEV)
    xs = x0.clone()
    y_last = torch.empty((T, spec.hidden), dtype=torch.float32, device=gu.DEV)
    api.moe_stack_forward(layers, xs, T, y_last, ws)
    torch.cuda.synchronize()
    per = []
    cur = x0.clone()
    for l, L in enumerate(layers):
        f = gu.run_forward(L, cur, T, x_next=True)
        g = gu.run_steps(L, cur, T)  # the split calls: logits, permutation, h and per-pair outputs
        assert np.array_equal(g["ids"], f["ids"]) and np.array_equal(g["w"], f["w"])
        assert np.array_equal(g["y"], f["y"]), f"layer {l}: the split calls differ from moe_layer_forward"
        g["x"] = cur.float().cpu().numpy().astype(np.float64)
        g["x_next"] = f["x_next"].float().numpy().astype(np.float64)
        per.append(g)
        cur = f["x_next"].to(gu.DEV)
    assert torch.equal(xs.view(torch.int16), cur.view(torch.int16)), "stack differs from the layers one by one"
    assert np.array_equal(y_last.cpu().numpy(), per[-1]["y"])
    _RUNS[T] = per
    return per


def _layer_data(spec, kw, l, ids):
    """The oracle's view of layer l: its router, and the touched experts read back from the device."""
    w, b = synth.gen_router(spec, layer=l)
    used = np.unique(ids)
    idx = torch.from_numpy(used).to(gu.DEV)

    def mat(parts, sel):
        c, s, m = parts
        host = lambda t: None if t is None else t.index_select(0, sel).cpu().numpy()
        return synth.PackedMat(host(c), host(s).view(np.uint16), None if m is None else host(m).view(np.uint16))

    r, sh = kw["routed"], kw["shared"]
    zero = torch.zeros(1, dtype=torch.int64, device=gu.DEV)
    routed = synth.ExpertSet(mat(r["gate"], idx), mat(r["up"], idx), mat(r["down"], idx), used.astype(np.int64))
    shared = synth.ExpertSet(mat(sh["gate"], zero), mat(sh["up"], zero), mat(sh["down"], zero),
                             np.zeros(1, np.int64))
    return synth.LayerData(spec, l, w, b, routed, shared)


def _check_layer(spec, kw, l, g, T):
    ld = _layer_data(spec, kw, l, g["ids"])
    assert np.all(np.isfinite(g["y"])), f"layer {l}: y not finite"
    differs = gu.check_routing(ld, g["x"], g)
    gu.check_permutation(g, spec.n_experts)
    rf, direct, flips = gu.check_y_teacher_forced(ld, g["x"], g)
    assert np.array_equal(g["x_next"], mo.residual_step(g["x"], g["y"])), f"layer {l}: x_next"
    return rf, direct, flips, differs, len(np.unique(g["ids"]))


@pytest.mark.parametrize("chunk", range(N_LAYERS // CHUNK), ids=lambda c: f"layers{c * CHUNK}-{c * CHUNK + CHUNK - 1}")
@pytest.mark.parametrize("T", [1, 8])
def test_stack48_layers_against_oracle(stack, T, chunk):
    spec, kw, _ = stack
    per = _run(stack, T)
    ls = range(chunk * CHUNK, (chunk + 1) * CHUNK)
    with ThreadPoolExecutor(6) as ex:
        res = list(ex.map(lambda l: _check_layer(spec, kw[l], l, per[l], T), ls))
    worst = 0.0
    for l, (rf, direct, flips, differs, u) in zip(ls, res):
        worst = max(worst, direct)
        gu.say(f"  T={T} layer {l}: max|dy|/rms teacher-forced {rf:.2e}, direct {direct:.2e}; certified h flips "
               f"{flips}, differing ids {differs}; distinct experts {u}")
    gu.say(f"  T={T} layers {ls[0]}-{ls[-1]}: worst direct max|dy|/rms {worst:.2e}")
