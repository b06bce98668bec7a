"""GPU checks whose expected values are exact (bit for bit), through the C ABI.

* The dequantisation the expert kernels do in registers: one-hot rows of h
  (a single 1.0) through moe_expert_down_q make every output element a single
  dequantised down-projection weight, computed with exact arithmetic on every
  path (the offset codes, the group sums and the scale factors are all exact
  for a one-hot input), so o must equal the oracle's dequantised W_d column bit
  for bit.  Each down-projection kernel family is driven: the one-token
  kernel, the small-batch kernel, the per-expert GEMV (bf16 and fp32
  activations) and the matrix-core grouped GEMM.
* Exact logit ties: experts with identical router rows and biases have
  bitwise-equal logits, and the selection must order them by id (the lower id
  first) in every selection kernel: the fused one-token gate/up, the fused
  few-token gate/up, the one-block small-batch routing, the register top-k
  (after the fp32 and after the matrix-core router) and the LDS top-k.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import moe_oracle as mo
from sparse_moe_router_amd import api
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    api.lib()


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(gu.DEV)


# ----------------------------------------------------------------------------- one-hot down projections

# (name, T, K, E, hidden, inter, act): shapes that select each down-projection kernel
DOWN_PATHS = [
    ("one_token", 1, 10, 16, 2048, 768, "bf16"),      # k_down1
    ("small_batch", 8, 4, 8, 2048, 768, "bf16"),      # k_down_sb (T K <= 256)
    ("gemv", 100, 3, 64, 160, 768, "bf16"),           # k_down (T K > 256, H not a multiple of 128)
    ("gemv_f32", 20, 3, 8, 256, 768, "f32"),          # k_down, fp32 activations
    ("grouped_gemm", 512, 2, 8, 256, 768, "bf16"),    # k_expert_mfma (>= 8 tokens per expert)
]
FORMATS = ["q4_sym_g32", "q3_sym_g32", "q2_asym_g32"]


def _routing(T, K, E, seed):
    """Distinct experts per token (a seeded choice), the stable permutation from the oracle."""
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int64)
    off, sp, pp = mo.permute(ids, E)
    return ids, off, sp, pp


@pytest.mark.parametrize("qfmt", FORMATS)
@pytest.mark.parametrize("path", DOWN_PATHS, ids=[p[0] for p in DOWN_PATHS])
def test_one_hot_down_is_the_dequantised_column(path, qfmt):
    name, T, K, E, H, I, act = path
    spec = synth.LayerSpec("onehot", H, E, K, I, T, qfmt, act, 0.02, None, family=90 + E + K)
    ld = synth.gen_layer(spec)
    L = gu.device_layer(ld)
    ids, off, sp, pp = _routing(T, K, E, seed=T + K)
    n = T * K
    # sorted position j carries a one-hot h row at column (37 j + 5) mod I; the shared
    # expert's row t at column (11 t + 3) mod I
    cols = (37 * np.arange(n) + 5) % I
    scols = (11 * np.arange(T) + 3) % I
    dt = torch.bfloat16 if act == "bf16" else torch.float32
    h = torch.zeros((n, I), dtype=dt, device=gu.DEV)
    h[torch.arange(n, device=gu.DEV), _t(cols)] = 1.0
    hs = torch.zeros((T, I), dtype=dt, device=gu.DEV)
    hs[torch.arange(T, device=gu.DEV), _t(scols)] = 1.0
    o = torch.full((n, H), float("nan"), dtype=torch.float32, device=gu.DEV)
    so = torch.full((T, H), float("nan"), dtype=torch.float32, device=gu.DEV)
    gu.say(f"one-hot down: {name} T{T} K{K} E{E} H{H} I{I} {qfmt} {act}")
    api.moe_expert_down_q(L, h, hs, T, _t(ids.astype(np.int32)), _t(off.astype(np.int32)),
                          _t(sp.astype(np.int32)), o, so)
    torch.cuda.synchronize()
    got, sgot = o.cpu().numpy().astype(np.float64), so.cpu().numpy().astype(np.float64)
    flat = ids.reshape(-1)
    for e in np.unique(flat):
        wd = mo.dequant(ld.routed.down.codes[e], ld.routed.down.scales[e],
                        None if ld.routed.down.mins is None else ld.routed.down.mins[e], qfmt)
        rows = np.arange(off[e], off[e + 1])
        want = wd[:, cols[rows]].T
        assert np.array_equal(got[rows], want), f"expert {e}: max|do| {np.abs(got[rows] - want).max():.3e}"
    wds = mo.dequant(ld.shared.down.codes[0], ld.shared.down.scales[0],
                     None if ld.shared.down.mins is None else ld.shared.down.mins[0], qfmt)
    assert np.array_equal(sgot, wds[:, scols].T)


# ----------------------------------------------------------------------------- exact logit ties

def _tie_layer(E, K, H=256, I=64, family=95):
    """A layer whose router has groups of identical rows with identical biases,
    placed so that the top-K are (per group, by bias) tied pairs and the K-th and
    (K+1)-th slots fall inside one tied triple:  bias 400, 300, 200, ... per
    group (gaps far above |W x|), the rest of the experts a Zipf bias far below.
    All experts share one weight set (only the routing is under test)."""
    spec = synth.LayerSpec("ties", H, E, K, I, 1, "q4_sym_g32", "bf16", H ** -0.5, 1.1, family=family)
    ld = synth.gen_layer(spec, routed_ids=[0])
    rng = np.random.default_rng(E + K)
    w = ld.router_w.copy()
    b = (ld.router_b - 1000.0).astype(np.float32)
    npairs = (K - 1) // 2          # tied pairs fill slots 0 .. 2 npairs - 1
    rest = K - 2 * npairs           # 1 or 2 slots left: taken from a tied triple
    perm = rng.permutation(E)
    groups, at = [], 0
    for gi in range(npairs + 1):
        size = 2 if gi < npairs else 3
        g = np.sort(perm[at:at + size])
        at += size
        groups.append(g)
        w[g] = w[g[0]]
        b[g] = np.float32(400.0 - 100.0 * gi)
    expect = np.concatenate([g for g in groups[:-1]] + [groups[-1][:rest]])
    rep = lambda m: synth.PackedMat(np.repeat(m.codes, E, 0), np.repeat(m.scales, E, 0),
                                    None if m.mins is None else np.repeat(m.mins, E, 0))
    routed = synth.ExpertSet(rep(ld.routed.gate), rep(ld.routed.up), rep(ld.routed.down), np.arange(E))
    return synth.LayerData(spec, 0, w, b, routed, ld.shared), expect


def _check_tied(ld, x, ids, logits=None):
    K = ld.spec.top_k
    exact = mo.router_logits(x, ld.router_w, ld.router_b)
    want = mo.select_topk(exact, K)
    assert np.array_equal(ids, want), f"ids {ids[0].tolist()} vs {want[0].tolist()}"
    if logits is not None:  # the GPU's own logits of tied experts are bitwise equal
        sel = np.take_along_axis(logits, want, axis=-1)
        assert np.all(sel[:, 0] == sel[:, 1])


# (name, E, K, T, call): the selection kernel each case reaches
TIE_CASES = [
    ("fused_one_token", 512, 10, 1, "forward"),       # k_fused_gateup1 (E <= 512, K <= 16)
    ("fused_few_tokens_k20", 512, 20, 1, "forward"),  # k_fused_gateup (K > 16)
    ("route_small", 512, 10, 5, "forward"),           # k_route_small (T K <= 256)
    ("topk_regs_fp32_router", 512, 10, 3, "router"),  # k_router_logits + k_topk_regs
    ("topk_regs_mfma_router", 512, 10, 130, "router"),  # k_router_mfma split over k + k_topk_regs
    ("topk_regs_mfma_wide_router", 512, 10, 1030, "router"),  # k_router_mfma split over experts
    ("topk_lds", 1500, 10, 4, "router"),              # E > 1024: k_topk_lds
]


@pytest.mark.parametrize("case", TIE_CASES, ids=[c[0] for c in TIE_CASES])
def test_exact_ties_go_to_the_lower_id(case):
    name, E, K, T, call = case
    ld, expect = _tie_layer(E, K)
    x = synth.gen_x(ld.spec, tokens=T)
    L = gu.device_layer(ld)
    xd = gu.x_dev(x, "bf16")
    gu.say(f"ties: {name} E{E} K{K} T{T}; expected ids {expect.tolist()}")
    if call == "forward":
        f = gu.run_forward(L, xd, T)
        ids = f["ids"]
        logits = None
    else:
        idt = torch.empty((T, K), dtype=torch.int32, device=gu.DEV)
        wt = torch.empty((T, K), dtype=torch.float32, device=gu.DEV)
        lg = torch.empty((T, E), dtype=torch.float32, device=gu.DEV)
        api.moe_router_topk(L, xd, T, idt, wt, lg, api.workspace(L, T, gu.DEV))
        torch.cuda.synchronize()
        ids, logits = idt.cpu().numpy().astype(np.int64), lg.cpu().numpy().astype(np.float64)
    assert np.array_equal(ids, np.tile(expect, (T, 1)))
    _check_tied(ld, x.values, ids, logits)
