"""Pins of the CPU oracle against things other than itself (CPU only).

* brute force: the scalar pure-Python oracle on tiny layers (config 'tiny' and
  200+ random tiny shapes, both formats, both activation types);
* textbook routines: top-k against numpy.lexsort, the permutation against a
  stable argsort and a counting loop;
* closed forms and special cases: K = E gives the full softmax, E = K = 1 is a
  dense SwiGLU FFN, a zero router gives ids 0..K-1 with weights 1/K, x = 0 gives
  y = 0 exactly;
* exhaustive dequant against struct-decoded halves, and the quantizer round trip;
* invariants: weights sum to 1, expert relabelling, token permutation, exact
  doubling under power-of-two down-projection scales.
"""
import math
import struct

import numpy as np
import pytest
from scipy.special import softmax

import synth
from oracle import bruteforce as bf
from oracle import moe_oracle as mo


def small_spec(rng, qfmt=None, act=None, hidden=None, e=None, k=None, inter=None, t=None, bias=None):
    hidden = hidden or int(rng.choice([32, 64]))
    e = e or int(rng.integers(1, 17))
    k = k or int(rng.integers(1, e + 1))
    inter = inter or int(rng.choice([32, 64, 128]))
    t = t or int(rng.integers(1, 9))
    qfmt = qfmt or str(rng.choice([synth.Q4, synth.Q3, synth.Q2]))
    act = act or (synth.ACT_F32 if rng.random() < 0.5 else synth.ACT_BF16)
    use_bias = bool(rng.random() < 0.5) if bias is None else bias
    return synth.LayerSpec("rand", hidden, e, k, inter, t, qfmt, act, 0.3, 1.1 if use_bias else None,
                           family=99 + int(rng.integers(0, 1 << 30)))


def run_both(spec, seed=0):
    layer = synth.gen_layer(spec, seed=seed, threads=1)
    x = synth.gen_x(spec, seed=seed).values
    ref = mo.layer_forward(layer, x)
    brute = bf.layer_forward(layer, x.astype(np.float64).tolist())
    return layer, x, ref, brute


def check_agree(ref, brute):
    assert np.array_equal(ref["ids"], np.array(brute["ids"]))
    assert np.array_equal(ref["offsets"], np.array(brute["offsets"]))
    assert np.array_equal(ref["sorted_pairs"], np.array(brute["sorted_pairs"]))
    assert np.array_equal(ref["pair_pos"], np.array(brute["pair_pos"]))
    np.testing.assert_allclose(ref["w"], np.array(brute["w"]), rtol=1e-12, atol=0)
    y_b = np.array(brute["y"])
    scale = max(np.abs(y_b).max(), 1e-300)
    assert np.abs(ref["y"] - y_b).max() <= 1e-12 * scale


# ----------------------------------------------------------------------------- P1

def test_tiny_config_bruteforce():
    spec = synth.SPECS["tiny"]
    _, _, ref, brute = run_both(spec)
    check_agree(ref, brute)
    assert ref["y"].shape == (4, 64)
    assert np.all(np.abs(ref["y"]) > 0)


@pytest.mark.parametrize("block", range(4))
def test_random_tiny_shapes_bruteforce(block):
    rng = np.random.default_rng(1234 + block)
    for _ in range(52):
        spec = small_spec(rng)
        _, _, ref, brute = run_both(spec, seed=int(rng.integers(0, 1000)))
        check_agree(ref, brute)


# ----------------------------------------------------------------------------- P2

def test_topk_matches_lexsort():
    rng = np.random.default_rng(5)
    for _ in range(50):
        t, e = int(rng.integers(1, 20)), int(rng.integers(1, 70))
        k = int(rng.integers(1, e + 1))
        # coarse values create many exact ties
        logits = rng.integers(-4, 5, size=(t, e)).astype(np.float64) * 0.5
        ids = mo.select_topk(logits, k)
        for tt in range(t):
            ref = np.lexsort((np.arange(e), -logits[tt]))[:k]
            assert np.array_equal(ids[tt], ref)


def test_permute_matches_textbook():
    rng = np.random.default_rng(6)
    for _ in range(50):
        e = int(rng.integers(1, 40))
        t, k = int(rng.integers(0, 30)), int(rng.integers(1, 6))
        ids = rng.integers(0, e, size=(t, k))
        off, sp, pp = mo.permute(ids, e)
        flat = ids.reshape(-1)
        # counting loop
        cnt = [0] * e
        for v in flat:
            cnt[v] += 1
        assert off.tolist() == [0] + list(np.cumsum(cnt)) if e else True
        # stable sort by expert, equal experts in pair order
        pairs = sorted(range(flat.size), key=lambda p: (flat[p], p))
        assert sp.tolist() == pairs
        assert all(sp[pp[p]] == p for p in range(flat.size))


# ----------------------------------------------------------------------------- P3

def test_k_equals_e_gives_full_softmax():
    rng = np.random.default_rng(7)
    spec = small_spec(rng, e=6, k=6, t=5, bias=True)
    layer = synth.gen_layer(spec, threads=1)
    x = synth.gen_x(spec).values
    ref = mo.layer_forward(layer, x)
    logits = x.astype(np.float64) @ layer.router_w.astype(np.float64).T + layer.router_b
    full = softmax(logits, axis=-1)
    np.testing.assert_allclose(ref["w"], np.take_along_axis(full, ref["ids"], -1), rtol=1e-13)
    assert np.array_equal(np.sort(ref["ids"], -1), np.tile(np.arange(6), (5, 1)))


def _on_grid_q4(rng, rows, cols, exp):
    """Float weights that the 4-bit quantizer represents exactly: s = 2^exp, codes in [-7, 7], amax = 7 s."""
    q = rng.integers(-7, 8, size=(rows, cols))
    q[:, ::32] = 7 * rng.choice([-1, 1], size=(rows, cols // 32))
    return (q * 2.0 ** exp).astype(np.float32)


@pytest.mark.parametrize("act", [synth.ACT_F32, synth.ACT_BF16])
def test_single_expert_is_dense_swiglu(act):
    """E = K = 1: the layer is routed-expert + shared-expert SwiGLU with weight 1 (closed form via matmul)."""
    rng = np.random.default_rng(8)
    h_, i_ = 64, 96
    spec = synth.LayerSpec("dense", h_, 1, 1, i_, 3, synth.Q4, act, 0.1, None, family=7)
    mats = [_on_grid_q4(rng, *shape, exp) for shape, exp in
            [((i_, h_), -6), ((i_, h_), -5), ((h_, i_), -7), ((i_, h_), -5), ((i_, h_), -6), ((h_, i_), -6)]]
    packed = [synth.quantize_q4(m) for m in mats]

    def eset(parts, idx):
        pm = [synth.PackedMat(c[None], s[None]) for c, s in parts]
        return synth.ExpertSet(*pm, index=np.array([idx]))

    layer = synth.LayerData(spec, 0, rng.standard_normal((1, h_)).astype(np.float32), None,
                            eset(packed[:3], 0), eset(packed[3:], 1))
    x = rng.standard_normal((3, h_)).astype(np.float32)
    if act == synth.ACT_BF16:
        x = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    ref = mo.layer_forward(layer, x)
    x64 = x.astype(np.float64)

    def ffn(wg, wu, wd):
        g, u = x64 @ wg.T.astype(np.float64), x64 @ wu.T.astype(np.float64)
        h = g / (1 + np.exp(-g)) * u
        h = h.astype(np.float32).astype(np.float64)
        if act == synth.ACT_BF16:
            h = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(h.astype(np.float32))).astype(np.float64)
        return h @ wd.T.astype(np.float64)

    want = ffn(*mats[3:]) + ffn(*mats[:3])
    assert np.array_equal(ref["ids"], np.zeros((3, 1)))
    assert np.all(ref["w"] == 1.0)
    np.testing.assert_allclose(ref["y"], want, rtol=1e-12, atol=1e-14)


def test_zero_router_picks_first_k_uniformly():
    rng = np.random.default_rng(9)
    spec = small_spec(rng, e=12, k=5, t=4, bias=False)
    layer = synth.gen_layer(spec, threads=1)
    layer.router_w[:] = 0
    ref = mo.layer_forward(layer, synth.gen_x(spec).values)
    assert np.array_equal(ref["ids"], np.tile(np.arange(5), (4, 1)))
    assert np.all(ref["w"] == 0.2)


def test_zero_input_gives_zero_output():
    rng = np.random.default_rng(10)
    for qfmt in (synth.Q4, synth.Q2):
        spec = small_spec(rng, qfmt=qfmt, e=8, k=3, t=3, bias=True)
        layer = synth.gen_layer(spec, threads=1)
        ref = mo.layer_forward(layer, np.zeros((3, spec.hidden)))
        assert np.all(ref["y"] == 0.0)


# ----------------------------------------------------------------------------- P4, P5

def _all_finite_f16_bits():
    b = np.arange(1 << 16, dtype=np.uint32)
    return b[((b >> 10) & 0x1F) != 0x1F].astype(np.uint16)


def test_dequant_q4_exhaustive():
    """Every code x every finite fp16 scale, against struct-decoded halves."""
    sb = _all_finite_f16_bits()
    codes_u = np.tile(np.arange(16, dtype=np.uint8), 2)       # 32 codes = one group
    packed = synth.pack_q4(np.tile(codes_u, (sb.size, 1)))
    got = mo.dequant_q4(packed, sb[:, None])
    halves = np.array([struct.unpack("<e", struct.pack("<H", int(v)))[0] for v in sb])
    want = halves[:, None] * (codes_u.astype(np.float64) - 8)[None, :]
    assert np.array_equal(got, want)
    # every value is exactly a float32
    assert np.array_equal(got.astype(np.float32).astype(np.float64), got)


def test_dequant_q2_grid():
    rng = np.random.default_rng(11)
    sb = _all_finite_f16_bits()
    s_bits = np.concatenate([sb, rng.choice(sb, 20000)])
    m_bits = np.concatenate([rng.choice(sb, sb.size), rng.choice(sb, 20000)])
    codes_u = np.tile(np.arange(4, dtype=np.uint8), 8)
    packed = synth.pack_q2(np.tile(codes_u, (s_bits.size, 1)))
    got = mo.dequant_q2(packed, s_bits[:, None], m_bits[:, None])
    dec = lambda v: struct.unpack("<e", struct.pack("<H", int(v)))[0]
    f32 = lambda v: struct.unpack("<f", struct.pack("<f", v))[0]
    for r in range(0, s_bits.size, 97):
        s, m = dec(s_bits[r]), dec(m_bits[r])
        want = [f32(s * u + m) for u in codes_u.tolist()]
        assert got[r].tolist() == want


def test_q3_layout_hand_packed_bytes():
    """The 3-bit layout on bytes written out by hand: codes u_i = i mod 8 give
    low fields (0, 1, 2, 3) in every low byte (0xE4) and the third bit set for
    elements 4..7 of every 8 (0xF0); a lone code 7 at element 13 sets bits 2, 3
    of byte 3 and bit 5 of byte 9."""
    a = np.array([0xE4] * 8 + [0xF0] * 4, np.uint8)
    assert mo.unpack_q3(a).tolist() == [i % 8 for i in range(32)]
    b = np.zeros(12, np.uint8)
    b[3], b[9] = 0x0C, 0x20
    want = [0] * 32
    want[13] = 7
    assert mo.unpack_q3(b).tolist() == want
    # two groups per row: the second group's 12 bytes follow the first's
    assert mo.unpack_q3(np.concatenate([b, a])).tolist() == want + [i % 8 for i in range(32)]
    assert synth.pack_q3(np.array([i % 8 for i in range(32)], np.uint8)).tolist() == a.tolist()


def test_dequant_q3_exhaustive():
    """Every code x every finite fp16 scale, against struct-decoded halves, and the
    scalar decoder of the brute-force oracle on random packed rows."""
    sb = _all_finite_f16_bits()
    codes_u = np.tile(np.arange(8, dtype=np.uint8), 4)
    packed = synth.pack_q3(np.tile(codes_u, (sb.size, 1)))
    got = mo.dequant_q3(packed, sb[:, None])
    halves = np.array([struct.unpack("<e", struct.pack("<H", int(v)))[0] for v in sb])
    want = halves[:, None] * (codes_u.astype(np.float64) - 4)[None, :]
    assert np.array_equal(got, want)
    assert np.array_equal(got.astype(np.float32).astype(np.float64), got)
    rng = np.random.default_rng(21)
    for _ in range(20):
        row = rng.integers(0, 256, size=12 * 3, dtype=np.uint8)
        assert mo.unpack_q3(row).tolist() == [bf.code3(row.tolist(), c) for c in range(96)]


def test_quantizer_round_trip():
    rng = np.random.default_rng(12)
    for _ in range(20):
        rows = 8
        u4 = rng.integers(0, 16, size=(rows, 64)).astype(np.uint8)
        s4 = synth.f64_to_f16_bits(rng.uniform(1e-3, 1.0, size=(rows, 2)))
        w4 = mo.dequant_q4(synth.pack_q4(u4), s4)
        assert np.array_equal(synth.requantize_codes_q4(w4, s4), u4)
        u2 = rng.integers(0, 4, size=(rows, 64)).astype(np.uint8)
        s2 = synth.f64_to_f16_bits(rng.uniform(1e-3, 1.0, size=(rows, 2)))
        m2 = synth.f64_to_f16_bits(-1.5 * rng.uniform(1e-3, 1.0, size=(rows, 2)))
        w2 = mo.dequant_q2(synth.pack_q2(u2), s2, m2)
        assert np.array_equal(synth.requantize_codes_q2(w2, s2, m2), u2)
        u3 = rng.integers(0, 8, size=(rows, 64)).astype(np.uint8)
        s3 = synth.f64_to_f16_bits(rng.uniform(1e-3, 1.0, size=(rows, 2)))
        w3 = mo.dequant_q3(synth.pack_q3(u3), s3)
        assert np.array_equal(synth.requantize_codes_q3(w3, s3), u3)


def test_quantizer_error_within_half_step():
    rng = np.random.default_rng(13)
    w = rng.standard_normal((16, 128)).astype(np.float32) * 0.02
    c4, s4 = synth.quantize_q4(w)
    d4 = mo.dequant_q4(c4, s4)
    step = np.repeat(s4.view(np.float16).astype(np.float64), 32, -1)
    assert np.all(np.abs(d4 - w) <= 0.5 * step * (1 + 1e-3) + 1e-12)
    c3, s3 = synth.quantize_q3(w)
    d3 = mo.dequant_q3(c3, s3)
    step3 = np.repeat(s3.view(np.float16).astype(np.float64), 32, -1)
    assert np.all(np.abs(d3 - w) <= 0.5 * step3 * (1 + 1e-3) + 1e-12)
    c2, s2, m2 = synth.quantize_q2(w)
    d2 = mo.dequant_q2(c2, s2, m2)
    step2 = np.repeat(s2.view(np.float16).astype(np.float64), 32, -1)
    assert np.all(np.abs(d2 - w) <= 0.5 * step2 * 1.01 + 1e-4)


# ----------------------------------------------------------------------------- P6 .. P9

def test_weights_sum_to_one():
    rng = np.random.default_rng(14)
    for _ in range(20):
        spec = small_spec(rng, bias=True)
        layer = synth.gen_layer(spec, threads=1)
        ref = mo.layer_forward(layer, synth.gen_x(spec).values)
        assert np.all(np.abs(ref["w"].sum(-1) - 1) <= 1e-15)
        assert np.all(ref["w"] > 0) and np.all(np.diff(ref["w"], axis=-1) <= 0)


def _relabel(layer, perm):
    """Expert e becomes expert perm[e]: router rows, bias and expert slots move together."""
    inv = np.argsort(perm)
    es = layer.routed
    moved = synth.subset(es, inv)
    moved.index = np.arange(len(perm))
    return synth.LayerData(layer.spec, layer.layer, layer.router_w[inv].copy(),
                           None if layer.router_b is None else layer.router_b[inv].copy(), moved, layer.shared)


def test_expert_relabelling_invariance():
    rng = np.random.default_rng(15)
    for _ in range(10):
        spec = small_spec(rng, bias=True, t=6)
        layer = synth.gen_layer(spec, threads=1)
        x = synth.gen_x(spec).values
        ref = mo.layer_forward(layer, x)
        perm = rng.permutation(spec.n_experts)
        ref2 = mo.layer_forward(_relabel(layer, perm), x)
        assert np.array_equal(ref2["ids"], perm[ref["ids"]])
        # exact in exact arithmetic; the float64 router product may round a moved
        # row differently in the last bit (the BLAS blocking depends on row position)
        np.testing.assert_allclose(ref2["w"], ref["w"], rtol=1e-14, atol=0)
        np.testing.assert_allclose(ref2["y"], ref["y"], rtol=1e-14, atol=1e-16)


def test_token_permutation_equivariance():
    rng = np.random.default_rng(16)
    for _ in range(10):
        spec = small_spec(rng, t=8)
        layer = synth.gen_layer(spec, threads=1)
        x = synth.gen_x(spec).values
        perm = rng.permutation(spec.tokens)
        a = mo.layer_forward(layer, x)
        b = mo.layer_forward(layer, x[perm])
        assert np.array_equal(b["ids"], a["ids"][perm])
        np.testing.assert_allclose(b["y"], a["y"][perm], rtol=1e-13, atol=1e-16)


def _double_down(layer):
    def dbl(es):
        d = es.down
        s = (d.scales.view(np.float16) * np.float16(2)).view(np.uint16)
        m = None if d.mins is None else (d.mins.view(np.float16) * np.float16(2)).view(np.uint16)
        return synth.ExpertSet(es.gate, es.up, synth.PackedMat(d.codes, s, m), es.index)
    return synth.LayerData(layer.spec, layer.layer, layer.router_w, layer.router_b, dbl(layer.routed), dbl(layer.shared))


def test_power_of_two_down_scales_double_y_exactly():
    rng = np.random.default_rng(17)
    for qfmt in (synth.Q4, synth.Q2):
        spec = small_spec(rng, qfmt=qfmt, t=5, bias=True)
        layer = synth.gen_layer(spec, threads=1)
        x = synth.gen_x(spec).values
        a = mo.layer_forward(layer, x)
        b = mo.layer_forward(_double_down(layer), x)
        assert np.array_equal(b["y"], 2 * a["y"])


# ----------------------------------------------------------------------------- hand-checked case

def test_hand_worked_layer():
    """H = I = 32, E = 2, K = 1, T = 1, 4-bit, fp32 activations, every weight of a matrix equal.

    Router row 1 = 0.5 e_0, row 0 = 0; x = e_0, so expert 1 wins with weight 1.
    Expert 1: gate codes q = 1 at scale 1 -> g = 1; up q = 2 at scale 0.5 -> u = 1;
    h = fp32(silu(1)); down q = 1 at scale 0.25 -> o_j = 32 * 0.25 * h.
    Shared: gate q = -1 -> g = -1; up q = 1 -> u = 1; h_s = fp32(silu(-1)); down q = 3 at
    scale 0.5 -> s_j = 32 * 1.5 * h_s.  y_j = s_j + o_j for every j.
    """
    spec = synth.LayerSpec("hand", 32, 2, 1, 32, 1, synth.Q4, synth.ACT_F32, 0.0, None, family=0)

    def mat(q, s):
        u = np.full((1, 32, 32), q + 8, np.uint8)
        return synth.PackedMat(synth.pack_q4(u), synth.f64_to_f16_bits(np.full((1, 32, 1), s)))

    routed = synth.ExpertSet(mat(1, 1.0), mat(2, 0.5), mat(1, 0.25), index=np.array([1]))
    shared = synth.ExpertSet(mat(-1, 1.0), mat(1, 1.0), mat(3, 0.5), index=np.array([2]))
    rw = np.zeros((2, 32), np.float32)
    rw[1, 0] = 0.5
    layer = synth.LayerData(spec, 0, rw, None, routed, shared)
    x = np.zeros((1, 32))
    x[0, 0] = 1.0
    ref = mo.layer_forward(layer, x)
    f32 = lambda v: struct.unpack("<f", struct.pack("<f", v))[0]
    h1 = f32(1.0 / (1.0 + math.exp(-1.0)))
    hs = f32(-1.0 / (1.0 + math.exp(1.0)))
    assert ref["ids"].tolist() == [[1]] and ref["w"].tolist() == [[1.0]]
    assert np.allclose(ref["y"], 32 * 1.5 * hs + 32 * 0.25 * h1, rtol=1e-15, atol=0)


# ----------------------------------------------------------------------------- rounding points

def _torch_bf16(v32):
    """torch's CPU float32 -> bfloat16 conversion (round to nearest, ties to even)."""
    import torch
    return torch.from_numpy(np.asarray(v32, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def test_round_bf16_exact_ties_against_torch():
    """float32 values whose low half is exactly 0x8000 (a tie), with bit 16 even and
    odd, both signs, normal and subnormal, round to even as torch's conversion does;
    values one ulp either side of the tie round to the nearer neighbour."""
    his = np.array([0x3F80, 0x3F81, 0x4049, 0x404A, 0x0001, 0x0002, 0x7F7E, 0x7F7D, 0x0080, 0x3FFF], np.uint32)
    his = np.concatenate([his, his | 0x8000])
    ties = ((his << 16) | 0x8000).astype(np.uint32)
    near = np.concatenate([ties, ties - 1, ties + 1])
    v = near.view(np.float32)
    got = mo.round_bf16(v.astype(np.float64))
    assert np.array_equal(got, _torch_bf16(v).astype(np.float64))
    # the tie cases written out: even upper halves stay, odd ones go up by one unit
    t = ties.view(np.float32)
    want_bits = np.where(his & 1, his + 1, his) << 16
    assert np.array_equal(got[:ties.size], want_bits.astype(np.uint32).view(np.float32).astype(np.float64))
    assert np.array_equal(got[:ties.size], np.array([bf.to_bf16(float(a)) for a in t]))


def test_round_bf16_goes_through_float32():
    """The storage rounding of h (and of the residual stream) is fp32 first, then bf16.
    1 + 2^-8 + 2^-30 lies above the bf16 tie 1 + 2^-8, but its fp32 rounding is the
    tie itself (2^-30 is below half an fp32 ulp at 1), which then rounds to even:
    1.0.  A single rounding from float64 would give 1 + 2^-7."""
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert mo.round_bf16(np.array([v])).tolist() == [1.0]
    assert mo.round_bf16(np.array([-v])).tolist() == [-1.0]
    assert bf.to_bf16(v) == 1.0
    # just above the fp32 half ulp the fp32 value moves off the tie and bf16 rounds up
    w = 1.0 + 2.0 ** -8 + 2.0 ** -23
    assert mo.round_bf16(np.array([w])).tolist() == [1.0 + 2.0 ** -7]


def test_residual_step_rounds_fp32_then_bf16():
    """x_next = bf16(fp32(x + y)) with bf16 x and fp32 y, on sums where the two-step
    rounding differs from one rounding of the exact sum (values worked by hand):
      1 + fp32(2^-8 + 2^-30)          -> 1.0        (one rounding: 1 + 2^-7)
      (1 + 2^-7) + 2^-8               -> 1 + 2^-6   (an exact tie, odd -> even, up)
      256 + fp32(-(2^-1 + 2^-24))     -> 256.0      (fp32 sum is 255.5, a tie, even stays;
                                                     one rounding: 255.0)
      -3 + fp32(-2^-7 - 2^-28)        -> -3.0       (fp32 sum is the tie -(3 + 2^-7);
                                                     one rounding: -3.015625)"""
    f32 = lambda v: struct.unpack("<f", struct.pack("<f", v))[0]
    cases = [
        (1.0, f32(2.0 ** -8 + 2.0 ** -30), 1.0),
        (1.0 + 2.0 ** -7, 2.0 ** -8, 1.0 + 2.0 ** -6),
        (256.0, f32(-(2.0 ** -1 + 2.0 ** -24)), 256.0),
        (-3.0, f32(-(2.0 ** -7 + 2.0 ** -28)), -3.0),
    ]
    for x, y, want in cases:
        assert f32(y) == y
        assert mo.residual_step(np.array([[x]]), np.array([[y]])).tolist() == [[want]], (x, y)


# ----------------------------------------------------------------------------- router bound helpers

def _router_case():
    rng = np.random.default_rng(18)
    x = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(rng.standard_normal((3, 2048)).astype(np.float32)))
    w = (rng.standard_normal((16, 2048)) * 0.022).astype(np.float32)
    b = rng.standard_normal(16).astype(np.float32)
    return x, w, b


def test_router_bound_covers_fp32_evaluation():
    """An fp32 dot-product evaluation of the logits (sequential sum) stays within
    the one-part bound gamma_{H+1} (sum |W x| + |b|)."""
    x, w, b = _router_case()
    exact = mo.router_logits(x, w, b)
    beta = mo.router_error_bound(x, w, b)
    f32 = np.zeros((3, 16), np.float32)
    for i in range(2048):
        f32 = (f32 + x[:, i:i + 1] * w[None, :, i]).astype(np.float32)
    f32 = (f32 + b).astype(np.float32)
    assert np.all(np.abs(f32.astype(np.float64) - exact) <= beta)
    # the bound is the textbook gamma_{H+1}: 2049 u / (1 - 2049 u) times the magnitudes
    mag = np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T + np.abs(b.astype(np.float64))
    g = 2049 * 2.0 ** -24 / (1 - 2049 * 2.0 ** -24)
    assert np.allclose(beta, g * mag, rtol=1e-15, atol=0)


def test_router_bound_covers_three_part_split():
    """The logits evaluated as 3 H exact products of x with the bf16 parts of each
    fp32 weight (hi, mid, lo by truncation), summed in fp32, stay within the
    three-part bound; the parts are exact (hi + mid + lo == w)."""
    x, w, b = _router_case()
    trunc = lambda a: (np.asarray(a, np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32)
    hi = trunc(w)
    mid = trunc((w - hi).astype(np.float32))
    lo = ((w - hi).astype(np.float32) - mid).astype(np.float32)
    assert np.array_equal(hi.astype(np.float64) + mid + lo, w.astype(np.float64))
    exact = mo.router_logits(x, w, b)
    beta3 = mo.router_error_bound(x, w, b, parts=3)
    acc = np.zeros((3, 16), np.float32)
    for part in (lo, mid, hi):
        for i in range(2048):
            acc = (acc + x[:, i:i + 1] * part[None, :, i]).astype(np.float32)
    acc = (acc + b).astype(np.float32)
    assert np.all(np.abs(acc.astype(np.float64) - exact) <= beta3)
    assert np.all(beta3 > mo.router_error_bound(x, w, b))


def test_certify_ids_rules():
    logits = np.array([[3.0, 2.0, 2.0 + 1e-9, 0.0]])
    beta = np.full_like(logits, 1e-6)
    ok, differs = mo.certify_ids(logits, beta, [[0, 2]], [[0, 1]])
    assert ok and differs.tolist() == [True]
    ok, _ = mo.certify_ids(logits, beta, [[0, 3]], [[0, 1]])
    assert not ok
