"""Byte and flop counts, and the layer shapes, against what the pages state and
closed forms (CPU only).

The page facts sit in tests/golden/page_facts.json, each with its citation."""
import json
import os

import synth
from sparse_moe_router_amd import workload as wl

FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def fact(name):
    return FACTS[name]["value"]


def test_layer_shape_matches_the_pages():
    for name in ("decode", "verify", "prefill", "stack_t1", "stack_t8"):
        s = synth.SPECS[name]
        assert s.n_experts == fact("experts_per_layer")
        assert s.top_k == fact("routed_experts_per_token")
        assert s.n_shared == fact("shared_experts_per_token")
    assert synth.SPECS["verify"].tokens == fact("verify_batch_tokens")
    st = synth.SPECS["stack_t1"]
    assert st.n_layers * st.n_experts == fact("total_experts")


def test_two_bit_codes_compress_fp16_eightfold():
    assert 16 // wl.code_bits("q2_asym_g32") == fact("two_bit_compression_vs_fp16")


def test_expert_size_is_consistent_with_the_pages_totals():
    """3 H I weights per expert: the 24,576 experts hold most of the 125B parameters,
    and a 2-bit group-32 scale-only pack (2.5 bits per weight) gives ~700 experts
    per GB, as the pages state."""
    s = synth.SPECS["decode"]
    per_expert = 3 * s.hidden * s.inter
    total = fact("total_experts") * per_expert
    assert 0.85 * fact("total_params_billion") * 1e9 <= total <= fact("total_params_billion") * 1e9
    per_gb = 1e9 / (per_expert * 2.5 / 8)
    assert abs(per_gb - fact("experts_per_extra_GB")) <= 0.05 * fact("experts_per_extra_GB")


def test_expert_bytes_closed_form():
    h, i = 2048, 768
    n = 3 * h * i
    assert wl.expert_bytes("q4_sym_g32", h, i) == n // 2 + 2 * (n // 32) == 2_654_208
    assert wl.expert_bytes("q2_asym_g32", h, i) == n // 4 + 4 * (n // 32) == 1_769_472


def test_layer_bytes_and_flops_closed_form():
    h, i, e, k = 2048, 768, 512, 10
    # decode: router (fp32 W and bias) + 11 experts + bf16 x + fp32 y
    assert wl.layer_bytes("q4_sym_g32", "bf16", h, i, e, 1, 10) == 4 * e * h + 4 * e + 11 * 2_654_208 + 2 * h + 4 * h
    assert wl.layer_bytes("q4_sym_g32", "bf16", h, i, e, 1, 10) == 33_404_928
    t = 4096
    assert wl.layer_flops(h, i, e, k, t) == 2 * t * e * h + 2 * t * (k + 1) * 3 * h * i
    assert abs(wl.layer_flops(h, i, e, k, t) - 4.338e11) < 1e8
