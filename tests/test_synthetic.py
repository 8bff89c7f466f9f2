"""The seeded input generator: determinism, layout and storage formats."""

import json
import os

import numpy as np
import torch

from non_gated_relu_amd import synthetic
from non_gated_relu_amd.synthetic import WORKLOADS, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nemotron_h_moe_shapes.json")


def test_deterministic_and_prefix_of_larger_T():
    wl = WORKLOADS["tiny-f32-T64"]
    a = make_inputs(wl)
    b = make_inputs(wl)
    for k in a:
        if a[k] is not None:
            np.testing.assert_array_equal(a[k], b[k])
    c = make_inputs(wl.with_tokens(100), experts=False)
    np.testing.assert_array_equal(c["x"][:64], a["x"])
    np.testing.assert_array_equal(c["w_gate"], a["w_gate"])


def test_distributions():
    wl = WORKLOADS["tiny-f32-T64"]
    a = make_inputs(wl)
    assert abs(a["x"].std() - 1.0) < 0.02
    assert abs(a["w_up"].std() - 0.02) < 0.001
    assert abs(a["e_bias"].std() - 0.01) < 0.005
    assert a["e_bias"].dtype == np.float32
    assert a["w_up"].shape == (16, 128, 256) and a["w_down"].shape == (16, 256, 128)
    assert a["ws_up"].shape == (256, 256) and a["ws_down"].shape == (256, 256)


def test_bf16_storage_matches_torch_rounding():
    v = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synthetic.f32_to_bf16_bits(v), ref)


def test_generator_e4m3_matches_torch():
    v = (np.random.default_rng(1).standard_normal(20000) * 100).astype(np.float32)
    v = v[np.abs(v) <= 448]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ref = np.where(ref == 0x80, 0, ref)
    np.testing.assert_array_equal(synthetic._e4m3_codes(v), ref)


def test_skew_bias_boost():
    base = make_inputs(WORKLOADS["prefill-bf16-T4096"].with_tokens(4), experts=False)
    sk = make_inputs(WORKLOADS["skew-bf16-T16384"].with_tokens(4), experts=False)
    diff = sk["e_bias"] - base["e_bias"]
    boosted = np.flatnonzero(diff)
    assert list(boosted) == [0, 4, 8, 12, 64, 68, 72, 76]
    np.testing.assert_allclose(diff[boosted], 2.0, atol=1e-6)


def test_full_size_workloads_follow_the_pages():
    g = json.load(open(GOLDEN))
    for name in ("decode-bf16-T32", "prefill-bf16-T4096", "skew-bf16-T16384", "fp8-T8192"):
        wl = WORKLOADS[name]
        assert (wl.hidden, wl.inter, wl.n_experts, wl.top_k) == \
            (g["hidden"], g["inter"], g["n_experts"], g["top_k"])
        assert (wl.n_group, wl.topk_group, wl.shared_inter) == \
            (g["n_group"], g["topk_group"], g["shared_inter"])
        assert wl.routed_scaling_factor == g["routed_scaling_factor"]
        assert wl.norm_topk_prob == g["norm_topk_prob"]
    assert g["model_card_hidden"] == g["hidden"]
    # per MoE block: one up and one down linear per routed expert plus the shared pair
    assert 2 * g["n_experts"] + 2 == g["linears_per_moe_block"]
    # the MoE parameters of all MoE layers fit inside the bf16 checkpoint
    d, I, E, Is = g["hidden"], g["inter"], g["n_experts"], g["shared_inter"]
    per_layer = E * 2 * d * I + 2 * d * Is + E * d + E
    assert g["moe_layers"] * per_layer * 2 <= g["model_bf16_bytes"]
    assert g["moe_layers"] * per_layer * 2 > 0.9 * g["model_bf16_bytes"]
