"""Pins of the oracle's block around the layer: the pre-mixer RMSNorm and the
residual add, block(x) = x + MoE(RMSNorm(x))."""

import numpy as np
import pytest
import torch

import oracle
from non_gated_relu_amd import synthetic
from non_gated_relu_amd.synthetic import bf16_bits_to_f32, f32_to_bf16_bits


def _rows(seed, T=6, d=256):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((T, d)) * 10.0 ** rng.uniform(-2, 2, (T, 1))).astype(np.float32)
    g = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    return x, g


def test_constant_row_closed_form():
    # every x_i = c, g = 1: n_i = c / sqrt(c^2 + eps), within one rounding of each fp32 step
    d, eps = 128, 1e-5
    for c in (0.5, -3.0, 0.01, 7.25):
        x = np.full((1, d), c, np.float32)
        n = oracle.rmsnorm(x, np.ones(d, np.float32), eps, "f32")
        exact = c / np.sqrt(c * c + eps)
        assert np.all(np.abs(n - exact) <= 4 * np.finfo(np.float32).eps * abs(exact))
        assert np.all(n == n[0, 0])


def test_unit_rms_and_weight_scale():
    # eps = 0, g = 1: the output rows have mean square 1; doubling g doubles n exactly
    x, g = _rows(1)
    n = oracle.rmsnorm(x, np.ones_like(g), 0.0, "f32").astype(np.float64)
    np.testing.assert_allclose((n ** 2).mean(axis=1), 1.0, rtol=1e-6)
    n1 = oracle.rmsnorm(x, g, 1e-5, "f32")
    n2 = oracle.rmsnorm(x, 2 * g, 1e-5, "f32")
    np.testing.assert_array_equal(n2, 2 * n1)


def test_power_of_two_scale_invariance_is_exact():
    # eps = 0: scaling a row by 2^k scales ss by 4^k and r by 2^-k exactly
    x, g = _rows(2)
    xb = f32_to_bf16_bits(x)
    gb = f32_to_bf16_bits(g)
    n = oracle.rmsnorm(xb, gb, 0.0, "bf16")
    for k in (-3, 5):
        xs = f32_to_bf16_bits(bf16_bits_to_f32(xb) * np.float32(2.0 ** k))
        np.testing.assert_array_equal(oracle.rmsnorm(xs, gb, 0.0, "bf16"), n)


def test_matches_torch_rms_norm_within_one_bf16_step():
    x, g = _rows(3, T=16, d=2688)
    xb, gb = f32_to_bf16_bits(x), f32_to_bf16_bits(g)
    got = bf16_bits_to_f32(oracle.rmsnorm(xb, gb, 1e-5, "bf16")).astype(np.float64)
    ref = torch.nn.functional.rms_norm(
        torch.from_numpy(bf16_bits_to_f32(xb).astype(np.float64)), (2688,),
        weight=torch.from_numpy(bf16_bits_to_f32(gb).astype(np.float64)), eps=1e-5).numpy()
    # one bf16 rounding of a value carrying a few fp32 roundings: within one step (2^-7 relative)
    assert np.all(np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-30)
    # and mostly the very value torch's result rounds to
    same = got == bf16_bits_to_f32(f32_to_bf16_bits(ref.astype(np.float32)))
    assert same.mean() > 0.99


def test_block_with_no_expert_output_is_the_residual():
    # zero W_down and zero shared W_down: the mixer adds nothing, block(x) = x exactly
    wl = synthetic.Workload("blk-tiny", 24, 128, 16, 4, 2, 2, 64, 64, "bf16", "bf16", seed=5)
    inp = synthetic.make_inputs(wl)
    inp["w_down"] = np.zeros_like(inp["w_down"])
    inp["ws_down"] = np.zeros_like(inp["ws_down"])
    out = oracle.block_forward(wl, inp)
    np.testing.assert_array_equal(out["y"], bf16_bits_to_f32(inp["x"]).astype(np.float64))


@pytest.mark.parametrize("name", ["tiny-f32-T64", "decode-bf16-T32"])
def test_block_routes_on_the_normalised_rows(name):
    # the block's routing is the layer's routing of x_norm, and y - x is the layer's output
    wl = synthetic.WORKLOADS[name].with_tokens(8)
    inp = synthetic.make_inputs(wl)
    out = oracle.block_forward(wl, inp)
    xn = oracle.rmsnorm(inp["x"], inp["norm_w"], wl.norm_eps, wl.act_dtype)
    lay = oracle.forward(wl, dict(inp, x=xn))
    np.testing.assert_array_equal(out["topk_idx"], lay["topk_idx"])
    x = inp["x"] if wl.act_dtype == "f32" else bf16_bits_to_f32(inp["x"])
    np.testing.assert_array_equal(out["y"], np.asarray(x, np.float64) + lay["y"])
