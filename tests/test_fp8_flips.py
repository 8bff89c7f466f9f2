"""Pins of the fp8 rounding-flip allowance used by the GPU parity tests."""

import numpy as np

import fp8_flips
import oracle
from non_gated_relu_amd.synthetic import f32_to_bf16_bits


def test_midpoints_and_code_steps():
    # e4m3 around 1: codes 1.0, 1.125 (step 2^-3); around 256: 256, 288 (step 32);
    # subnormals step 2^-9; the top interval 416 .. 448
    v = np.array([1.0625, 1.0625 * (1 + 5e-5), 1.0625 * (1 + 5e-4), 1.0, 1.125, 272.0,
                  1.5 * 2.0 ** -9, 432.0, 448.0, 0.0])
    near, step = fp8_flips.near_midpoint(v)
    assert near.tolist() == [True, True, False, False, False, True, True, True, False, False]
    assert step[0] == 0.125 and step[1] == 0.125 and step[5] == 32.0
    assert step[6] == 2.0 ** -9 and step[7] == 32.0


def _one_expert(u_target):
    """Inputs whose oracle pre-activation for token 0 through expert 0 is
    u_target (to fp32 rounding): x = 448 e_0 (quantised per token to code 448
    with scale 1), W_up[i, 0] = code 1.0 times the fp32 scale u_i / 448, and
    W_down = 1 everywhere."""
    I, d = u_target.size, 16
    x = np.zeros((1, d), np.float32)
    x[0, 0] = 448.0
    xq, xs = oracle.quantize_rows(x)
    assert oracle.e4m3_decode(xq)[0, 0] * xs[0] == 448.0
    codes = np.zeros((1, I, d), np.uint8)
    codes[0, :, 0] = 0x38  # e4m3 1.0
    scale = (u_target / 448.0).astype(np.float32)[None]
    wd_codes = np.full((1, d, I), 0x38, np.uint8)
    wd_scale = np.ones((1, d), np.float32)
    return f32_to_bf16_bits(x), codes, scale, wd_codes, wd_scale


def test_no_near_element_gives_zero_allowance():
    # h = u^2 = [3136, 7, 448]: s = 3136 / 448 = 7, h / s ~ [448, 1, 64], all codes
    xb, wu, su, wd, sd = _one_expert(np.sqrt([3136.0, 7.0, 448.0]))
    a = fp8_flips.row_allowance(xb, [0], [0], wu, su, wd, sd)
    assert a.tolist() == [0.0]


def test_one_midpoint_element_allowance_is_step_times_scale():
    # s = 7 and h_1 / s ~ 1.0625, the midpoint of 1 and 1.125 (step 1/8); every
    # W_down entry is 1, so the allowance is 7 / 8
    xb, wu, su, wd, sd = _one_expert(np.sqrt([3136.0, 7.0 * 1.0625, 28.0]))
    a = fp8_flips.row_allowance(xb, [0], [0], wu, su, wd, sd)
    assert a.tolist() == [0.875]
    # s = 28 and h_1 / s ~ 0.53125, the midpoint of 0.5 and 0.5625 (step 1/16):
    # allowance 28 / 16
    xb, wu, su, wd, sd = _one_expert(np.sqrt([12544.0, 28.0 * 0.53125, 28.0]))
    a = fp8_flips.row_allowance(xb, [0], [0], wu, su, wd, sd)
    assert a.tolist() == [1.75]


def test_token_allowance_weights_rows():
    rows = np.array([0.0, 0.5, 2.0])
    w = np.array([[1.0, -2.0], [0.25, 0.5]])
    slot_rows = np.array([[0, 1], [2, 1]])
    assert fp8_flips.token_allowance(rows, w, slot_rows).tolist() == [1.0, 0.75]
