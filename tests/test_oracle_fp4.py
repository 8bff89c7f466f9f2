"""Pins of the oracle's 4-bit expert weights: OCP e2m1 codes, E8M0 block
scales, and the fp4 expert FFN, which must equal the bf16 expert FFN on the
same weights written out in bf16 (every e2m1 code times a power of two is a
bf16 value, so the two are the same mathematics on the same numbers)."""

import dataclasses

import numpy as np
import pytest

import oracle
from non_gated_relu_amd import synthetic
from non_gated_relu_amd.synthetic import bf16_bits_to_f32, f32_to_bf16_bits


def _ocp_e2m1_value(code):
    # 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is subnormal
    s, E, M = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = M * 0.5 if E == 0 else (1 + M / 2) * 2.0 ** (E - 1)
    return -mag if s else mag


def test_e2m1_decode_all_codes():
    codes = np.arange(16, dtype=np.uint8)
    got = oracle.e2m1_decode(codes)
    np.testing.assert_array_equal(got, [_ocp_e2m1_value(int(c)) for c in codes])
    np.testing.assert_array_equal(got[:8], [0, 0.5, 1, 1.5, 2, 3, 4, 6])
    # only the low nibble is a code
    np.testing.assert_array_equal(oracle.e2m1_decode(codes | 0xA0), got)


def test_e8m0_decode():
    got = oracle.e8m0_decode(np.array([0, 1, 126, 127, 128, 254, 255], np.uint8))
    np.testing.assert_array_equal(got[:6], [2.0 ** -127, 2.0 ** -126, 0.5, 1.0, 2.0, 2.0 ** 127])
    assert np.isnan(got[6])


def _dequant(packed, bscale):
    """[.., rows, cols/2] codes (low nibble = even column) and [.., rows, cols/32]
    scales -> fp64 [.., rows, cols], written out independently of the oracle."""
    lut = np.array([_ocp_e2m1_value(c) for c in range(16)])
    lo, hi = lut[packed & 15], lut[packed >> 4]
    v = np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)
    s = np.ldexp(1.0, bscale.astype(np.int64) - 127)
    return v * np.repeat(s, 32, axis=-1)


def test_generator_mxfp4_scale_and_rounding():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((8, 128)) * 0.02).astype(np.float32)
    w[1, :32] = 0.0                                   # an all-zero block
    w[2, 32:64] = np.float32(6.0 * 2.0 ** -7)         # amax exactly on code 6
    w[3, :32] = 0.0
    w[3, 0], w[3, 1], w[3, 2] = 2.0 ** -4, 1.25 * 2.0 ** -6, 1.75 * 2.0 ** -6  # ties
    packed, bs = synthetic.quantize_weight_rows_mxfp4(w)
    assert packed.shape == (8, 64) and bs.shape == (8, 4)
    deq = _dequant(packed, bs)
    b = w.reshape(8, 4, 32).astype(np.float64)
    amax = np.abs(b).max(-1)
    X = bs.astype(np.int64) - 127
    nz = amax > 0
    # scale: 2^(floor(log2 amax) - 2), the largest e2m1 exponent being 2
    np.testing.assert_array_equal(X[nz], np.floor(np.log2(amax[nz])).astype(np.int64) - 2)
    assert bs[1, 0] == 0 and (deq[1, :32] == 0).all()
    assert deq[2, 32] == 6.0 * 2.0 ** -7
    # ties go to the even code: 1.25 -> 1, 1.75 -> 2 (block scale 2^-6)
    assert X[3, 0] == -6
    np.testing.assert_array_equal(deq[3, :3], [2.0 ** -4, 2.0 ** -6, 2.0 ** -5])
    # every element is the nearest grid value, or 6 * 2^X where it exceeds it
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    scaled = np.abs(b / np.ldexp(1.0, X)[..., None]).reshape(8, 128)
    err = np.abs(np.abs(deq) / np.repeat(np.ldexp(1.0, X), 32, -1) - scaled)
    best = np.abs(scaled[..., None] - grid).min(-1)
    np.testing.assert_allclose(err, best, rtol=0, atol=1e-12)
    assert (np.sign(deq) * np.sign(w) >= 0).all()


def _fp4_case(seed, rows_n=24, d=64, inter=96, E=3):
    rng = np.random.default_rng(seed)
    x = f32_to_bf16_bits(rng.standard_normal((rows_n, d)).astype(np.float32))
    up = (rng.standard_normal((E, inter, d)) * 0.05).astype(np.float32)
    dn = (rng.standard_normal((E, d, inter)) * 0.05).astype(np.float32)
    qu = [synthetic.quantize_weight_rows_mxfp4(u) for u in up]
    qd = [synthetic.quantize_weight_rows_mxfp4(u) for u in dn]
    wu, su = np.stack([q[0] for q in qu]), np.stack([q[1] for q in qu])
    wd, sd = np.stack([q[0] for q in qd]), np.stack([q[1] for q in qd])
    rows = rng.integers(0, rows_n, 40).astype(np.int32)
    mats = rng.integers(0, E, 40).astype(np.int32)
    return x, rows, mats, wu, su, wd, sd


def test_fp4_ffn_equals_bf16_ffn_on_the_dequantised_weights():
    x, rows, mats, wu, su, wd, sd = _fp4_case(4)
    got = oracle.ffn_rows(x, "bf16", rows, mats, wu, wd, "fp4", w_up_bscale=su,
                          w_down_bscale=sd)
    wu16 = f32_to_bf16_bits(_dequant(wu, su).astype(np.float32))
    wd16 = f32_to_bf16_bits(_dequant(wd, sd).astype(np.float32))
    assert (bf16_bits_to_f32(wu16) == _dequant(wu, su)).all()   # exact in bf16
    ref = oracle.ffn_rows(x, "bf16", rows, mats, wu16, wd16, "bf16")
    np.testing.assert_array_equal(got, ref)


def test_fp4_ffn_brute_force_one_row():
    x, rows, mats, wu, su, wd, sd = _fp4_case(5)
    got = oracle.ffn_rows(x, "bf16", rows[:1], mats[:1], wu, wd, "fp4", w_up_bscale=su,
                          w_down_bscale=sd)
    a = bf16_bits_to_f32(x[rows[0]]).astype(np.float64)
    u = _dequant(wu[mats[0]], su[mats[0]]) @ a
    h = np.maximum(u, 0.0) ** 2
    h = bf16_bits_to_f32(f32_to_bf16_bits(h.astype(np.float32))).astype(np.float64)
    ref = _dequant(wd[mats[0]], sd[mats[0]]) @ h
    np.testing.assert_allclose(got[0], ref, rtol=1e-5, atol=1e-6 * np.abs(ref).max())


@pytest.mark.parametrize("shared", ["bf16", "fp4"])
def test_fp4_forward_equals_bf16_forward_on_the_dequantised_weights(shared):
    wl = synthetic.Workload("fp4-tiny", 40, hidden=64, n_experts=16, n_group=4,
                            topk_group=1, top_k=2, inter=96, shared_inter=64,
                            act_dtype="bf16", expert_dtype="fp4", seed=11, shared_dtype=shared)
    inp = synthetic.make_inputs(wl)
    got = oracle.forward(wl, inp)
    ref_inp = dict(inp)
    names = [("w_up", "w_up_bscale"), ("w_down", "w_down_bscale")]
    if shared == "fp4":
        names += [("ws_up", "ws_up_bscale"), ("ws_down", "ws_down_bscale")]
    for w, b in names:
        ref_inp[w] = f32_to_bf16_bits(_dequant(inp[w], inp[b]).astype(np.float32))
        ref_inp[b] = None
    ref = oracle.forward(dataclasses.replace(wl, expert_dtype="bf16", shared_dtype=None), ref_inp)
    np.testing.assert_array_equal(got["topk_idx"], ref["topk_idx"])
    np.testing.assert_array_equal(got["y"], ref["y"])
    # the shared expert matters: dropping it changes y
    if shared == "fp4":
        ref_inp["ws_down"] = np.zeros_like(ref_inp["ws_down"])
        assert not np.array_equal(oracle.forward(dataclasses.replace(
            wl, expert_dtype="bf16", shared_dtype=None), ref_inp)["y"], got["y"])
