"""Pins of the oracle's number formats: bf16 rounding, OCP e4m3, the per-row quantiser."""

import numpy as np
import pytest
import torch

import oracle
from non_gated_relu_amd import synthetic


def test_bf16_round_matches_torch_on_fp32_values():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-40]]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_round(v.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_bf16_round_is_one_rounding_from_fp64():
    # 1 + 2^-8 is the midpoint between bf16 neighbours 1 and 1 + 2^-7; a value a hair
    # above it must round up, although rounding first to fp32 would land on the
    # midpoint and then tie to the even neighbour 1.0.
    v = np.array([1 + 2.0 ** -8 + 2.0 ** -30, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8,
                  -(1 + 2.0 ** -8 + 2.0 ** -30)])
    got = synthetic.bf16_bits_to_f32(oracle.bf16_round(v)).astype(np.float64)
    np.testing.assert_array_equal(got, [1 + 2.0 ** -7, 1.0, 1 + 2 * 2.0 ** -7,
                                        -(1 + 2.0 ** -7)])


def _ocp_e4m3_value(code):
    s, E, M = code >> 7, (code >> 3) & 15, code & 7
    if E == 15 and M == 7:
        return np.nan
    mag = M * 2.0 ** -9 if E == 0 else (1 + M / 8) * 2.0 ** (E - 7)
    return -mag if s else mag


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_decode(codes)
    ref = np.array([_ocp_e4m3_value(int(c)) for c in codes])
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def test_e4m3_round_trip_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)], np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    np.testing.assert_array_equal(oracle.e4m3_encode(vals), codes)
    assert oracle.e4m3_encode(np.float32(-0.0)) == 0


def test_e4m3_ties_to_even_and_saturates():
    v = np.array([1.0625, 1.1875, -1.0625, 2.0 ** -10, 3 * 2.0 ** -10, 464.0, 500.0, -1e9,
                  447.9, 2.0 ** -6 * 1.0625], np.float32)
    got = oracle.e4m3_decode(oracle.e4m3_encode(v))
    np.testing.assert_array_equal(got, [1.0, 1.25, -1.0, 0.0, 2.0 ** -8, 448.0, 448.0, -448.0,
                                        448.0, 2.0 ** -6])


def test_e4m3_matches_torch_within_range():
    rng = np.random.default_rng(1)
    v = (rng.standard_normal(50000) * 10.0 ** rng.uniform(-4, 2.5, 50000)).astype(np.float32)
    v = v[np.abs(v) <= 448.0]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode(v)
    # torch writes -0 for tiny negatives; the oracle writes +0
    ref = np.where(ref == 0x80, 0, ref)
    np.testing.assert_array_equal(got, ref)


def test_generator_weight_codes_agree_with_oracle_codec():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((64, 300)) * 0.02).astype(np.float32)
    q, s = synthetic.quantize_weight_rows_e4m3(w)
    q2, s2 = oracle.quantize_rows(w)
    np.testing.assert_array_equal(s, s2)
    np.testing.assert_array_equal(q, q2)


def test_quantize_rows_scale_and_extremes():
    v = np.array([[0.5, -2.0, 1.0, 0.0], [0, 0, 0, 0], [3e-3, 1e-3, -2e-3, 5e-4]], np.float32)
    q, s = oracle.quantize_rows(v)
    assert s[0] == np.float32(2.0) / np.float32(448.0)
    assert s[1] == 1.0 and (q[1] == 0).all()
    deq = oracle.e4m3_decode(q) * s[:, None].astype(np.float64)
    assert deq[0, 1] == pytest.approx(-2.0, rel=1e-6)        # amax lands on 448 * s
    assert oracle.e4m3_decode(q[0, 1:2])[0] == -448.0
    # each value is within half an e4m3 step (relative 2^-4) of the input
    rel = np.abs(deq - v) / np.maximum(np.abs(v), 1e-30)
    assert rel[v != 0].max() <= 2.0 ** -4 + 1e-7
