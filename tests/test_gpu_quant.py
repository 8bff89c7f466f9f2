"""GPU parity of the fp8 path's per-row quantiser (moe_quantize_rows) with the
oracle's: the e4m3 codes and the fp32 scales, bit for bit.  Both sides divide
in fp32 and round the same quotient, so every code must agree."""

import numpy as np
import pytest
import torch

import oracle
from non_gated_relu_amd import binding
from non_gated_relu_amd.synthetic import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    binding.lib()


def _run(v32, bf16):
    """Quantise fp32 rows v32 on the GPU, as bf16 rows when ``bf16`` (v32 must
    then hold bf16 values), and compare with the oracle."""
    if bf16:
        bits = f32_to_bf16_bits(v32)
        assert np.array_equal(bf16_bits_to_f32(bits), v32)
        x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        x = torch.from_numpy(np.ascontiguousarray(v32)).cuda()
    q, s = binding.quantize_rows(x)
    torch.cuda.synchronize()
    ref_q, ref_s = oracle.quantize_rows(v32)
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))
    got = q.cpu().numpy()
    bad = np.argwhere(got != ref_q)
    assert bad.size == 0, [(tuple(i), float(v32[tuple(i)]), int(got[tuple(i)]),
                            int(ref_q[tuple(i)])) for i in bad[:8]]


@pytest.mark.parametrize("bf16", [True, False], ids=["bf16", "f32"])
@pytest.mark.parametrize("cols", [64, 1856, 2688, 3712, 8192])
def test_random_rows_match_the_oracle(cols, bf16):
    # 77 rows (not a multiple of the 4 rows per workgroup) of normal values at
    # magnitudes from 1e-30 to 1e30; rows past 3072 columns take the two-pass path
    rng = np.random.default_rng(cols + 7 * bf16)
    v = rng.standard_normal((77, cols)) * 10.0 ** rng.uniform(-30, 30, (77, 1))
    v = v.astype(np.float32)
    if bf16:
        v = bf16_bits_to_f32(f32_to_bf16_bits(v))
    v[5] = 0.0  # an all-zero row: scale 1, codes 0
    _run(v, bf16)


def _e4m3_grid():
    mags = oracle.e4m3_decode(np.arange(128, dtype=np.uint8))
    return np.unique(mags[np.isfinite(mags)]).astype(np.float64)  # 0 .. 448


def test_rounding_at_every_midpoint_with_unit_scale():
    # amax = 448 makes the scale exactly 1, so each quotient is the value
    # itself: every representable magnitude, every midpoint between
    # neighbours (ties to even), one fp32 ulp either side of each midpoint,
    # both signs, and magnitudes that round to zero (a +0 code)
    g = _e4m3_grid()
    mid = (g[:-1] + g[1:]) / 2
    vals = [g, mid, np.nextafter(mid.astype(np.float32), np.float32(0)),
            np.nextafter(mid.astype(np.float32), np.float32(np.inf)),
            np.array([2.0 ** -11, 2.0 ** -10 * 0.99, 1e-30, 0.0])]
    v = np.concatenate([np.asarray(a, np.float64) for a in vals]).astype(np.float32)
    v = np.concatenate([v, -v])
    pad = (-(v.size + 1)) % 64
    row = np.concatenate([[448.0], v, np.zeros(pad)]).astype(np.float32)
    _run(row[None, :], False)
    # the same in bf16 rows, where every such value is a bf16 value too
    keep = bf16_bits_to_f32(f32_to_bf16_bits(row)) == row
    rb = np.where(keep, row, 0.0).astype(np.float32)
    _run(rb[None, :], True)


def test_saturation_when_the_scale_is_subnormal():
    # v_k = k * 2^-149 (fp32 subnormals) for k = 0..627: amax / 448 = 1.3996 *
    # 2^-149 rounds to the scale 2^-149, so the quotients are k themselves and
    # those above 448 saturate to the largest code
    k = np.arange(640, dtype=np.float64)
    k[628:] = 0
    row = (k * 2.0 ** -149).astype(np.float32)
    assert np.array_equal(row.astype(np.float64) / 2.0 ** -149, k)
    v = np.stack([row, -row])
    _run(v, False)
    q, s = oracle.quantize_rows(v)
    assert s[0] == np.float32(2.0 ** -149)
    assert np.all(q[0, 464:628] == 0x7E) and np.all(q[1, 464:628] == 0xFE)
