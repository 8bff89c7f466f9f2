"""Pins of the oracle's layer output: textbook MLPs, special cases and invariants."""

import numpy as np
import pytest

import oracle
from bruteforce import relu2_mlp, route_token, sigmoid
from non_gated_relu_amd.synthetic import WORKLOADS, Workload, bf16_bits_to_f32, make_inputs

TINY = WORKLOADS["tiny-f32-T64"]
SMALL_BF16 = Workload("small-bf16", 24, 128, 16, 4, 2, 3, 64, 96, "bf16", "bf16", seed=11)
SMALL_FP8 = Workload("small-fp8", 24, 128, 16, 4, 2, 3, 64, 96, "bf16", "fp8", seed=12)


def _f64(a, dtype):
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, np.float64)


def _weights(wl, inp):
    """Stored weights widened to fp64 (fp8 codes times their row scales)."""
    if wl.expert_dtype == "fp8":
        wu = oracle.e4m3_decode(inp["w_up"]) * inp["w_up_scale"][..., None]
        wd = oracle.e4m3_decode(inp["w_down"]) * inp["w_down_scale"][..., None]
    else:
        wu, wd = _f64(inp["w_up"], wl.expert_dtype), _f64(inp["w_down"], wl.expert_dtype)
    return (wu, wd, _f64(inp["ws_up"], wl.act_dtype), _f64(inp["ws_down"], wl.act_dtype))


def _textbook(wl, inp, hold_h=None, quant_x=None):
    """Per-token layer written from the statement, with numpy and the brute-force router."""
    x = _f64(inp["x"], wl.act_dtype)
    wg = _f64(inp["w_gate"], wl.act_dtype)
    wu, wd, su, sd = _weights(wl, inp)
    logits = x @ wg.T
    xr = quant_x(x) if quant_x else x
    y = np.zeros_like(x)
    for t in range(x.shape[0]):
        ids, w = route_token(logits[t], inp["e_bias"], wl.n_group, wl.topk_group, wl.top_k,
                             wl.routed_scaling_factor, wl.norm_topk_prob)
        for e, we in zip(ids, w):
            u = wu[e] @ xr[t]
            h = np.maximum(u, 0) ** 2
            if hold_h:
                h = hold_h(h)
            y[t] += we * (wd[e] @ h)
        h = np.maximum(su @ x[t], 0) ** 2
        if hold_h and wl.act_dtype == "bf16":
            h = bf16_bits_to_f32(oracle.bf16_round(h)).astype(np.float64)
        elif hold_h:
            h = h.astype(np.float32).astype(np.float64)
        y[t] += sd @ h
    return y


def _rms(a):
    return float(np.sqrt(np.mean(np.asarray(a, np.float64) ** 2)))


def test_tiny_exact_matches_textbook():
    inp = make_inputs(TINY)
    y = oracle.forward(TINY, inp, mode=oracle.EXACT)["y"]
    ref = _textbook(TINY, inp)
    assert np.abs(y - ref).max() <= 1e-12 * _rms(ref)


def test_tiny_as_configured_holds_h_in_fp32():
    inp = make_inputs(TINY)
    y = oracle.forward(TINY, inp)["y"]
    ref = _textbook(TINY, inp, hold_h=lambda h: h.astype(np.float32).astype(np.float64))
    assert np.abs(y - ref).max() <= 1e-12 * _rms(ref)
    exact = oracle.forward(TINY, inp, mode=oracle.EXACT)["y"]
    assert 0 < np.abs(y - exact).max() <= 1e-6 * _rms(ref)


def test_bf16_as_configured_rounds_h_once():
    inp = make_inputs(SMALL_BF16)
    y = oracle.forward(SMALL_BF16, inp)["y"]
    ref = _textbook(SMALL_BF16, inp,
                    hold_h=lambda h: bf16_bits_to_f32(oracle.bf16_round(h)).astype(np.float64))
    assert np.abs(y - ref).max() <= 1e-12 * _rms(ref)
    exact = oracle.forward(SMALL_BF16, inp, mode=oracle.EXACT)["y"]
    np.testing.assert_allclose(exact, _textbook(SMALL_BF16, inp), rtol=0,
                               atol=1e-12 * _rms(ref))
    # rounding h to bf16 moves y by about 2^-9 relative, not more
    d = np.abs(y - exact).max() / _rms(ref)
    assert 1e-5 < d < 2e-2


def test_fp8_as_configured_quantises_x_and_h_per_row():
    inp = make_inputs(SMALL_FP8)

    def qx(x):
        q, s = oracle.quantize_rows(x.astype(np.float32))
        return oracle.e4m3_decode(q) * s[:, None].astype(np.float64)

    def qh(h):
        q, s = oracle.quantize_rows(h.astype(np.float32)[None, :])
        return oracle.e4m3_decode(q[0]) * np.float64(s[0])

    y = oracle.forward(SMALL_FP8, inp)["y"]
    ref = _textbook(SMALL_FP8, inp, hold_h=qh, quant_x=qx)
    assert np.abs(y - ref).max() <= 1e-12 * _rms(ref)
    exact = oracle.forward(SMALL_FP8, inp, mode=oracle.EXACT)["y"]
    assert np.abs(exact - _textbook(SMALL_FP8, inp)).max() <= 1e-12 * _rms(ref)


def test_identical_experts_equal_one_dense_mlp_times_scale():
    wl = SMALL_BF16
    inp = make_inputs(wl)
    inp["w_up"][:] = inp["w_up"][3]
    inp["w_down"][:] = inp["w_down"][3]
    y = oracle.forward(wl, inp, mode=oracle.EXACT)["y"]
    x = _f64(inp["x"], "bf16")
    ref = 2.5 * relu2_mlp(x, _f64(inp["w_up"][0], "bf16"), _f64(inp["w_down"][0], "bf16")) + \
        relu2_mlp(x, _f64(inp["ws_up"], "bf16"), _f64(inp["ws_down"], "bf16"))
    assert np.abs(y - ref).max() <= 1e-12 * _rms(ref)


def test_all_experts_active_is_a_dense_soft_mixture():
    wl = Workload("all-active", 16, 64, 8, 2, 2, 8, 32, 48, "f32", "f32", seed=5)
    inp = make_inputs(wl)
    y = oracle.forward(wl, inp, mode=oracle.EXACT)["y"]
    x = inp["x"].astype(np.float64)
    s = sigmoid(x @ inp["w_gate"].astype(np.float64).T)
    p = s / s.sum(1, keepdims=True)
    ref = relu2_mlp(x, inp["ws_up"], inp["ws_down"])
    for e in range(8):
        ref += 2.5 * p[:, e:e + 1] * relu2_mlp(x, inp["w_up"][e], inp["w_down"][e])
    assert np.abs(y - ref).max() <= 1e-12 * _rms(ref)


def test_zero_routed_down_leaves_the_shared_expert():
    inp = make_inputs(TINY)
    inp["w_down"] = np.zeros_like(inp["w_down"])
    y = oracle.forward(TINY, inp, mode=oracle.EXACT)["y"]
    ref = relu2_mlp(inp["x"], inp["ws_up"], inp["ws_down"])
    assert np.abs(y - ref).max() <= 1e-13 * _rms(ref)


def test_zero_shared_leaves_the_routed_part():
    inp = make_inputs(TINY)
    inp["ws_up"] = np.zeros_like(inp["ws_up"])
    y = oracle.forward(TINY, inp, mode=oracle.EXACT)["y"]
    inp2 = dict(inp)
    ref = _textbook(TINY, inp2)
    assert np.abs(y - ref).max() <= 1e-12 * _rms(ref)


def test_homogeneity_in_the_expert_weights():
    inp = make_inputs(TINY)
    inp["ws_up"] = np.zeros_like(inp["ws_up"])
    base = oracle.forward(TINY, inp)["y"]
    two_down = dict(inp, w_down=inp["w_down"] * np.float32(2))
    np.testing.assert_array_equal(oracle.forward(TINY, two_down)["y"], 2 * base)
    two_up = dict(inp, w_up=inp["w_up"] * np.float32(2))
    np.testing.assert_array_equal(oracle.forward(TINY, two_up)["y"], 4 * base)


def test_token_permutation_equivariance_is_exact():
    inp = make_inputs(SMALL_BF16)
    out = oracle.forward(SMALL_BF16, inp)
    perm = np.random.default_rng(0).permutation(SMALL_BF16.tokens)
    out_p = oracle.forward(SMALL_BF16, dict(inp, x=inp["x"][perm]))
    np.testing.assert_array_equal(out_p["y"], out["y"][perm])
    np.testing.assert_array_equal(out_p["topk_idx"], out["topk_idx"][perm])


def test_token_subset_equals_rows_of_full_run():
    inp = make_inputs(TINY)
    full = oracle.forward(TINY, inp)
    sub = [63, 0, 17, 17]
    part = oracle.forward(TINY, inp, tokens=sub)
    np.testing.assert_array_equal(part["y"], full["y"][sub])
    np.testing.assert_array_equal(part["topk_w"], full["topk_w"][sub])


def test_forward_routing_equals_route():
    inp = make_inputs(SMALL_BF16)
    out = oracle.forward(SMALL_BF16, inp)
    idx, w, _ = oracle.route(SMALL_BF16, inp["x"], inp["w_gate"], inp["e_bias"])
    np.testing.assert_array_equal(out["topk_idx"], idx)
    np.testing.assert_array_equal(out["topk_w"], w)


@pytest.mark.parametrize("wl", [TINY, SMALL_BF16, SMALL_FP8], ids=lambda w: w.name)
def test_ffn_rows_compose_to_the_layer(wl):
    inp = make_inputs(wl)
    out = oracle.forward(wl, inp)
    T, k = wl.tokens, wl.top_k
    rows = np.repeat(np.arange(T), k)
    o = oracle.ffn_rows(inp["x"], wl.act_dtype, rows, out["topk_idx"].reshape(-1), inp["w_up"],
                        inp["w_down"], wl.expert_dtype, inp["w_up_scale"], inp["w_down_scale"],
                        quant_a=wl.expert_dtype == "fp8")
    sh = oracle.ffn_rows(inp["x"], wl.act_dtype, np.arange(T), np.zeros(T), inp["ws_up"][None],
                         inp["ws_down"][None], wl.act_dtype)
    y = (out["topk_w"][..., None] * o.reshape(T, k, -1)).sum(1) + sh
    assert np.abs(y - out["y"]).max() <= 1e-12 * _rms(out["y"])


def test_permute_definition_matches_loops():
    rng = np.random.default_rng(4)
    idx = np.sort(rng.choice(16, size=(40, 3)), axis=1)
    counts, offsets, sorted_slot, slot_pos = oracle.permute(idx, 16)
    flat = idx.reshape(-1)
    ref = [s for e in range(16) for s in range(flat.size) if flat[s] == e]
    np.testing.assert_array_equal(sorted_slot, ref)
    for e in range(16):
        assert counts[e] == (flat == e).sum()
        assert offsets[e + 1] - offsets[e] == counts[e]
    for s in range(flat.size):
        assert sorted_slot[slot_pos[s]] == s
    assert offsets[0] == 0 and offsets[-1] == flat.size


def test_combine_definition_matches_loops():
    rng = np.random.default_rng(6)
    T, k, d = 5, 3, 7
    w = rng.random((T, k))
    yp = rng.standard_normal((T * k, d))
    pos = rng.permutation(T * k)
    sh = rng.standard_normal((T, d))
    got = oracle.combine(w, yp, pos, sh)
    for t in range(T):
        ref = sh[t].copy()
        for j in range(k):
            ref += w[t, j] * yp[pos[t * k + j]]
        np.testing.assert_allclose(got[t], ref, rtol=1e-14, atol=1e-14)
