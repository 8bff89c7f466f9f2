"""GPU parity at the full Nemotron-H sizes, in the launch configuration the
benchmark times (one moe_forward per step): routing and per-expert counts for
every token, the layer output on 1024 tokens the oracle computes one by one,
and the routed expert MLP rows of moe_expert_ffn on at least 4096 rows per
workload (the first rows, both ends of every active expert's rows, the last
partial 256-row tile of every expert, and seeded random rows)."""

import numpy as np
import pytest
import torch

import oracle
import fp8_flips
from gpu_util import assert_close_rms, assert_routing_equal, to_f64, upload
from non_gated_relu_amd import binding
from non_gated_relu_amd.synthetic import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

_cache = {}


def _inputs(name):
    """Full-size inputs; prefill and skew share every weight (same seeds)."""
    if name in _cache:
        return _cache[name]
    wl = WORKLOADS[name]
    if name in ("prefill-bf16-T4096", "skew-bf16-T16384"):
        if "bf16-weights" not in _cache:
            _cache["bf16-weights"] = make_inputs(WORKLOADS["skew-bf16-T16384"])
        base = _cache["bf16-weights"]
        inp = dict(base)
        if name == "prefill-bf16-T4096":
            small = make_inputs(wl, experts=False)
            inp["x"], inp["e_bias"] = small["x"], small["e_bias"]
            assert np.array_equal(small["x"], base["x"][:wl.tokens])
    else:
        inp = make_inputs(wl)
    _cache[name] = inp
    return inp


TOKENS_CHECKED = 1024
ROWS_CHECKED = 4096


def _sample(T, n=TOKENS_CHECKED, seed=0):
    """n distinct tokens: the first 3n/4, seeded random ones, and the last."""
    rng = np.random.default_rng(seed)
    first = np.arange(min(3 * n // 4, T))
    rest = np.setdiff1d(np.arange(T), np.append(first, T - 1))
    extra = rng.choice(rest, size=min(n - first.size - 1, rest.size), replace=False)
    return np.unique(np.concatenate([first, extra, [T - 1]]))


def _row_sample(offsets, n=ROWS_CHECKED, tile=256, seed=1):
    """Sorted routed-row positions to check: the first 512, the first two and
    last two rows of every active expert, up to 16 rows of every expert's last
    (partial) tile of `tile` rows, then seeded random rows up to n."""
    S = int(offsets[-1])
    pick = [np.arange(min(512, S))]
    for e in range(offsets.size - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi <= lo:
            continue
        pick.append(np.array([lo, min(lo + 1, hi - 1), max(hi - 2, lo), hi - 1]))
        last = lo + (hi - lo - 1) // tile * tile  # first row of the last tile
        pick.append(np.linspace(last, hi - 1, num=min(16, hi - last)).astype(np.int64))
    rows = np.unique(np.concatenate(pick))
    rng = np.random.default_rng(seed)
    rest = np.setdiff1d(np.arange(S), rows)
    extra = rng.choice(rest, size=min(max(n - rows.size, 0), rest.size), replace=False)
    return np.unique(np.concatenate([rows, extra]))


@pytest.mark.parametrize("name", ["prefill-bf16-T4096", "skew-bf16-T16384", "fp8-T8192"])
def test_full_size_layer(name):
    print(f"case {name}", flush=True)
    wl = WORKLOADS[name]
    inp = _inputs(name)
    layer = binding.MoELayer(wl, inp)
    x = binding.to_device(inp["x"], "cuda", "x", wl)
    y = layer(x)
    torch.cuda.synchronize()
    # routing of every token, and the per-expert counts
    idx, w, margin = oracle.route(wl, inp["x"], inp["w_gate"], inp["e_bias"])
    assert_routing_equal(layer.topk_idx, layer.topk_w, idx, w, margin, name)
    counts = np.bincount(idx.reshape(-1), minlength=wl.n_experts)
    np.testing.assert_array_equal(layer.expert_counts.cpu().numpy(), counts)
    if name.startswith("skew"):
        frac = counts[list(wl.bias_boost)].sum() / counts.sum()
        print(f"{name}: {frac:.4f} of slots on the boosted experts, "
              f"{(counts == 0).sum()} experts empty, max count {counts.max()}", flush=True)
    # output rows of a token sample
    tok = _sample(wl.tokens)
    ref = oracle.forward(wl, inp, tokens=tok)
    allow = None
    if wl.expert_dtype == "fp8":
        rows = np.repeat(tok, wl.top_k)
        allow = fp8_flips.token_allowance(
            fp8_flips.row_allowance(inp["x"], rows, idx[tok].reshape(-1), inp["w_up"],
                                    inp["w_up_scale"], inp["w_down"], inp["w_down_scale"]),
            w[tok], np.arange(rows.size).reshape(tok.size, wl.top_k))
    assert_close_rms(to_f64(y[torch.from_numpy(tok).cuda()]), ref["y"], f"{name} layer",
                     row_allow=allow)
    # a second call gives the same bits
    y2 = layer(x)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    # Every output row: tokens are independent, routing does not depend on the
    # batch, and a row's result does not depend on the tile shape, so the
    # layer over T/8-token chunks (smaller tiles, other router path) must
    # reproduce all T rows bit for bit.
    chunk = wl.tokens // 8
    parts = [layer(x[i:i + chunk]).clone() for i in range(0, wl.tokens, chunk)]
    torch.cuda.synchronize()
    yc = torch.cat(parts)
    bad = (yc.view(torch.int16) != y.view(torch.int16)).any(dim=1).nonzero().flatten()
    assert bad.numel() == 0, f"{name}: {bad.numel()} rows differ from the chunked run, " \
                             f"first {bad[:8].tolist()}"


@pytest.mark.parametrize("name", ["prefill-bf16-T4096", "skew-bf16-T16384", "fp8-T8192"])
def test_full_size_expert_rows(name):
    """moe_expert_ffn over all routed rows of the workload (the routed problem
    moe_forward runs, in its tile shape) against the oracle's per-row expert
    MLP on at least ROWS_CHECKED rows."""
    print(f"case {name} expert rows", flush=True)
    wl = WORKLOADS[name]
    inp = _inputs(name)
    t = upload({k: v for k, v in inp.items() if k != "norm_w"}, wl)
    cfg = binding.config_from(wl)
    idx, _, _ = oracle.route(wl, inp["x"], inp["w_gate"], inp["e_bias"])
    counts, offsets, sorted_slot, _ = oracle.permute(idx, wl.n_experts)
    k = wl.top_k
    off_d = torch.from_numpy(offsets).cuda()
    ss_d = torch.from_numpy(sorted_slot).cuda()
    S = int(offsets[-1])
    y_perm = binding.expert_ffn(cfg, t["w_up"], t["w_down"], t["x"], off_d, S, row_index=ss_d,
                                index_div=k, w_dtype=wl.expert_dtype,
                                w_up_scale=t.get("w_up_scale"), w_down_scale=t.get("w_down_scale"))
    torch.cuda.synchronize()
    pos = _row_sample(offsets)
    assert pos.size >= ROWS_CHECKED
    rows = sorted_slot[pos] // k
    mats = np.repeat(np.arange(wl.n_experts), counts)[pos]
    active = np.flatnonzero(counts)
    assert np.isin(active, mats).all(), "every active expert is checked"
    ref = oracle.ffn_rows(inp["x"], wl.act_dtype, rows, mats, inp["w_up"], inp["w_down"],
                          wl.expert_dtype, inp.get("w_up_scale"), inp.get("w_down_scale"),
                          quant_a=wl.expert_dtype == "fp8")
    allow = None
    if wl.expert_dtype == "fp8":
        allow = fp8_flips.row_allowance(inp["x"], rows, mats, inp["w_up"], inp["w_up_scale"],
                                        inp["w_down"], inp["w_down_scale"])
    got = to_f64(y_perm[torch.from_numpy(pos).cuda()])
    print(f"{name}: {pos.size} routed rows over {active.size} experts", flush=True)
    assert_close_rms(got, ref, f"{name} expert rows", row_allow=allow)
