"""GPU parity: every libmoe entry point against the fp64 oracle, at sizes the
oracle finishes in seconds (several tiles, ragged tails, edge cases)."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import fp8_flips
from gpu_util import (assert_close_rms, assert_routing_equal, rms, to_f64, upload)
from non_gated_relu_amd import binding
from non_gated_relu_amd.synthetic import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

# Ragged shapes: T not a multiple of 16, I and Is leaving partial 128-wide N tiles.
RAGGED_BF16 = Workload("ragged-bf16-T77", 77, 256, 32, 4, 2, 4, 192, 320, "bf16", "bf16", seed=21)
RAGGED_FP8 = Workload("ragged-fp8-T77", 77, 256, 32, 4, 2, 4, 192, 320, "bf16", "fp8", seed=22)
PLAIN_TOPK = Workload("one-group-T40", 40, 128, 16, 1, 1, 5, 64, 128, "bf16", "bf16", seed=23)
ALL_GROUPS = Workload("all-groups-T33", 33, 128, 64, 8, 8, 8, 128, 64, "bf16", "bf16", seed=24)
WHOLE_GROUP = Workload("k-fills-group-T50", 50, 128, 32, 4, 1, 8, 64, 0, "bf16", "bf16", seed=25)
BIG_ROWS = Workload("many-rows-T600", 600, 128, 16, 2, 1, 2, 128, 128, "bf16", "bf16", seed=26)
SINGLE = dataclasses.replace(WORKLOADS["decode-bf16-T32"], name="decode-bf16-T1", tokens=1)
# a few tokens: selection and permute share one launch in moe_forward (one
# token per wave of its 16; at 16 tokens every wave selects)
FEW_FP4 = dataclasses.replace(WORKLOADS["decode-fp4-T32"], name="decode-fp4-T3", tokens=3)
FUSED_SELECT_16 = dataclasses.replace(WORKLOADS["decode-bf16-T32"], name="decode-bf16-T16",
                                      tokens=16)
# Hundreds of rows per expert: the 256 x 256 tile kernels (I = 320 leaves a
# partial N tile; d = 64 gives a K loop shorter than the DMA ring).
BIG_GROUPS_BF16 = Workload("big-groups-bf16-T1024", 1024, 256, 16, 4, 1, 2, 320, 192, "bf16",
                           "bf16", seed=27)
BIG_GROUPS_FP8 = Workload("big-groups-fp8-T1024", 1024, 256, 16, 4, 1, 2, 320, 192, "bf16", "fp8",
                          seed=28)
SHORT_K = Workload("big-groups-bf16-d64", 1024, 64, 16, 4, 1, 2, 128, 64, "bf16", "bf16", seed=29)
# fp8 K loops with 6 to 9 ring stages (K = 384 .. 576 bytes): the first
# lengths where main steps (all fetches inside K) run before the last steps,
# with an even and an odd stage count in each projection
RING_FP8_K7 = Workload("big-groups-fp8-d448", 1024, 448, 16, 4, 1, 2, 384, 0, "bf16", "fp8",
                       seed=35)
RING_FP8_K9 = Workload("big-groups-fp8-d576", 1024, 576, 16, 4, 1, 2, 512, 0, "bf16", "fp8",
                       seed=36)
# 4-bit experts: K = 192 and 320 end in half a 128-element super-block; the
# shared expert is fp4 (one launch with the routed experts) or bf16 (its own).
RAGGED_FP4 = Workload("ragged-fp4-T77", 77, 256, 32, 4, 2, 4, 192, 320, "bf16", "fp4", seed=30,
                      shared_dtype="fp4")
FP4_BF16_SHARED = Workload("fp4-bf16-shared-T77", 77, 256, 32, 4, 2, 4, 192, 320, "bf16", "fp4",
                           seed=31)
FP4_MANY_ROWS = Workload("many-rows-fp4-T600", 600, 128, 16, 2, 1, 2, 128, 192, "bf16", "fp4",
                         seed=32, shared_dtype="fp4")
BIG_GROUPS_FP4 = Workload("big-groups-fp4-T1024", 1024, 256, 16, 4, 1, 2, 320, 192, "bf16", "fp4",
                          seed=33, shared_dtype="fp4")
# the largest K of fp4 weights: a 64-row tile's block scales fill the LDS they are staged in
FP4_MAX_K = Workload("fp4-max-k-T20", 20, 8192, 16, 4, 1, 2, 256, 0, "bf16", "fp4", seed=34)

SMALL = [WORKLOADS["tiny-f32-T64"], RAGGED_BF16, RAGGED_FP8, PLAIN_TOPK, ALL_GROUPS, WHOLE_GROUP,
         BIG_ROWS, WORKLOADS["decode-bf16-T32"], SINGLE, BIG_GROUPS_BF16, BIG_GROUPS_FP8, SHORT_K,
         RAGGED_FP4, FP4_BF16_SHARED, FP4_MANY_ROWS, WORKLOADS["decode-fp4-T32"], FP4_MAX_K,
         FEW_FP4, FUSED_SELECT_16]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    binding.lib()


def _tol(wl):
    # fp32 end to end: only accumulation order differs from fp64
    return dict(max_tol=1e-4, mean_tol=1e-5) if wl.act_dtype == "f32" else {}


def _scales(d, wl, shared=False):
    """(up, down) scale arrays of the routed (or shared) weights in d, or Nones:
    fp32 per-row scales for fp8, E8M0 block scales for fp4."""
    dt = wl.shared_weight_dtype if shared else wl.expert_dtype
    pre = "ws_" if shared else "w_"
    key = {"fp8": "_scale", "fp4": "_bscale"}.get(dt)
    if key is None:
        return None, None
    up, down = d.get(pre + "up" + key), d.get(pre + "down" + key)
    return (up[None], down[None]) if shared else (up, down)


def _zero_some_fp4_blocks(inp, wl):
    """All-zero 32-element blocks with scale code 0, as the quantiser writes
    for all-zero weights: a few in the routed and shared matrices."""
    rng = np.random.default_rng(5)
    names = [("w_up", "w_up_bscale"), ("w_down", "w_down_bscale")]
    if wl.shared_weight_dtype == "fp4" and wl.shared_inter:
        names += [("ws_up", "ws_up_bscale"), ("ws_down", "ws_down_bscale")]
    for w, b in names:
        sc = inp[b].reshape(-1, inp[b].shape[-1])
        codes = inp[w].reshape(-1, inp[w].shape[-1])
        for _ in range(8):
            r, blk = rng.integers(sc.shape[0]), rng.integers(sc.shape[1])
            sc[r, blk] = 0
            codes[r, 16 * blk:16 * blk + 16] = 0


def _layer_parts(wl, t, cfg):
    T = t["x"].shape[0]
    idx, w = binding.route(cfg, t["x"], t["w_gate"], t["e_bias"])
    perm = binding.permute(cfg, idx, t["x"], with_x_perm=True)
    su, sd = _scales(t, wl)
    y_perm = binding.expert_ffn(cfg, t["w_up"], t["w_down"], t["x"], perm["offsets"], T * wl.top_k,
                                row_index=perm["sorted_slot"], index_div=wl.top_k,
                                w_dtype=wl.expert_dtype, w_up_scale=su, w_down_scale=sd)
    shared = None
    if wl.shared_inter:
        off = torch.tensor([0, T], dtype=torch.int32, device=t["x"].device)
        su, sd = _scales(t, wl, shared=True)
        shared = binding.expert_ffn(cfg, t["ws_up"][None], t["ws_down"][None], t["x"], off, T,
                                    w_dtype=wl.shared_weight_dtype, w_up_scale=su,
                                    w_down_scale=sd)
    y = binding.combine(cfg, perm["slot_pos"], w, y_perm, shared)
    return dict(idx=idx, w=w, perm=perm, y_perm=y_perm, shared=shared, y=y)


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_small_layer_every_entry_point(wl):
    print(f"case {wl.name}", flush=True)
    inp = make_inputs(wl)
    if wl.expert_dtype == "fp4":
        _zero_some_fp4_blocks(inp, wl)
    t = upload(inp, wl)
    cfg = binding.config_from(wl)
    ref = oracle.forward(wl, inp)
    T, k = wl.tokens, wl.top_k

    parts = _layer_parts(wl, t, cfg)
    torch.cuda.synchronize()
    # route: exact ids, weights within rounding
    assert_routing_equal(parts["idx"], parts["w"], ref["topk_idx"], ref["topk_w"], ref["margin"],
                         wl.name)
    # permute: exact against the stable grouping of the same ids
    counts, offsets, sorted_slot, slot_pos = oracle.permute(parts["idx"].cpu().numpy(),
                                                            wl.n_experts)
    p = parts["perm"]
    np.testing.assert_array_equal(p["counts"].cpu().numpy(), counts)
    np.testing.assert_array_equal(p["offsets"].cpu().numpy(), offsets)
    np.testing.assert_array_equal(p["sorted_slot"].cpu().numpy(), sorted_slot)
    np.testing.assert_array_equal(p["slot_pos"].cpu().numpy(), slot_pos)
    xs = t["x"].view(torch.int16) if t["x"].dtype == torch.bfloat16 else t["x"]
    xp = p["x_perm"].view(torch.int16) if p["x_perm"].dtype == torch.bfloat16 else p["x_perm"]
    assert torch.equal(xp, xs[torch.from_numpy(sorted_slot // k).long().cuda()])
    # routed expert MLPs, row by row
    rows = sorted_slot // k
    mats = parts["idx"].cpu().numpy().reshape(-1)[sorted_slot]
    ffn_ref = oracle.ffn_rows(inp["x"], wl.act_dtype, rows, mats, inp["w_up"], inp["w_down"],
                              wl.expert_dtype, inp["w_up_scale"], inp["w_down_scale"],
                              quant_a=wl.expert_dtype == "fp8", w_up_bscale=inp["w_up_bscale"],
                              w_down_bscale=inp["w_down_bscale"])
    allow_rows = allow_tok = None
    if wl.expert_dtype == "fp8":
        allow_rows = fp8_flips.row_allowance(inp["x"], rows, mats, inp["w_up"], inp["w_up_scale"],
                                             inp["w_down"], inp["w_down_scale"])
        allow_tok = fp8_flips.token_allowance(allow_rows, parts["w"].cpu().numpy(),
                                              slot_pos.reshape(T, k))
    assert_close_rms(to_f64(parts["y_perm"]), ffn_ref, f"{wl.name} expert_ffn", **_tol(wl),
                     row_allow=allow_rows)
    if wl.shared_inter:
        bu, bd = _scales(inp, wl, shared=True)
        sh_ref = oracle.ffn_rows(inp["x"], wl.act_dtype, np.arange(T), np.zeros(T),
                                 inp["ws_up"][None], inp["ws_down"][None], wl.shared_weight_dtype,
                                 w_up_bscale=bu, w_down_bscale=bd)
        assert_close_rms(to_f64(parts["shared"]), sh_ref, f"{wl.name} shared", **_tol(wl))
    # combine: only the final rounding separates it from the fp64 sum of its inputs
    comb_ref = oracle.combine(parts["w"].cpu().numpy(), to_f64(parts["y_perm"]), slot_pos,
                              None if parts["shared"] is None else to_f64(parts["shared"]))
    got = to_f64(parts["y"])
    ulp = 2.0 ** -8 if wl.act_dtype == "bf16" else 2.0 ** -22
    assert (np.abs(got - comb_ref) <= ulp * np.abs(comb_ref) + 1e-6 * rms(comb_ref)).all()
    # the layer against the oracle
    assert_close_rms(got, ref["y"], f"{wl.name} layer", **_tol(wl), row_allow=allow_tok)

    # the fused entry point equals the composition bit for bit, routing included
    # (decode-sized calls select and permute in one launch of their own)
    su, sd = _scales(t, wl)
    ssu, ssd = t.get("ws_up_bscale"), t.get("ws_down_bscale")
    f_idx = torch.empty_like(parts["idx"])
    f_w = torch.empty_like(parts["w"])
    y = binding.forward(cfg, t["x"], t["w_gate"], t["e_bias"], t["w_up"], t["w_down"],
                        t.get("ws_up"), t.get("ws_down"), su, sd, ws_up_scale=ssu,
                        ws_down_scale=ssd, topk_idx=f_idx, topk_w=f_w)
    torch.cuda.synchronize()
    assert torch.equal(f_idx, parts["idx"])
    assert torch.equal(f_w.view(torch.int32), parts["w"].view(torch.int32))
    assert torch.equal(y.view(torch.int16) if y.dtype == torch.bfloat16 else y,
                       parts["y"].view(torch.int16) if y.dtype == torch.bfloat16 else parts["y"])


def _bits(y):
    return y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32)


@pytest.mark.parametrize("wl", [RAGGED_BF16, RAGGED_FP8, WORKLOADS["tiny-f32-T64"], RAGGED_FP4],
                         ids=lambda w: w.name)
def test_deterministic_and_token_permutation_equivariant(wl):
    inp = make_inputs(wl)
    t = upload(inp, wl)
    layer = binding.MoELayer(wl, inp)
    y1 = layer(t["x"]).clone()
    y2 = layer(t["x"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(_bits(y1), _bits(y2))
    perm = torch.from_numpy(np.random.default_rng(0).permutation(wl.tokens)).long().cuda()
    y3 = layer(t["x"][perm].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(_bits(y3), _bits(y1)[perm])


def test_routing_does_not_depend_on_batch_or_router_path():
    # up to 2048 tokens the one-kernel router runs; beyond, the logits are a
    # GEMM (given workspace).  Both accumulate the same K steps in the same order.
    wl = WORKLOADS["prefill-bf16-T4096"].with_tokens(2500)
    inp = make_inputs(wl, experts=False)
    t = upload(inp, wl)
    cfg = binding.config_from(wl)
    idx_gemm, w_gemm = binding.route(cfg, t["x"], t["w_gate"], t["e_bias"])
    idx_direct, w_direct = binding.route(cfg, t["x"], t["w_gate"], t["e_bias"],
                                         use_workspace=False)
    idx_few, w_few = binding.route(cfg, t["x"][:40].contiguous(), t["w_gate"], t["e_bias"])
    torch.cuda.synchronize()
    assert torch.equal(idx_gemm, idx_direct) and torch.equal(w_gemm, w_direct)
    assert torch.equal(idx_few, idx_gemm[:40]) and torch.equal(w_few, w_gemm[:40])
    ref_idx, ref_w, margin = oracle.route(wl, inp["x"], inp["w_gate"], inp["e_bias"])
    assert_routing_equal(idx_gemm, w_gemm, ref_idx, ref_w, margin, "T=2500")


def test_exact_ties_go_to_the_lowest_index():
    wl = RAGGED_BF16
    inp = make_inputs(wl)
    inp["w_gate"] = np.zeros_like(inp["w_gate"])
    inp["e_bias"] = np.zeros_like(inp["e_bias"])
    t = upload(inp, wl)
    idx, w = binding.route(binding.config_from(wl), t["x"], t["w_gate"], t["e_bias"])
    torch.cuda.synchronize()
    assert (idx.cpu().numpy() == np.arange(wl.top_k)).all()
    np.testing.assert_allclose(w.cpu().numpy(), 2.5 / wl.top_k, rtol=1e-7)


@pytest.mark.parametrize("wl", [WORKLOADS["decode-bf16-T32"].with_tokens(20), ALL_GROUPS,
                                WORKLOADS["tiny-f32-T64"]], ids=lambda w: f"{w.name}-T{w.tokens}")
def test_exact_ties_in_the_forward_selection(wl):
    """All logits and biases zero: every score ties, so the lowest groups and
    then the lowest expert ids win, each with weight scale / k; through
    moe_forward, whose decode-sized calls select inside the permute launch."""
    inp = make_inputs(wl)
    inp["w_gate"] = np.zeros_like(inp["w_gate"])
    inp["e_bias"] = np.zeros_like(inp["e_bias"])
    layer = binding.MoELayer(wl, inp)
    x = binding.to_device(inp["x"], "cuda", "x", wl)
    layer(x)
    torch.cuda.synchronize()
    ref_idx, ref_w, margin = oracle.route(wl, inp["x"], inp["w_gate"], inp["e_bias"])
    assert (ref_idx == np.arange(wl.top_k)).all()
    assert np.array_equal(layer.topk_idx[:wl.tokens].cpu().numpy(), ref_idx)
    np.testing.assert_allclose(layer.topk_w[:wl.tokens].cpu().numpy(), 2.5 / wl.top_k, rtol=1e-7)


# (E, G, topk_group, top_k) on both selection paths: the register path (a
# power-of-two group of 1 to 64 experts, at most 64 experts in the kept
# groups) and the general one (6 or 128 experts per group, or 96 kept); E =
# 48, 80 and 96 leave the last wave-wide run of experts partly empty.
SELECT_SHAPES = [(48, 48, 6, 6), (64, 32, 3, 4), (80, 5, 2, 8), (128, 4, 2, 8), (256, 4, 1, 8),
                 (96, 16, 3, 8), (128, 4, 3, 8), (256, 2, 1, 8)]


@pytest.mark.parametrize("E,G,tg,k", SELECT_SHAPES,
                         ids=[f"E{e}-G{g}-tg{t}-k{k}" for e, g, t, k in SELECT_SHAPES])
def test_selection_over_group_shapes(E, G, tg, k):
    """Expert ids exact and weights within the routing gate against the
    oracle, on every router path: logit waves then the selection launch (40
    tokens), the one-kernel router (300), the logits GEMM (2100), and inside
    moe_forward, where a few tokens select in the permute launch (5)."""
    base = Workload(f"select-E{E}-G{G}", 2100, 128, E, G, tg, k, 64, 0, "bf16", "bf16",
                    seed=40 + E + G, bias_boost=tuple(range(0, E, 7)), bias_boost_value=0.02)
    inp = make_inputs(base, experts=False)
    t = upload(inp, base)
    cfg = binding.config_from(base)
    ref_idx, ref_w, margin = oracle.route(base, inp["x"], inp["w_gate"], inp["e_bias"])
    for T in (40, 300, 2100):
        print(f"case E={E} G={G} tg={tg} k={k} T={T}", flush=True)
        idx, w = binding.route(cfg, t["x"][:T].contiguous(), t["w_gate"], t["e_bias"])
        torch.cuda.synchronize()
        assert_routing_equal(idx, w, ref_idx[:T], ref_w[:T], margin[:T], f"route T={T}")
    few = base.with_tokens(5)  # x of 5 tokens is the prefix of x of 2100
    print(f"case E={E} G={G} tg={tg} k={k} forward T=5", flush=True)
    inp5 = make_inputs(few)
    layer = binding.MoELayer(few, inp5)
    layer(binding.to_device(inp5["x"], "cuda", "x", few))
    torch.cuda.synchronize()
    assert_routing_equal(layer.topk_idx[:5], layer.topk_w[:5], ref_idx[:5], ref_w[:5], margin[:5],
                         "forward T=5")


def test_zero_tokens_and_growing_calls_reuse_one_workspace():
    wl = RAGGED_BF16
    inp = make_inputs(wl)
    t = upload(inp, wl)
    layer = binding.MoELayer(wl, inp)
    empty = t["x"][:0]
    y0 = torch.empty((0, wl.hidden), dtype=torch.bfloat16, device="cuda")
    layer(empty, y=y0)
    ref = oracle.forward(wl, inp)
    for T in (1, 5, 77):
        y = layer(t["x"][:T].contiguous())
        torch.cuda.synchronize()
        assert_close_rms(to_f64(y), ref["y"][:T], f"T={T}", R=rms(ref["y"]))


def test_unnormalised_weights_and_other_scale():
    wl = Workload("unnorm-T40", 40, 128, 16, 4, 2, 3, 64, 64, "bf16", "bf16",
                  norm_topk_prob=False, routed_scaling_factor=1.5, seed=27)
    inp = make_inputs(wl)
    t = upload(inp, wl)
    ref = oracle.forward(wl, inp)
    y = binding.MoELayer(wl, inp)(t["x"])
    torch.cuda.synchronize()
    assert_close_rms(to_f64(y), ref["y"], wl.name)


def test_identical_experts_reduce_to_one_dense_mlp():
    wl = RAGGED_BF16
    inp = make_inputs(wl)
    inp["w_up"][:] = inp["w_up"][5]
    inp["w_down"][:] = inp["w_down"][5]
    t = upload(inp, wl)
    y = binding.MoELayer(wl, inp)(t["x"])
    # every token: 2.5 * FFN_5(x) + S(x), whatever the routing
    T = wl.tokens
    ffn = oracle.ffn_rows(inp["x"], "bf16", np.arange(T), np.full(T, 5), inp["w_up"],
                          inp["w_down"], "bf16")
    sh = oracle.ffn_rows(inp["x"], "bf16", np.arange(T), np.zeros(T), inp["ws_up"][None],
                         inp["ws_down"][None], "bf16")
    torch.cuda.synchronize()
    assert_close_rms(to_f64(y), 2.5 * ffn + sh, "identical experts")


# 6000 routing slots: the multi-workgroup permute, and 256-row tiles of the ring kernel
MANY_CHUNKS = Workload("many-chunks-T3000", 3000, 128, 16, 2, 1, 2, 64, 64, "bf16", "bf16",
                       seed=35)


@pytest.mark.parametrize("wl", [WORKLOADS["decode-bf16-T32"], RAGGED_FP8,
                                WORKLOADS["decode-fp4-T32"], SINGLE, MANY_CHUNKS],
                         ids=lambda w: w.name)
def test_graph_replays_match_eager(wl):
    # every replay is checked, with eager work and synchronisations between them
    inp = make_inputs(wl)
    t = upload(inp, wl)
    layer = binding.MoELayer(wl, inp)
    x = t["x"].clone()
    y = torch.empty((wl.tokens, wl.hidden), dtype=x.dtype, device="cuda")
    eager = layer(x).clone()
    torch.cuda.synchronize()
    step = binding.GraphStep(layer, x, y)
    other = layer(x[: max(1, wl.tokens // 2)].contiguous())  # eager call on the same workspace
    for _ in range(3):
        y.zero_()
        torch.cuda.synchronize()
        step.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(y), _bits(eager))
        _ = layer(x).sum().item()
    # new input contents flow through the captured graph
    x.copy_(t["x"].flip(0))
    step.replay()
    ref = layer(t["x"].flip(0).contiguous())
    torch.cuda.synchronize()
    assert torch.equal(_bits(y), _bits(ref))
    del other


@pytest.mark.parametrize("wl", [BIG_GROUPS_BF16, BIG_GROUPS_FP8, BIG_GROUPS_FP4, RING_FP8_K7,
                                RING_FP8_K9], ids=lambda w: w.name)
def test_expert_rows_do_not_depend_on_the_tile_shape(wl):
    """A row's result is the same whichever tile shape computes it: a call
    with hundreds of rows per expert (256-row tiles) and a call with a few
    rows (16-row tiles) give identical bits for the rows they share."""
    print(f"case {wl.name}", flush=True)
    inp = make_inputs(wl)
    t = upload(inp, wl)
    cfg = binding.config_from(wl)
    T = wl.tokens
    rng = np.random.default_rng(7)
    src = torch.from_numpy(rng.integers(0, T, size=1200).astype(np.int32)).cuda()
    su, sd = _scales(t, wl)
    sc = dict(w_dtype=wl.expert_dtype, w_up_scale=None if su is None else su[:2],
              w_down_scale=None if sd is None else sd[:2])
    big_off = torch.tensor([0, 700, 1200], dtype=torch.int32, device="cuda")
    big = binding.expert_ffn(cfg, t["w_up"][:2], t["w_down"][:2], t["x"], big_off, 1200,
                             row_index=src, **sc)
    pick = torch.tensor([0, 5, 699, 700, 1199], device="cuda").long()
    small_off = torch.tensor([0, 3, 5], dtype=torch.int32, device="cuda")
    small = binding.expert_ffn(cfg, t["w_up"][:2], t["w_down"][:2], t["x"], small_off, 5,
                               row_index=src[pick].contiguous(), **sc)
    torch.cuda.synchronize()
    assert torch.equal(big[pick], small)
    mats = np.repeat([0, 1], [700, 500])
    bu, bd = _scales(inp, wl)
    fp8 = wl.expert_dtype == "fp8"
    ref = oracle.ffn_rows(inp["x"], wl.act_dtype, src.cpu().numpy(), mats, inp["w_up"][:2],
                          inp["w_down"][:2], wl.expert_dtype,
                          bu[:2] if fp8 else None, bd[:2] if fp8 else None, quant_a=fp8,
                          w_up_bscale=None if fp8 or bu is None else bu[:2],
                          w_down_bscale=None if fp8 or bd is None else bd[:2])
    allow = None
    if wl.expert_dtype == "fp8":
        allow = fp8_flips.row_allowance(inp["x"], src.cpu().numpy(), mats, inp["w_up"],
                                        inp["w_up_scale"], inp["w_down"], inp["w_down_scale"])
    assert_close_rms(to_f64(big), ref, f"{wl.name} expert_ffn 256-row tiles", row_allow=allow)


# 256-row tiles at the edges of the ring kernels: groups whose last tile holds
# 1 to 17 rows (so one row of waves has no rows of its own), empty groups, and
# enough tiles (at least two per compute unit) for the persistent bf16 launch.
EDGE_TILE_ROWS = [1, 10, 16, 17, 255, 0, 129, 3, 64, 200, 33, 1, 16, 90, 7, 250]


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_ring_tiles_with_few_rows(dt):
    """Rows in 256-row tiles that end 1..17 rows into a tile, over a launch
    large enough for the persistent ring kernel: the oracle's rows within the
    gates, and the bits of the same rows computed in 16-row tiles."""
    # the Nemotron-H expert shape (hidden 2688, intermediate 1856) over 16 experts
    wl = Workload(f"edge-tiles-{dt}", 4096, 2688, 16, 4, 1, 2, 1856, 0, "bf16", dt, seed=41)
    print(f"case {wl.name}", flush=True)
    inp = make_inputs(wl)
    t = upload(inp, wl)
    cfg = binding.config_from(wl)
    sizes = np.array([256 * (g % 9) + r if r else 0 for g, r in enumerate(EDGE_TILE_ROWS)])
    sizes[sizes.argmax()] += 256 * 60  # one hot expert: more tiles than compute units
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    S = int(offsets[-1])
    rng = np.random.default_rng(41)
    src = rng.integers(0, wl.tokens, size=S).astype(np.int32)
    su, sd = _scales(t, wl)
    sc = dict(w_dtype=dt, w_up_scale=su, w_down_scale=sd)
    big = binding.expert_ffn(cfg, t["w_up"], t["w_down"], t["x"],
                             torch.from_numpy(offsets).cuda(), S,
                             row_index=torch.from_numpy(src).cuda(), **sc)
    # rows sampled from every group: its first and last rows, the last tile's
    # rows, and random rows
    pick = []
    for g in range(wl.n_experts):
        a, b = int(offsets[g]), int(offsets[g + 1])
        if b > a:
            pick += [a, b - 1] + list(range(max(a, b - 17), b))
            pick += list(rng.integers(a, b, size=8))
    pick = np.unique(np.array(pick))
    mats = np.searchsorted(offsets, pick, side="right") - 1
    counts = np.bincount(mats, minlength=wl.n_experts).astype(np.int32)
    small_off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    small = binding.expert_ffn(cfg, t["w_up"], t["w_down"], t["x"],
                               torch.from_numpy(small_off).cuda(), int(pick.size),
                               row_index=torch.from_numpy(src[pick]).cuda(), **sc)
    torch.cuda.synchronize()
    got = big[torch.from_numpy(pick).cuda().long()]
    assert torch.equal(got, small), "256-row tiles and 16-row tiles differ"
    fp8 = dt == "fp8"
    bu, bd = _scales(inp, wl)
    ref = oracle.ffn_rows(inp["x"], wl.act_dtype, src[pick], mats, inp["w_up"], inp["w_down"], dt,
                          bu if fp8 else None, bd if fp8 else None, quant_a=fp8)
    allow = None
    if fp8:
        allow = fp8_flips.row_allowance(inp["x"], src[pick], mats, inp["w_up"],
                                        inp["w_up_scale"], inp["w_down"], inp["w_down_scale"])
    assert_close_rms(to_f64(got), ref, f"{wl.name} expert_ffn, {pick.size} rows", row_allow=allow)


@pytest.mark.parametrize("T,k,E,skew", [(1500, 6, 128, False), (4097, 6, 128, True),
                                        (16384, 6, 128, True), (3000, 3, 16, False),
                                        (2000, 4, 48, True), (5000, 8, 256, False)])
def test_permute_many_chunks_matches_the_oracle(T, k, E, skew):
    """The multi-workgroup permute (slots beyond one workgroup's share) gives
    exactly the oracle's stable grouping, counts and offsets."""
    print(f"case T={T} k={k} E={E} skew={skew}", flush=True)
    rng = np.random.default_rng(T + k + E)
    if skew:  # two thirds of the slots on 8 experts, some experts empty
        hot = rng.choice(E, size=8, replace=False)
        p = np.full(E, 1.0 / (3 * (E - 8)))
        p[hot] = 2.0 / (3 * 8)
        p[rng.choice(np.setdiff1d(np.arange(E), hot), size=E // 4, replace=False)] = 0.0
        p /= p.sum()
    else:
        p = np.full(E, 1.0 / E)
    idx = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    idx.sort(axis=1)
    cfg = binding.config_from(dataclasses.replace(WORKLOADS["decode-bf16-T32"], n_experts=E,
                                                  n_group=1 if E == 16 else 8, top_k=k))
    perm = binding.permute(cfg, torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    counts, offsets, sorted_slot, slot_pos = oracle.permute(idx, E)
    np.testing.assert_array_equal(perm["counts"].cpu().numpy(), counts)
    np.testing.assert_array_equal(perm["offsets"].cpu().numpy(), offsets)
    np.testing.assert_array_equal(perm["sorted_slot"].cpu().numpy(), sorted_slot)
    np.testing.assert_array_equal(perm["slot_pos"].cpu().numpy(), slot_pos)


def test_decode_rows_past_32_bit_offsets():
    """Activations over 2 GiB: the decode tiles fall back from the buffer-load
    kernel (32-bit offsets) to gemm_kernel, with the same bits per row as the
    buffer-load kernel on the same rows gathered into a small array."""
    d, I, E = 2688, 1856, 4
    a_rows = (1 << 31) // (2 * d) + 2000  # just past 2 GiB of bf16 rows
    print(f"case a_rows={a_rows}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(3)
    a = torch.randn((a_rows, d), generator=gen, device="cuda").to(torch.bfloat16)
    w_up = (torch.randn((E, I, d), generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
    w_down = (torch.randn((E, d, I), generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
    rng = np.random.default_rng(4)
    src = np.concatenate([rng.integers(a_rows - 3000, a_rows, 36), [0, 1, 2, a_rows - 1]])
    src = src.astype(np.int32)
    off = torch.tensor([0, 9, 21, 30, 40], dtype=torch.int32, device="cuda")  # ~10 rows each
    cfg = binding.config_from(dataclasses.replace(WORKLOADS["decode-bf16-T32"], n_experts=16,
                                                  n_group=4, top_k=2))
    idx = torch.from_numpy(src).cuda()
    big = binding.expert_ffn(cfg, w_up, w_down, a, off, 40, row_index=idx, w_dtype="bf16")
    a_small = a[idx.long()].contiguous()
    small = binding.expert_ffn(cfg, w_up, w_down, a_small, off, 40, w_dtype="bf16")
    torch.cuda.synchronize()
    assert torch.equal(big, small)
    mats = np.repeat(np.arange(E), [9, 12, 9, 10])
    pick = np.array([0, 10, 25, 39])
    a_np = a_small.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle.ffn_rows(a_np, "bf16", pick, mats[pick],
                          w_up.view(torch.int16).cpu().numpy().view(np.uint16),
                          w_down.view(torch.int16).cpu().numpy().view(np.uint16), "bf16")
    assert_close_rms(to_f64(big)[pick], ref, "rows past 2 GiB")
    del a
    torch.cuda.empty_cache()


@pytest.mark.parametrize("wl", [RAGGED_BF16, RAGGED_FP8, RAGGED_FP4], ids=lambda w: w.name)
def test_concurrent_calls_on_two_streams(wl):
    # the library keeps no state between calls: two layers with workspaces of
    # their own, enqueued on two streams at once, give the bits of sequential calls
    inp = make_inputs(wl)
    t = upload(inp, wl)
    la, lb = binding.MoELayer(wl, inp), binding.MoELayer(wl, inp)
    xa, xb = t["x"], t["x"][:40].contiguous()
    ref_a, ref_b = la(xa).clone(), lb(xb).clone()
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(4):
        sa.wait_stream(torch.cuda.current_stream())
        sb.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(sa):
            ya = la(xa)
        with torch.cuda.stream(sb):
            yb = lb(xb)
        torch.cuda.synchronize()
        assert torch.equal(_bits(ya), _bits(ref_a)) and torch.equal(_bits(yb), _bits(ref_b))


def test_bf16_rounding_is_nearest_even():
    """The kernels' fp32 -> bf16 rounding (one hardware conversion, shared by
    every epilogue) against the oracle's nearest-even rounding, bit for bit.
    moe_combine with one slot of weight 1 and no shared rows returns
    round(fma(1, v, 0)) = round(v) for any fp32 v: exact ties with an even and
    an odd upper half, one ulp either side of them, subnormals, the largest
    finite values (a tie above the largest bf16 rounds to infinity), signed
    zeros and random finite patterns."""
    rng = np.random.default_rng(5)
    d = 256
    n = 64 * d

    def finite(u):
        return u[((u >> 23) & 0xFF) != 0xFF]

    hi = rng.integers(0, 1 << 16, size=n, dtype=np.uint64).astype(np.uint32) << 16
    pats = [finite(rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)),
            finite(hi | 0x8000), finite(hi | 0x7FFF), finite(hi | 0x8001),
            (rng.integers(0, 1 << 23, size=4096, dtype=np.uint64).astype(np.uint32) |
             (rng.integers(0, 2, size=4096, dtype=np.uint64).astype(np.uint32) << 31)),
            np.array([0x00008000, 0x00018000, 0x007F8000, 0x80008000, 0x7F7F7FFF, 0x7F7F8000,
                      0x7F7FFFFF, 0x7F7E8000, 0xFF7F8000, 0xFF7E8000, 0x00000000, 0x80000000,
                      0x00000001, 0x3F808000, 0x3F818000], dtype=np.uint32)]
    u = np.concatenate(pats)
    u = np.concatenate([u, np.zeros((-u.size) % d, np.uint32)])
    v = u.view(np.float32)
    T = v.size // d
    wl = Workload("bf16-rounding", T, d, 16, 1, 1, 1, 64, 0, "bf16", "bf16")
    cfg = binding.config_from(wl)
    y_perm = torch.from_numpy(v.reshape(T, d).copy()).cuda()
    w = torch.ones((T, 1), dtype=torch.float32, device="cuda")
    slot_pos = torch.arange(T, dtype=torch.int32, device="cuda")
    y = binding.combine(cfg, slot_pos, w, y_perm)
    torch.cuda.synchronize()
    got = y.view(torch.int16).cpu().numpy().astype(np.uint16).reshape(-1)
    ref = oracle.bf16_round(v.astype(np.float64) * 1.0 + 0.0).reshape(-1)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, [(hex(int(u[i])), hex(int(got[i])), hex(int(ref[i]))) for i in bad[:8]]
