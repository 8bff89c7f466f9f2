"""GPU parity of the block around the layer, out = x + MoE(RMSNorm(x)):
moe_rmsnorm and moe_block_forward against the oracle."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close_rms, assert_routing_equal, to_f64, upload
from non_gated_relu_amd import binding
from non_gated_relu_amd.synthetic import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

RAGGED = Workload("block-ragged-T77", 77, 256, 32, 4, 2, 4, 192, 320, "bf16", "bf16", seed=41)
RAGGED_FP4 = Workload("block-ragged-fp4-T77", 77, 256, 32, 4, 2, 4, 192, 320, "bf16", "fp4",
                      seed=42, shared_dtype="fp4")
RAGGED_FP8 = Workload("block-ragged-fp8-T77", 77, 256, 32, 4, 2, 4, 192, 320, "bf16", "fp8",
                      seed=43)
# Hundreds of rows per expert: the 256 x 256 tile kernels, with the residual
# added in the combine.
BIG = Workload("block-big-groups-T1024", 1024, 256, 16, 4, 1, 2, 320, 192, "bf16", "bf16",
               seed=44)
BIG_FP8 = Workload("block-big-groups-fp8-T1024", 1024, 256, 16, 4, 1, 2, 320, 192, "bf16", "fp8",
                   seed=45)
CASES = [WORKLOADS["tiny-f32-T64"], RAGGED, RAGGED_FP4, RAGGED_FP8, WORKLOADS["decode-bf16-T32"],
         WORKLOADS["decode-fp4-T32"], BIG, BIG_FP8]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    binding.lib()


def _bits(y):
    return y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32)


def _tol(wl):
    return dict(max_tol=1e-4, mean_tol=1e-5) if wl.act_dtype == "f32" else {}


@pytest.mark.parametrize("wl", [RAGGED, WORKLOADS["decode-bf16-T32"], WORKLOADS["tiny-f32-T64"]],
                         ids=lambda w: w.name)
def test_rmsnorm_matches_the_oracle(wl):
    print(f"case {wl.name}", flush=True)
    inp = make_inputs(wl, experts=False)
    t = upload(inp, wl)
    got = binding.rmsnorm(binding.config_from(wl), t["x"], t["norm_w"], wl.norm_eps)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(inp["x"], inp["norm_w"], wl.norm_eps, wl.act_dtype)
    if wl.act_dtype == "bf16":
        # the fp64 sum of bf16 squares is exact: the same bits as the oracle
        np.testing.assert_array_equal(got.view(torch.int16).cpu().numpy().view(np.uint16), ref)
    else:
        # fp32 rows: the fp64 sum may round in another order, moving r by an ulp
        np.testing.assert_allclose(got.cpu().numpy(), ref, rtol=4 * 2.0 ** -23, atol=0)


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_block_matches_the_oracle(wl):
    print(f"case {wl.name}", flush=True)
    inp = make_inputs(wl)
    t = upload(inp, wl)
    layer = binding.MoELayer(wl, inp)
    out = layer.block(t["x"])
    torch.cuda.synchronize()
    ref = oracle.block_forward(wl, inp)
    assert_routing_equal(layer.topk_idx, layer.topk_w, ref["topk_idx"], ref["topk_w"],
                         ref["margin"], f"{wl.name} block")
    assert_close_rms(to_f64(out), ref["y"], f"{wl.name} block", **_tol(wl))
    # in place (the residual stream updated where it lies) gives the same bits
    x2 = t["x"].clone()
    layer.block(x2, out=x2)
    torch.cuda.synchronize()
    assert torch.equal(_bits(x2), _bits(out))
    # the fused residual add agrees with adding x to the layer's own output on the
    # normalised rows, up to that output's extra rounding
    xn = binding.rmsnorm(layer.cfg, t["x"], layer.t["norm_w"], wl.norm_eps)
    y = layer(xn)
    torch.cuda.synchronize()
    assert torch.equal(layer.topk_idx[:wl.tokens].cpu(), torch.from_numpy(ref["topk_idx"]))
    step = 2.0 ** -8 if wl.act_dtype == "bf16" else 2.0 ** -23
    comp = to_f64(t["x"]) + to_f64(y)
    assert np.all(np.abs(to_f64(out) - comp) <= step * (np.abs(to_f64(out)) + np.abs(to_f64(y))))


def test_block_without_expert_output_is_the_residual():
    wl = RAGGED
    inp = make_inputs(wl)
    inp["w_down"] = np.zeros_like(inp["w_down"])
    inp["ws_down"] = np.zeros_like(inp["ws_down"])
    t = upload(inp, wl)
    out = binding.MoELayer(wl, inp).block(t["x"])
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(t["x"]))


@pytest.mark.parametrize("wl", [WORKLOADS["decode-bf16-T32"], RAGGED_FP4], ids=lambda w: w.name)
def test_block_graph_replays_match_eager(wl):
    inp = make_inputs(wl)
    t = upload(inp, wl)
    layer = binding.MoELayer(wl, inp)
    x = t["x"].clone()
    y = torch.empty_like(x)
    eager = layer.block(x).clone()
    torch.cuda.synchronize()
    step = binding.GraphStep(layer, x, y, block=True)
    for _ in range(3):
        y.zero_()
        torch.cuda.synchronize()
        step.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(y), _bits(eager))
        _ = layer.block(x).sum().item()  # eager work on the same workspace between replays


def test_block_timed_reports_the_norm_stage():
    wl = dataclasses.replace(RAGGED, name="block-timed")
    inp = make_inputs(wl)
    t = upload(inp, wl)
    layer = binding.MoELayer(wl, inp)
    ev = binding.StageEvents()
    out = layer.block(t["x"], stage_events=ev)
    plain = layer.block(t["x"])
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(plain))
    ms = ev.elapsed_ms(binding.stages_of(wl, block=True))
    assert set(ms) >= {"norm", "route", "combine"} and all(v > 0 for v in ms.values())
