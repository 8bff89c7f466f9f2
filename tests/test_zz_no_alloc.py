"""moe_forward_static, the layer entry point that allocates nothing, against
moe_forward on the same inputs: the same kernels on the same data, so the
outputs and the routing must be the same bits.  Two calls in a row, the
second with fewer tokens (the static scratch keeps the first call's
contents), and a size beyond the scratch refused on the host."""

import dataclasses

import numpy as np
import pytest
import torch

from gpu_util import upload
from non_gated_relu_amd import binding
from non_gated_relu_amd.synthetic import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

RAGGED_FP8 = Workload("ragged-fp8-T77", 77, 256, 32, 4, 2, 4, 192, 320, "bf16", "fp8", seed=22)
CASES = [(WORKLOADS["decode-bf16-T32"].with_tokens(64), 64, 5),
         (WORKLOADS["decode-fp4-T32"].with_tokens(64), 48, 1),
         (RAGGED_FP8, 77, 13)]


def _bits(y):
    return y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32)


def _call(fn, cfg, t, x, **kw):
    T = x.shape[0]
    idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, cfg.top_k), dtype=torch.float32, device=x.device)
    cnt = torch.empty((cfg.n_experts,), dtype=torch.int32, device=x.device)
    y = fn(cfg, x, t["w_gate"], t["e_bias"], t["w_up"], t["w_down"], t.get("ws_up"),
           t.get("ws_down"), t.get("w_up_scale", t.get("w_up_bscale")),
           t.get("w_down_scale", t.get("w_down_bscale")), topk_idx=idx, topk_w=w,
           expert_counts=cnt, ws_up_scale=t.get("ws_up_bscale"),
           ws_down_scale=t.get("ws_down_bscale"), **kw)
    return y, idx, w, cnt


@pytest.mark.parametrize("wl,t1,t2", CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_static_scratch_forward_equals_forward(wl, t1, t2):
    print(f"case {wl.name}: static forward at T={t1} then T={t2}", flush=True)
    inp = make_inputs(wl)
    t = upload(inp, wl)
    cfg = binding.config_from(wl)
    for T in (t1, t2):
        x = t["x"][:T].contiguous()
        ref = _call(binding.forward, cfg, t, x)
        got = _call(binding.forward_static, cfg, t, x)
        torch.cuda.synchronize()
        assert torch.equal(_bits(got[0]), _bits(ref[0])), f"T={T}: outputs differ"
        assert torch.equal(got[1], ref[1]) and torch.equal(got[3], ref[3]), f"T={T}: routing"
        assert torch.equal(got[2].view(torch.int32), ref[2].view(torch.int32)), f"T={T}: weights"


def test_static_scratch_refuses_sizes_beyond_it():
    wl = WORKLOADS["decode-bf16-T32"]
    cfg = binding.config_from(wl)
    T = 4096
    assert binding.workspace_size(cfg, T) > binding.STATIC_SCRATCH_BYTES
    x = torch.zeros((T, wl.hidden), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((16,), dtype=torch.bfloat16, device="cuda")  # never read: refused first
    with pytest.raises(binding.MoeValueError) as e:
        binding.forward_static(cfg, x, w, w, w, w, w, w)
    assert e.value.status == binding.MOE_ERR_WORKSPACE
