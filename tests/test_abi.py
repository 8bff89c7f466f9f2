"""The C ABI on the host: exported symbols, argument checks, workspace sizing.

No GPU is touched: every call here either fails its host-side checks or has
nothing to enqueue (zero tokens), which the ABI answers before any HIP call.
"""

import ctypes
import os
import re

import pytest

from non_gated_relu_amd import binding
from non_gated_relu_amd.binding import (MOE_BF16, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED,
                                        MOE_ERR_WORKSPACE, MOE_F32, MOE_FP4_E2M1, MOE_FP8_E4M3,
                                        MOE_OK, MoeConfig)
from non_gated_relu_amd.synthetic import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_layer_entry_points():
    names = _declared()
    for n in ("moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_forward",
              "moe_workspace_size", "moe_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(binding.LIB_PATH)
    for n in _declared():
        assert hasattr(L, n), n
    assert binding.lib().moe_abi_version() == 6


def _cfg(**kw):
    c = binding.config_from(WORKLOADS["decode-bf16-T32"])
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _ws(cfg, T=32):
    n = ctypes.c_size_t()
    st = binding.lib().moe_workspace_size(ctypes.byref(cfg) if cfg is not None else None, T,
                                          ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,status", [
    (dict(n_group=3), MOE_ERR_INVALID_ARG),          # 128 % 3 != 0
    (dict(topk_group=9), MOE_ERR_INVALID_ARG),       # more groups kept than exist
    (dict(topk_group=0), MOE_ERR_INVALID_ARG),
    (dict(top_k=17), MOE_ERR_INVALID_ARG),           # > topk_group * 16
    (dict(top_k=0), MOE_ERR_INVALID_ARG),
    (dict(hidden=0), MOE_ERR_INVALID_ARG),
    (dict(norm_topk_prob=2), MOE_ERR_INVALID_ARG),
    (dict(routed_scaling_factor=float("nan")), MOE_ERR_INVALID_ARG),
    (dict(act_dtype=7), MOE_ERR_INVALID_ARG),
    (dict(hidden=2690), MOE_ERR_UNSUPPORTED),        # not a multiple of 64
    (dict(inter=1800), MOE_ERR_UNSUPPORTED),
    (dict(n_experts=512, n_group=8), MOE_ERR_UNSUPPORTED),
    (dict(act_dtype=MOE_F32), MOE_ERR_UNSUPPORTED),  # fp32 activations with bf16 experts
    (dict(act_dtype=MOE_FP8_E4M3), MOE_ERR_UNSUPPORTED),
    (dict(shared_dtype=9), MOE_ERR_INVALID_ARG),
    (dict(shared_dtype=MOE_FP4_E2M1), MOE_ERR_UNSUPPORTED),  # fp4 shared needs fp4 experts
    (dict(shared_dtype=MOE_FP8_E4M3, expert_dtype=MOE_FP8_E4M3), MOE_ERR_UNSUPPORTED),
    (dict(expert_dtype=MOE_FP4_E2M1, act_dtype=MOE_F32, shared_dtype=MOE_F32),
     MOE_ERR_UNSUPPORTED),
    (dict(), MOE_OK),
    (dict(expert_dtype=MOE_FP8_E4M3), MOE_OK),
    (dict(expert_dtype=MOE_FP4_E2M1), MOE_OK),
    (dict(expert_dtype=MOE_FP4_E2M1, shared_dtype=MOE_FP4_E2M1), MOE_OK),
    (dict(expert_dtype=MOE_FP4_E2M1, hidden=8192), MOE_OK),             # the largest fp4 K
    (dict(expert_dtype=MOE_FP4_E2M1, hidden=8256), MOE_ERR_UNSUPPORTED),
    (dict(expert_dtype=MOE_FP4_E2M1, shared_dtype=MOE_FP4_E2M1, shared_inter=8256),
     MOE_ERR_UNSUPPORTED),
])
def test_config_checks(kw, status):
    assert _ws(_cfg(**kw))[0] == status


def test_null_config_and_negative_tokens():
    assert _ws(None)[0] == MOE_ERR_INVALID_ARG
    assert _ws(_cfg(), -1)[0] == MOE_ERR_INVALID_ARG
    assert _ws(_cfg(), 2 ** 30)[0] == MOE_ERR_UNSUPPORTED  # slot ids must fit int32


def test_workspace_grows_with_tokens():
    c = _cfg()
    sizes = [_ws(c, T)[1] for T in (1, 32, 4096, 16384)]
    assert sizes == sorted(sizes) and sizes[0] > 0
    # fp32 routed outputs dominate: at least T*k*d*4 bytes
    assert sizes[2] >= 4096 * 6 * 2688 * 4


def test_zero_tokens_enqueue_nothing():
    L = binding.lib()
    c = _cfg()
    assert L.moe_route(ctypes.byref(c), 0, None, None, None, None, None, None, 0, None) == MOE_OK
    assert L.moe_forward(ctypes.byref(c), 0, *([None] * 16), 0, None) == MOE_OK
    assert L.moe_combine(ctypes.byref(c), 0, None, None, None, None, None, None) == MOE_OK


@pytest.mark.parametrize("name,tokens,stages", [
    ("decode-bf16-T32", 32, ["route", "permute", "routed_up", "routed_down", "combine"]),
    # a bf16 shared expert rides in the routed launches as one more group
    ("skew-bf16-T16384", 16384, ["route", "permute", "routed_up", "routed_down", "combine"]),
    # a bf16 shared expert beside fp8 experts rides in their launches when both
    # take the 256 x 256 ring tiles (the mixed ring kernel) ...
    ("fp8-T8192", 8192, ["route", "permute", "quant_x", "routed_up", "quant_h", "routed_down",
                         "combine"]),
    # ... and has launches of its own for fewer rows per expert
    ("fp8-T8192", 64, ["route", "permute", "quant_x", "routed_up", "quant_h", "routed_down",
                       "shared_up", "shared_down", "combine"]),
    ("decode-fp4-T32", 32, ["route", "permute", "routed_up", "routed_down", "combine"]),
    ("tiny-f32-T64", 64, ["route", "permute", "routed_up", "routed_down", "combine"]),
])
def test_forward_stage_mask(name, tokens, stages):
    """moe_forward_stage_mask answers on the host which launches a forward runs."""
    wl = WORKLOADS[name]
    assert binding.stages_of(wl, tokens=tokens) == stages
    assert binding.stages_of(wl, block=True, tokens=tokens) == ["norm"] + stages
    m = ctypes.c_uint32(7)
    c = binding.config_from(wl)
    assert binding.lib().moe_forward_stage_mask(ctypes.byref(c), 0, ctypes.byref(m)) == MOE_OK
    assert m.value == 0


def test_static_forward_refuses_sizes_beyond_its_scratch():
    """moe_forward_static checks its size against the static scratch on the
    host, before it resolves the scratch or enqueues anything."""
    L = binding.lib()
    c = _cfg()
    assert L.moe_forward_static(ctypes.byref(c), 0, *([None] * 16)) == MOE_OK
    big = 1
    while _ws(c, big)[1] <= binding.STATIC_SCRATCH_BYTES:
        big *= 2
    fake = ctypes.c_void_p(1 << 20)
    assert L.moe_forward_static(ctypes.byref(c), big, *([fake] * 16)) == MOE_ERR_WORKSPACE
    # the header's figure: a Nemotron-H-shaped bf16 layer fits up to about 600 tokens
    assert _ws(c, 512)[1] <= binding.STATIC_SCRATCH_BYTES < _ws(c, 700)[1]


def test_null_and_misaligned_pointers_are_refused():
    L = binding.lib()
    c = _cfg()
    fake = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10008)
    assert L.moe_route(ctypes.byref(c), 4, None, fake, fake, fake, fake, None, 0,
                       None) == MOE_ERR_INVALID_ARG
    assert L.moe_route(ctypes.byref(c), 4, odd, fake, fake, fake, fake, None, 0,
                       None) == MOE_ERR_INVALID_ARG
    args = [fake] * 6 + [None] * 2 + [fake] * 2 + [fake]
    # x, w_gate, e_bias, w_up, w_up_scale(NULL ok for bf16), ...
    st = L.moe_forward(ctypes.byref(c), 4, fake, fake, fake, fake, None, fake, None, fake, None,
                       fake, None, fake, None, None, None, None, 0, None)
    assert st == MOE_ERR_WORKSPACE
    c8 = _cfg(expert_dtype=MOE_FP8_E4M3)
    st = L.moe_forward(ctypes.byref(c8), 4, fake, fake, fake, fake, None, fake, None, fake, None,
                       fake, None, fake, None, None, None, fake, 1 << 40, None)
    assert st == MOE_ERR_INVALID_ARG  # fp8 weights need their scales
    c4 = _cfg(expert_dtype=MOE_FP4_E2M1)
    st = L.moe_forward(ctypes.byref(c4), 4, fake, fake, fake, fake, None, fake, None, fake, None,
                       fake, None, fake, None, None, None, fake, 1 << 40, None)
    assert st == MOE_ERR_INVALID_ARG  # fp4 weights need their block scales
    c44 = _cfg(expert_dtype=MOE_FP4_E2M1, shared_dtype=MOE_FP4_E2M1)
    st = L.moe_forward(ctypes.byref(c44), 4, fake, fake, fake, fake, fake, fake, fake, fake, None,
                       fake, None, fake, None, None, None, fake, 1 << 40, None)
    assert st == MOE_ERR_INVALID_ARG  # and so does an fp4 shared expert
    del args


def test_block_entry_points_check_on_the_host():
    L = binding.lib()
    c = _cfg()
    fake = ctypes.c_void_p(0x10000)
    # eps must be finite and non-negative; pointers present
    assert L.moe_rmsnorm(ctypes.byref(c), 4, fake, fake, -1.0, fake, None) == MOE_ERR_INVALID_ARG
    assert L.moe_rmsnorm(ctypes.byref(c), 4, fake, fake, float("nan"), fake,
                         None) == MOE_ERR_INVALID_ARG
    assert L.moe_rmsnorm(ctypes.byref(c), 4, None, fake, 1e-5, fake, None) == MOE_ERR_INVALID_ARG
    assert L.moe_rmsnorm(ctypes.byref(c), 0, None, None, 1e-5, None, None) == MOE_OK
    # the block's workspace holds the layer's and T x d normalised rows
    nb, nl = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.moe_block_workspace_size(ctypes.byref(c), 32, ctypes.byref(nb)) == MOE_OK
    assert L.moe_workspace_size(ctypes.byref(c), 32, ctypes.byref(nl)) == MOE_OK
    assert nb.value >= nl.value + 32 * c.hidden * 2
    # no norm weight; then a workspace one byte short
    args = [fake] * 11 + [None, None, None, fake]  # weights, out; routing outputs; workspace
    st = L.moe_block_forward(ctypes.byref(c), 4, fake, None, 1e-5, *args, 1 << 40, None)
    assert st == MOE_ERR_INVALID_ARG
    nb4 = ctypes.c_size_t()
    L.moe_block_workspace_size(ctypes.byref(c), 4, ctypes.byref(nb4))
    st = L.moe_block_forward(ctypes.byref(c), 4, fake, fake, 1e-5, *args, nb4.value - 1, None)
    assert st == MOE_ERR_WORKSPACE


def test_quantize_rows_checks_on_the_host():
    L = binding.lib()
    fake = ctypes.c_void_p(0x10000)
    assert L.moe_quantize_rows(MOE_FP8_E4M3, 4, 64, fake, fake, fake, None) == MOE_ERR_UNSUPPORTED
    assert L.moe_quantize_rows(MOE_BF16, -1, 64, fake, fake, fake, None) == MOE_ERR_INVALID_ARG
    assert L.moe_quantize_rows(MOE_BF16, 4, 60, fake, fake, fake, None) == MOE_ERR_INVALID_ARG
    assert L.moe_quantize_rows(MOE_F32, 4, 0, fake, fake, fake, None) == MOE_ERR_INVALID_ARG
    assert L.moe_quantize_rows(MOE_F32, 4, 64, fake, None, fake, None) == MOE_ERR_INVALID_ARG
    assert L.moe_quantize_rows(MOE_F32, 4, 64, ctypes.c_void_p(0x10004), fake, fake,
                               None) == MOE_ERR_INVALID_ARG
    assert L.moe_quantize_rows(MOE_BF16, 0, 64, None, None, None, None) == MOE_OK


def test_permute_x_and_x_perm_go_together():
    L = binding.lib()
    c = _cfg()
    fake = ctypes.c_void_p(0x10000)
    st = L.moe_permute(ctypes.byref(c), 4, fake, fake, fake, fake, fake, fake, None, fake, 1 << 20,
                       None)
    assert st == MOE_ERR_INVALID_ARG


def test_expert_ffn_checks():
    L = binding.lib()
    c = _cfg()
    fake = ctypes.c_void_p(0x10000)
    # index_div must be >= 1
    st = L.moe_expert_ffn(ctypes.byref(c), 4, 128, MOE_BF16, 8, fake, 8, fake, None, 0, fake, None,
                          fake, None, fake, fake, 1 << 30, None)
    assert st == MOE_ERR_INVALID_ARG
    # fp32 weights with bf16 activations is not a supported pairing
    st = L.moe_expert_ffn(ctypes.byref(c), 4, 128, MOE_F32, 8, fake, 8, fake, None, 1, fake, None,
                          fake, None, fake, fake, 1 << 30, None)
    assert st == MOE_ERR_UNSUPPORTED
    # workspace too small
    st = L.moe_expert_ffn(ctypes.byref(c), 4, 128, MOE_BF16, 8, fake, 8, fake, None, 1, fake, None,
                          fake, None, fake, fake, 16, None)
    assert st == MOE_ERR_WORKSPACE
    # no rows: nothing to do
    st = L.moe_expert_ffn(ctypes.byref(c), 4, 128, MOE_BF16, 8, fake, 0, fake, None, 1, fake, None,
                          fake, None, fake, fake, 16, None)
    assert st == MOE_OK
    # fp4 weights need their block scales; unknown weight types are refused
    st = L.moe_expert_ffn(ctypes.byref(c), 4, 128, MOE_FP4_E2M1, 8, fake, 8, fake, None, 1, fake,
                          None, fake, fake, fake, fake, 1 << 30, None)
    assert st == MOE_ERR_INVALID_ARG
    st = L.moe_expert_ffn(ctypes.byref(c), 4, 128, 4, 8, fake, 8, fake, None, 1, fake, fake,
                          fake, fake, fake, fake, 1 << 30, None)
    assert st == MOE_ERR_INVALID_ARG


def test_status_strings():
    L = binding.lib()
    for s in range(5):
        assert L.moe_status_string(s)
    with pytest.raises(ValueError):
        binding._check(MOE_ERR_UNSUPPORTED, "x")
    with pytest.raises(RuntimeError):
        binding._check(4, "x")


def test_config_struct_layout_matches_header():
    # 8 int32 + float + 3 int32
    assert ctypes.sizeof(MoeConfig) == 48
    c = binding.config_from(WORKLOADS["fp8-T8192"])
    assert (c.act_dtype, c.expert_dtype, c.shared_dtype) == (MOE_BF16, MOE_FP8_E4M3, MOE_BF16)
    c = binding.config_from(WORKLOADS["decode-fp4-T32"])
    assert (c.act_dtype, c.expert_dtype, c.shared_dtype) == (MOE_BF16, MOE_FP4_E2M1, MOE_FP4_E2M1)
