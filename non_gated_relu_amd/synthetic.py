"""Seeded synthetic inputs for the Nemotron-H MoE layer.

This module only draws random numbers and puts them in their storage format
(fp32, bf16 bits, or fp8 e4m3 codes with per-row fp32 scales).  It holds none
of the layer's arithmetic, so both the fp64 CPU oracle and the HIP path take
their inputs from here and from nowhere else.

Shapes follow the layer statement on the baseRT issue "Requesting converter +
runtime support for the Nemotron-H architecture" (section "Architecture
(config.json)": 128 routed experts, 6 per token, 8 routing groups with one
picked per token, scale 2.5, one 3712-wide shared expert, relu^2 experts
without a gate projection) and the auto-round PR "feat: support Nemotron-H /
Nemotron-Cascade-2" quantisation log (per-expert ``up_proj`` 2688 -> 1856 and
``down_proj`` 1856 -> 2688, both without bias).  The pages ship no trained
weights, so every tensor is a Gaussian draw:

* x ~ N(0, 1), every weight ~ N(0, 0.02), router correction bias ~ N(0, 0.01),
  the bias kept in fp32 (the auto-round discussion names it as a tensor that
  must stay fp32);
* ``np.random.SeedSequence(seed)`` spawns one child per tensor in the order
  x, w_gate, e_bias, w_up, w_down, ws_up, ws_down; the two routed-expert
  tensors spawn one grandchild per expert so any expert regenerates alone;
* draws are ``PCG64(child).standard_normal(shape, float32) * std`` and the
  bf16 workloads round them to bf16 (round to nearest even);
* rows of x for T tokens are a prefix of the rows for any larger T.

The low-precision workloads store the routed expert weights as they arrive at
the layer: OCP fp8 e4m3 codes with one fp32 scale per output channel
(amax / 448), or 4-bit OCP MXFP4 (e2m1 codes, two per byte with the lower
index in the low nibble, and one E8M0 power-of-two scale per block of 32
along the input dimension, chosen as the OCP MX spec's conversion does:
shared exponent floor(log2 amax) - 2, codes rounded to nearest even and
saturated at 6).  Quantising the layer's activations is the layer's own work
and does not happen here.
"""

from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

F32, BF16, FP8, FP4 = "f32", "bf16", "fp8", "fp4"


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic layer configuration (names mirror the model config)."""

    name: str
    tokens: int             # T
    hidden: int             # d            (hidden_size)
    n_experts: int          # E            (n_routed_experts)
    n_group: int            # G            (n_group: routing groups)
    topk_group: int         # tg
    top_k: int              # k            (num_experts_per_tok)
    inter: int              # I            (moe_intermediate_size)
    shared_inter: int       # Is           (moe_shared_expert_intermediate_size)
    act_dtype: str          # x, w_gate, y, and the shared weights unless shared_dtype
    expert_dtype: str       # routed expert weights
    norm_topk_prob: bool = True
    routed_scaling_factor: float = 2.5
    bias_boost: tuple = ()  # experts whose correction bias is raised
    bias_boost_value: float = 0.0
    seed: int = 0
    shared_dtype: str = None  # shared-expert weights; None = act_dtype
    norm_eps: float = 1e-5    # the block's RMSNorm eps (layer_norm_epsilon)
    block: bool = False       # measured as the block x + MoE(RMSNorm(x))

    @property
    def shared_weight_dtype(self) -> str:
        return self.shared_dtype or self.act_dtype

    def with_tokens(self, tokens: int) -> "Workload":
        return dataclasses.replace(self, tokens=int(tokens))


_NEMOTRON = dict(hidden=2688, n_experts=128, n_group=8, topk_group=1, top_k=6,
                 inter=1856, shared_inter=3712)

WORKLOADS = {
    "tiny-f32-T64": Workload("tiny-f32-T64", 64, 256, 16, 4, 2, 2, 128, 256, F32, F32),
    "decode-bf16-T32": Workload("decode-bf16-T32", 32, act_dtype=BF16, expert_dtype=BF16,
                                **_NEMOTRON),
    "prefill-bf16-T4096": Workload("prefill-bf16-T4096", 4096, act_dtype=BF16,
                                   expert_dtype=BF16, **_NEMOTRON),
    # +2.0 on four experts in each of groups 0 and 4.
    "skew-bf16-T16384": Workload("skew-bf16-T16384", 16384, act_dtype=BF16, expert_dtype=BF16,
                                 bias_boost=(0, 4, 8, 12, 64, 68, 72, 76), bias_boost_value=2.0,
                                 **_NEMOTRON),
    "fp8-T8192": Workload("fp8-T8192", 8192, act_dtype=BF16, expert_dtype=FP8, **_NEMOTRON),
    # the decode step as the block around the layer: x + MoE(RMSNorm(x))
    "block-decode-bf16-T32": Workload("block-decode-bf16-T32", 32, act_dtype=BF16,
                                      expert_dtype=BF16, block=True, **_NEMOTRON),
    # routed and shared experts in 4-bit MXFP4 (W4A16: activations and h stay bf16)
    "decode-fp4-T32": Workload("decode-fp4-T32", 32, act_dtype=BF16, expert_dtype=FP4,
                               shared_dtype=FP4, **_NEMOTRON),
}


# ---------------------------------------------------------------------------
# storage conversions (input preparation only)

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest even) and return the 16-bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _e4m3_codes(v: np.ndarray) -> np.ndarray:
    """fp32 -> OCP e4m3fn codes, nearest even, saturating at +-448 (weights only)."""
    v = np.asarray(v, dtype=np.float64)
    mag = np.abs(v)
    _, ex = np.frexp(mag)                  # mag = m * 2**ex, m in [0.5, 1)
    unb = np.maximum(ex - 1, -6)           # binade exponent, subnormals share -6
    quantum = np.ldexp(1.0, unb - 3)       # 3 mantissa bits
    r = np.minimum(np.rint(mag / quantum) * quantum, 448.0)
    _, rex = np.frexp(r)
    normal = r >= 2.0 ** -6
    e_field = np.where(normal, rex - 1 + 7, 0)
    m_field = np.where(normal, r / np.ldexp(1.0, rex - 1) * 8 - 8, r / 2.0 ** -9)
    code = (e_field.astype(np.int64) << 3) | np.rint(m_field).astype(np.int64)
    code = np.where(r == 0, 0, code)
    sign = (np.signbit(v) & (r != 0)).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def quantize_weight_rows_e4m3(w: np.ndarray):
    """Per-output-channel (per-row) e4m3 codes and fp32 scales amax/448."""
    w = np.asarray(w, dtype=np.float32)
    amax = np.abs(w).max(axis=-1)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    scale = np.where(scale == 0, np.float32(1.0), scale).astype(np.float32)
    q = _e4m3_codes((w / scale[..., None]).astype(np.float32))
    return q, scale


_E2M1_MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def _e2m1_codes(v: np.ndarray) -> np.ndarray:
    """Values -> OCP e2m1 codes (0, 0.5, 1, 1.5, 2, 3, 4, 6 and signs), nearest,
    ties to the even code, magnitudes above 6 saturating to 6."""
    v = np.asarray(v, dtype=np.float64)
    mag = np.abs(v)
    code = np.searchsorted(_E2M1_MIDS, mag, side="left")
    tie = (code < 7) & (mag == _E2M1_MIDS[np.minimum(code, 6)])
    code = np.where(tie & (code % 2 == 1), code + 1, code)
    sign = ((v < 0) & (code != 0)).astype(np.int64) << 3
    return (code | sign).astype(np.uint8)


def quantize_weight_rows_mxfp4(w: np.ndarray):
    """[rows, cols] (cols % 32 == 0) -> (packed codes [rows, cols/2] uint8,
    E8M0 block scales [rows, cols/32] uint8)."""
    w = np.asarray(w, dtype=np.float32)
    rows, cols = w.shape
    b = w.reshape(rows, cols // 32, 32).astype(np.float64)
    amax = np.abs(b).max(axis=-1)
    _, ex = np.frexp(amax)                      # amax = m 2^ex, m in [0.5, 1)
    X = np.where(amax > 0, ex - 1 - 2, -127)    # floor(log2 amax) - emax(e2m1)
    X = np.clip(X, -127, 127)
    codes = _e2m1_codes(b / np.ldexp(1.0, X)[..., None]).reshape(rows, cols)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, (X + 127).astype(np.uint8)


# ---------------------------------------------------------------------------

def _draw(seed_seq, shape, std):
    g = np.random.Generator(np.random.PCG64(seed_seq))
    return g.standard_normal(shape, dtype=np.float32) * np.float32(std)


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F32:
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == BF16:
        return f32_to_bf16_bits(a)
    raise ValueError(dtype)


def make_inputs(wl: Workload, experts: bool = True, threads: int = 8) -> dict:
    """Return the workload's tensors in storage form (numpy arrays).

    Keys: x [T,d], w_gate [E,d], e_bias [E] f32, w_up [E,I,d], w_down [E,d,I],
    ws_up [Is,d], ws_down [d,Is]; plus w_up_scale [E,I] and w_down_scale [E,d]
    (fp32, or None) when the routed weights are fp8, or w_up_bscale [E,I,d/32]
    and w_down_bscale [E,d,I/32] (E8M0, or None) when they are fp4, whose
    codes are then packed two per byte (w_up [E,I,d/2], w_down [E,d,I/2]);
    likewise ws_up_bscale [Is,d/32] and ws_down_bscale [d,Is/32] with packed
    ws_up [Is,d/2] and ws_down [d,Is/2] when the shared expert is fp4.
    bf16 tensors are uint16 bit patterns, fp8 / fp4 tensors uint8 codes.
    norm_w [d] (act dtype) is the weight of the RMSNorm before the layer in
    its block.  ``experts=False`` skips the routed expert weights (router-only
    work).
    """
    T, d, E, I, Is = wl.tokens, wl.hidden, wl.n_experts, wl.inter, wl.shared_inter
    root = np.random.SeedSequence(wl.seed)
    c_x, c_wg, c_b, c_up, c_down, c_sup, c_sdown = root.spawn(7)
    out = {}
    # x for T rows is a prefix of x for more rows: draw row by row blocks from one stream
    out["x"] = _store(_draw(c_x, (T, d), 1.0), wl.act_dtype)
    out["w_gate"] = _store(_draw(c_wg, (E, d), 0.02), wl.act_dtype)
    b = _draw(c_b, (E,), 0.01)
    for e in wl.bias_boost:
        b[e] = b[e] + np.float32(wl.bias_boost_value)
    out["e_bias"] = b.astype(np.float32)
    # the block's RMSNorm weight, 1 + N(0, 0.1), from a stream of its own
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, 8])))
    out["norm_w"] = _store(np.float32(1.0) + g.standard_normal(d, dtype=np.float32)
                           * np.float32(0.1), wl.act_dtype)
    out["w_up_scale"] = out["w_down_scale"] = None
    out["w_up_bscale"] = out["w_down_bscale"] = None
    out["ws_up_bscale"] = out["ws_down_bscale"] = None
    sup, sdown = _draw(c_sup, (Is, d), 0.02), _draw(c_sdown, (d, Is), 0.02)
    if wl.shared_weight_dtype == FP4:
        out["ws_up"], out["ws_up_bscale"] = quantize_weight_rows_mxfp4(sup)
        out["ws_down"], out["ws_down_bscale"] = quantize_weight_rows_mxfp4(sdown)
    else:
        out["ws_up"] = _store(sup, wl.shared_weight_dtype)
        out["ws_down"] = _store(sdown, wl.shared_weight_dtype)
    if not experts:
        return out

    up_seeds = c_up.spawn(E)
    down_seeds = c_down.spawn(E)
    if wl.expert_dtype == FP8:
        w_up = np.empty((E, I, d), np.uint8)
        w_down = np.empty((E, d, I), np.uint8)
        s_up = np.empty((E, I), np.float32)
        s_down = np.empty((E, d), np.float32)
    elif wl.expert_dtype == FP4:
        w_up = np.empty((E, I, d // 2), np.uint8)
        w_down = np.empty((E, d, I // 2), np.uint8)
        s_up = np.empty((E, I, d // 32), np.uint8)
        s_down = np.empty((E, d, I // 32), np.uint8)
    else:
        edt = np.float32 if wl.expert_dtype == F32 else np.uint16
        w_up = np.empty((E, I, d), edt)
        w_down = np.empty((E, d, I), edt)

    def one(e):
        u = _draw(up_seeds[e], (I, d), 0.02)
        dn = _draw(down_seeds[e], (d, I), 0.02)
        if wl.expert_dtype == FP8:
            w_up[e], s_up[e] = quantize_weight_rows_e4m3(u)
            w_down[e], s_down[e] = quantize_weight_rows_e4m3(dn)
        elif wl.expert_dtype == FP4:
            w_up[e], s_up[e] = quantize_weight_rows_mxfp4(u)
            w_down[e], s_down[e] = quantize_weight_rows_mxfp4(dn)
        else:
            w_up[e] = _store(u, wl.expert_dtype)
            w_down[e] = _store(dn, wl.expert_dtype)

    with ThreadPoolExecutor(max_workers=max(1, threads)) as pool:
        list(pool.map(one, range(E)))
    out["w_up"], out["w_down"] = w_up, w_down
    if wl.expert_dtype == FP8:
        out["w_up_scale"], out["w_down_scale"] = s_up, s_down
    elif wl.expert_dtype == FP4:
        out["w_up_bscale"], out["w_down_bscale"] = s_up, s_down
    return out
