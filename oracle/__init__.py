"""fp64 CPU oracle of the Nemotron-H MoE layer forward (ctypes over moe_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use it; the product path never does.  It shares no code with
the HIP library and does not import it.

Sources of each step are cited in ``moe_oracle.c``.  Besides the C oracle this
module holds the permutation and combine definitions, which are plain enough
to state in NumPy:

* permute: slots s = t*k + j are grouped by expert, stably (within one expert
  the slot ids ascend); ``expert_offsets`` is the exclusive prefix sum of the
  per-expert counts; ``sorted_slot[p]`` is the slot at sorted position p and
  ``slot_pos`` its inverse (exo commit "Add support for Nemotron sharding":
  the experts are applied as ``switch_mlp(x, indices)``, one stacked weight
  tensor per projection, so rows are grouped per expert before the GEMMs);
* combine: y[t] = sum_j w[t,j] * y_perm[slot_pos[t*k+j]] + S[t].
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16, FP8, FP4 = 0, 1, 2, 3
EXACT, AS_CONFIGURED = 0, 1
_DT = {"f32": F32, "bf16": BF16, "fp8": FP8, "fp4": FP4}


class _Cfg(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("norm_topk_prob", ctypes.c_int32),
                ("routed_scaling_factor", ctypes.c_double), ("act_dtype", ctypes.c_int32),
                ("expert_dtype", ctypes.c_int32), ("shared_dtype", ctypes.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(
                os.path.join(_HERE, "moe_oracle.c")):
            from oracle import build as _b
            _b.build()
        _lib = ctypes.CDLL(_LIB)
        _lib.orc_bf16_from_double.restype = ctypes.c_uint16
        _lib.orc_bf16_from_double.argtypes = [ctypes.c_double]
        _lib.orc_e4m3_from_float.restype = ctypes.c_uint8
        _lib.orc_e4m3_from_float.argtypes = [ctypes.c_float]
        _lib.orc_e4m3_to_double.restype = ctypes.c_double
        _lib.orc_e4m3_to_double.argtypes = [ctypes.c_uint8]
    return _lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _cfg(wl):
    return _Cfg(wl.hidden, wl.n_experts, wl.n_group, wl.topk_group, wl.top_k, wl.inter,
                wl.shared_inter, int(bool(wl.norm_topk_prob)), float(wl.routed_scaling_factor),
                _DT[wl.act_dtype], _DT[wl.expert_dtype],
                _DT[getattr(wl, "shared_dtype", None) or wl.act_dtype])


def _c(a, dtype=None):
    if a is None:
        return None
    return np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))


# ----------------------------------------------------------------- codecs

def bf16_round(a) -> np.ndarray:
    """fp64 -> bf16 bit patterns, one nearest-even rounding."""
    a = _c(np.asarray(a, dtype=np.float64))
    out = np.empty(a.shape, np.uint16)
    lib().orc_bf16_from_double_array(_p(a), _p(out), ctypes.c_int64(a.size))
    return out


def e4m3_encode(a) -> np.ndarray:
    """fp32 -> OCP e4m3fn codes, nearest even, saturating at +-448."""
    a = _c(np.asarray(a, dtype=np.float32))
    out = np.empty(a.shape, np.uint8)
    lib().orc_e4m3_from_float_array(_p(a), _p(out), ctypes.c_int64(a.size))
    return out


def e4m3_decode(c) -> np.ndarray:
    c = _c(np.asarray(c, dtype=np.uint8))
    out = np.empty(c.shape, np.float64)
    lib().orc_e4m3_to_double_array(_p(c), _p(out), ctypes.c_int64(c.size))
    return out


def e2m1_decode(c) -> np.ndarray:
    """OCP e2m1 codes (low 4 bits of each byte) -> fp64."""
    c = _c(np.asarray(c, dtype=np.uint8))
    out = np.empty(c.shape, np.float64)
    lib().orc_e2m1_to_double_array(_p(c), _p(out), ctypes.c_int64(c.size))
    return out


def e8m0_decode(x) -> np.ndarray:
    """OCP MX E8M0 scales -> fp64 powers of two."""
    x = _c(np.asarray(x, dtype=np.uint8))
    out = np.empty(x.shape, np.float64)
    lib().orc_e8m0_to_double_array(_p(x), _p(out), ctypes.c_int64(x.size))
    return out


def quantize_rows(v):
    """Per-row e4m3 quantiser in fp32 arithmetic: (codes, fp32 scales)."""
    v = _c(np.asarray(v, dtype=np.float32))
    rows, cols = v.shape
    q = np.empty(v.shape, np.uint8)
    s = np.empty(rows, np.float32)
    lib().orc_quantize_rows(_p(v), ctypes.c_int64(rows), ctypes.c_int64(cols), _p(q), _p(s))
    return q, s


# ----------------------------------------------------------------- router

def rmsnorm(x, g, eps: float, dtype: str) -> np.ndarray:
    """The block's pre-mixer RMSNorm of rows x [T, d] with weight g [d], in the
    precision the C oracle states; returns storage form (fp32, or bf16 bits)."""
    x = _c(x)
    g = _c(g)
    T, d = x.shape
    out = np.empty_like(x)
    lib().orc_rmsnorm(_p(x), ctypes.c_int(_DT[dtype]), _p(g), ctypes.c_float(eps),
                      ctypes.c_int64(T), ctypes.c_int64(d), _p(out))
    return out


def block_forward(wl, inp: dict, tokens=None, mode: int = AS_CONFIGURED):
    """block(x) = x + MoE(RMSNorm(x)) for the listed tokens, fp64 (the
    residual add is exact here; the layer runs on the rounded x_norm).

    Returns forward()'s dict with y replaced by the block output, plus x_norm
    (storage form, all tokens)."""
    xn = rmsnorm(inp["x"], inp["norm_w"], wl.norm_eps, wl.act_dtype)
    out = forward(wl, dict(inp, x=xn), tokens=tokens, mode=mode)
    x = inp["x"] if wl.act_dtype == "f32" else _bf16_bits_to_f64(inp["x"])
    out["y"] = np.asarray(x, np.float64)[out["tokens"]] + out["y"]
    out["x_norm"] = xn
    return out


def _bf16_bits_to_f64(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def route(wl, x, w_gate, e_bias, logits=False):
    """Grouped top-k routing of every row of x.

    Returns (topk_idx int32 [T,k] ascending ids, topk_w fp64 [T,k],
    margin fp64 [T]) and, with ``logits=True``, the fp64 logits [T,E].
    """
    T = x.shape[0]
    k, E = wl.top_k, wl.n_experts
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    m = np.empty(T, np.float64)
    lg = np.empty((T, E), np.float64) if logits else None
    cfg = _cfg(wl)
    x, w_gate, e_bias = _c(x), _c(w_gate), _c(e_bias, np.float32)
    rc = lib().orc_route(ctypes.byref(cfg), ctypes.c_int64(T), _p(x), _p(w_gate), _p(e_bias),
                         _p(idx), _p(w), _p(m), _p(lg))
    if rc != 0:
        raise ValueError("invalid routing configuration")
    return (idx, w, m, lg) if logits else (idx, w, m)


# ------------------------------------------------------------------ layer

def forward(wl, inp: dict, tokens=None, mode: int = AS_CONFIGURED):
    """fp64 layer output for the listed tokens (all tokens by default).

    Returns dict(y [n,d] fp64, topk_idx [n,k], topk_w [n,k], margin [n], tokens).
    """
    x = _c(inp["x"])
    T = x.shape[0]
    tokens = np.arange(T, dtype=np.int64) if tokens is None else np.asarray(tokens, np.int64)
    tokens = _c(tokens)
    n, k, d = tokens.size, wl.top_k, wl.hidden
    y = np.empty((n, d), np.float64)
    idx = np.empty((n, k), np.int32)
    w = np.empty((n, k), np.float64)
    m = np.empty(n, np.float64)
    cfg = _cfg(wl)
    args = [_c(inp["w_gate"]), _c(inp["e_bias"], np.float32), _c(inp["w_up"]),
            _c(inp.get("w_up_scale")), _c(inp.get("w_up_bscale")), _c(inp["w_down"]),
            _c(inp.get("w_down_scale")), _c(inp.get("w_down_bscale")), _c(inp["ws_up"]),
            _c(inp.get("ws_up_bscale")), _c(inp["ws_down"]), _c(inp.get("ws_down_bscale"))]
    rc = lib().orc_forward(ctypes.byref(cfg), ctypes.c_int64(n), _p(tokens), _p(x),
                           *[_p(a) for a in args], ctypes.c_int(mode), _p(y), _p(idx), _p(w),
                           _p(m))
    if rc != 0:
        raise ValueError("invalid configuration")
    return dict(y=y, topk_idx=idx, topk_w=w, margin=m, tokens=tokens)


def ffn_rows(a, a_dtype: str, rows, mats, w_up, w_down, w_dtype: str, w_up_scale=None,
             w_down_scale=None, quant_a: bool = False, mode: int = AS_CONFIGURED,
             w_up_bscale=None, w_down_bscale=None):
    """out[p] = Wdown[mats[p]] relu(Wup[mats[p]] a[rows[p]])^2, fp64 [n, d].

    fp8 weights take per-row scales; fp4 weights (two codes per byte) take
    E8M0 block scales, one per 32 elements (``*_bscale``)."""
    a = _c(a)
    w_up, w_down = _c(w_up), _c(w_down)
    inter, d = w_up.shape[-2], w_up.shape[-1]
    if w_dtype == "fp4":
        d *= 2
    rows = _c(np.asarray(rows, np.int32))
    mats = _c(np.asarray(mats, np.int32))
    out = np.empty((rows.size, d), np.float64)
    lib().orc_ffn_rows(ctypes.c_int64(d), ctypes.c_int64(inter), _p(a), ctypes.c_int(_DT[a_dtype]),
                       ctypes.c_int64(rows.size), _p(rows), _p(mats), _p(w_up),
                       _p(_c(w_up_scale, np.float32)), _p(_c(w_up_bscale, np.uint8)), _p(w_down),
                       _p(_c(w_down_scale, np.float32)), _p(_c(w_down_bscale, np.uint8)),
                       ctypes.c_int(_DT[w_dtype]),
                       ctypes.c_int(int(quant_a)), ctypes.c_int(mode), _p(out))
    return out


# ------------------------------------------------ permute and combine

def permute(topk_idx, n_experts: int):
    """Stable grouping of the T*k routing slots by expert (see module doc)."""
    flat = np.asarray(topk_idx, np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=n_experts).astype(np.int32)
    offsets = np.zeros(n_experts + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    sorted_slot = np.argsort(flat, kind="stable").astype(np.int32)
    slot_pos = np.empty_like(sorted_slot)
    slot_pos[sorted_slot] = np.arange(flat.size, dtype=np.int32)
    return counts, offsets, sorted_slot, slot_pos


def combine(topk_w, y_perm, slot_pos, shared=None):
    """y[t] = sum_j w[t,j] y_perm[slot_pos[t*k+j]] (+ shared[t]), fp64."""
    w = np.asarray(topk_w, np.float64)
    T, k = w.shape
    yp = np.asarray(y_perm, np.float64)[np.asarray(slot_pos).reshape(T, k)]
    y = np.einsum("tj,tjd->td", w, yp)
    if shared is not None:
        y = y + np.asarray(shared, np.float64)
    return y
