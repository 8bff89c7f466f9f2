"""Thin ctypes binding of libmoe (include/moe.h) over torch device tensors.

Argument marshalling only: every step of the layer runs in the HIP kernels of
libmoe.so; torch provides device memory and the current stream.  There is no
fallback: without the built library every call raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_FP4_E2M1 = 0, 1, 2, 3
DTYPE_CODE = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3, "fp4": MOE_FP4_E2M1}
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8,
               "fp4": torch.uint8}


class MoeConfig(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("norm_topk_prob", ctypes.c_int32),
                ("routed_scaling_factor", ctypes.c_float), ("act_dtype", ctypes.c_int32),
                ("expert_dtype", ctypes.c_int32), ("shared_dtype", ctypes.c_int32)]


def config_from(wl) -> MoeConfig:
    """MoeConfig from any object with the workload fields (hidden, n_experts, ...)."""
    return MoeConfig(wl.hidden, wl.n_experts, wl.n_group, wl.topk_group, wl.top_k, wl.inter,
                     wl.shared_inter, int(bool(wl.norm_topk_prob)),
                     float(wl.routed_scaling_factor), DTYPE_CODE[wl.act_dtype],
                     DTYPE_CODE[wl.expert_dtype],
                     DTYPE_CODE[getattr(wl, "shared_dtype", None) or wl.act_dtype])


_lib = None
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_cfgp = ctypes.POINTER(MoeConfig)


def lib() -> ctypes.CDLL:
    """Load libmoe.so (torch is imported first so both share one HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "(python -m non_gated_relu_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_abi_version.restype = ctypes.c_int32
        L.moe_workspace_size.argtypes = [_cfgp, _i64, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_route.argtypes = [_cfgp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.moe_permute.argtypes = [_cfgp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  ctypes.c_size_t, _vp]
        L.moe_expert_ffn_workspace_size.argtypes = [_cfgp, _i32, _i32, _i32, _i64, _i64,
                                                    ctypes.POINTER(ctypes.c_size_t)]
        L.moe_expert_ffn.argtypes = [_cfgp, _i32, _i32, _i32, _i64, _vp, _i64, _vp, _vp, _i32,
                                     _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.moe_combine.argtypes = [_cfgp, _i64, _vp, _vp, _vp, _vp, _vp, _vp]
        L.moe_forward.argtypes = [_cfgp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.moe_forward_timed.argtypes = L.moe_forward.argtypes + [_vp]
        L.moe_forward_static.argtypes = [_cfgp, _i64] + [_vp] * 16
        L.moe_forward_stage_mask.argtypes = [_cfgp, _i64, ctypes.POINTER(ctypes.c_uint32)]
        L.moe_rmsnorm.argtypes = [_cfgp, _i64, _vp, _vp, ctypes.c_float, _vp, _vp]
        L.moe_block_workspace_size.argtypes = [_cfgp, _i64, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_block_forward.argtypes = ([_cfgp, _i64, _vp, _vp, ctypes.c_float] +
                                        [_vp] * 15 + [ctypes.c_size_t, _vp])
        L.moe_block_forward_timed.argtypes = L.moe_block_forward.argtypes + [_vp]
        L.moe_quantize_rows.argtypes = [_i32, _i64, _i32, _vp, _vp, _vp, _vp]
        for name in ("moe_workspace_size", "moe_route", "moe_permute",
                     "moe_expert_ffn_workspace_size", "moe_expert_ffn", "moe_combine",
                     "moe_forward", "moe_forward_timed", "moe_forward_static",
                     "moe_forward_stage_mask", "moe_rmsnorm",
                     "moe_block_workspace_size", "moe_block_forward",
                     "moe_block_forward_timed", "moe_quantize_rows"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lib().moe_status_string(status).decode()} ({status})")


class MoeValueError(MoeError, ValueError):
    """Invalid or unsupported arguments (nothing was enqueued)."""


def _check(status: int, where: str) -> None:
    if status == MOE_OK:
        return
    if status in (MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE):
        raise MoeValueError(status, where)
    raise MoeError(status, where)


def _p(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libmoe takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libmoe takes contiguous tensors")
    return _vp(t.data_ptr())


def _stream():
    return _vp(torch.cuda.current_stream().cuda_stream)


def _dev(t):
    return t.device


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


def workspace_size(cfg: MoeConfig, tokens: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_workspace_size(ctypes.byref(cfg), tokens, ctypes.byref(n)),
           "moe_workspace_size")
    return n.value


def expert_ffn_workspace_size(cfg: MoeConfig, n_mats: int, inter: int, w_dtype: int,
                              a_rows: int, rows: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_expert_ffn_workspace_size(ctypes.byref(cfg), n_mats, inter, w_dtype, a_rows,
                                               rows, ctypes.byref(n)),
           "moe_expert_ffn_workspace_size")
    return n.value


def workspace(nbytes: int, like: torch.Tensor) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=like.device)


def route(cfg: MoeConfig, x, w_gate, e_bias, topk_idx=None, topk_w=None,
          use_workspace: bool = True):
    T = x.shape[0]
    k = cfg.top_k
    topk_idx = _empty((T, k), torch.int32, x) if topk_idx is None else topk_idx
    topk_w = _empty((T, k), torch.float32, x) if topk_w is None else topk_w
    ws = workspace(workspace_size(cfg, T), x) if use_workspace else None
    _check(lib().moe_route(ctypes.byref(cfg), T, _p(x), _p(w_gate), _p(e_bias), _p(topk_idx),
                           _p(topk_w), _p(ws), 0 if ws is None else ws.numel(), _stream()),
           "moe_route")
    return topk_idx, topk_w


def permute(cfg: MoeConfig, topk_idx, x=None, with_x_perm: bool = False):
    T = topk_idx.shape[0]
    S = T * cfg.top_k
    E = cfg.n_experts
    counts = _empty((E,), torch.int32, topk_idx)
    offsets = _empty((E + 1,), torch.int32, topk_idx)
    sorted_slot = _empty((S,), torch.int32, topk_idx)
    slot_pos = _empty((S,), torch.int32, topk_idx)
    x_perm = None
    if with_x_perm:
        x_perm = _empty((S, x.shape[1]), x.dtype, x)
    ws = workspace(workspace_size(cfg, T), topk_idx)
    _check(lib().moe_permute(ctypes.byref(cfg), T, _p(topk_idx), _p(counts), _p(offsets),
                             _p(sorted_slot), _p(slot_pos), _p(x) if with_x_perm else None,
                             _p(x_perm), _p(ws), ws.numel(), _stream()), "moe_permute")
    return dict(counts=counts, offsets=offsets, sorted_slot=sorted_slot, slot_pos=slot_pos,
                x_perm=x_perm)


def expert_ffn(cfg: MoeConfig, w_up, w_down, a, row_offsets, rows: int, row_index=None,
               index_div: int = 1, w_dtype: str = None, w_up_scale=None, w_down_scale=None,
               out=None):
    """out[r] = Wdown[m] relu(Wup[m] a[src(r)])^2 over the grouped rows (see moe.h).

    uint8 weights are fp8 codes, or packed fp4 codes when their rows hold
    hidden / 2 bytes; the scales are fp32 per row (fp8) or E8M0 blocks (fp4)."""
    n_mats, inter = w_up.shape[0], w_up.shape[1]
    if w_dtype is None:
        w_dtype = {torch.float32: "f32", torch.bfloat16: "bf16", torch.uint8: "fp8"}[w_up.dtype]
        if w_dtype == "fp8" and 2 * w_up.shape[2] == cfg.hidden:
            w_dtype = "fp4"
    code = DTYPE_CODE[w_dtype]
    a_rows = a.shape[0]
    out = _empty((rows, cfg.hidden), torch.float32, a) if out is None else out
    ws = workspace(expert_ffn_workspace_size(cfg, n_mats, inter, code, a_rows, rows), a)
    _check(lib().moe_expert_ffn(ctypes.byref(cfg), n_mats, inter, code, a_rows, _p(a), rows,
                                _p(row_offsets), _p(row_index), index_div, _p(w_up),
                                _p(w_up_scale), _p(w_down), _p(w_down_scale), _p(out), _p(ws),
                                ws.numel(), _stream()), "moe_expert_ffn")
    return out


def combine(cfg: MoeConfig, slot_pos, topk_w, y_perm, shared_out=None, y=None):
    T = topk_w.shape[0]
    if y is None:
        y = _empty((T, cfg.hidden), torch.bfloat16 if cfg.act_dtype == MOE_BF16 else torch.float32,
                   y_perm)
    _check(lib().moe_combine(ctypes.byref(cfg), T, _p(slot_pos), _p(topk_w), _p(y_perm),
                             _p(shared_out), _p(y), _stream()), "moe_combine")
    return y


STAGES = ("route", "permute", "quant_x", "routed_up", "quant_h", "routed_down", "shared_up",
          "shared_down", "combine", "norm")


def forward(cfg: MoeConfig, x, w_gate, e_bias, w_up, w_down, ws_up, ws_down, w_up_scale=None,
            w_down_scale=None, ws=None, y=None, topk_idx=None, topk_w=None, expert_counts=None,
            stage_events=None, ws_up_scale=None, ws_down_scale=None):
    """moe_forward; with ``stage_events`` (a StageEvents) moe_forward_timed.

    Scales: fp8 experts take fp32 per-row ``w_*_scale``; fp4 experts take E8M0
    block scales there, and an fp4 shared expert takes them in ``ws_*_scale``."""
    T = x.shape[0]
    if y is None:
        y = torch.empty((T, cfg.hidden), dtype=x.dtype, device=x.device)
    if ws is None:
        ws = workspace(workspace_size(cfg, T), x)
    args = [ctypes.byref(cfg), T, _p(x), _p(w_gate), _p(e_bias), _p(w_up), _p(w_up_scale),
            _p(w_down), _p(w_down_scale), _p(ws_up), _p(ws_up_scale), _p(ws_down),
            _p(ws_down_scale), _p(y), _p(topk_idx), _p(topk_w), _p(expert_counts), _p(ws),
            ws.numel(), _stream()]
    if stage_events is None:
        _check(lib().moe_forward(*args), "moe_forward")
    else:
        _check(lib().moe_forward_timed(*args, stage_events.array), "moe_forward_timed")
    return y


def forward_static(cfg: MoeConfig, x, w_gate, e_bias, w_up, w_down, ws_up, ws_down,
                   w_up_scale=None, w_down_scale=None, y=None, topk_idx=None, topk_w=None,
                   expert_counts=None, ws_up_scale=None, ws_down_scale=None):
    """moe_forward_static: moe_forward with the library's static device scratch
    as its workspace (nothing is allocated by the library; ``y`` is allocated
    here only when not given)."""
    T = x.shape[0]
    if y is None:
        y = torch.empty((T, cfg.hidden), dtype=x.dtype, device=x.device)
    _check(lib().moe_forward_static(ctypes.byref(cfg), T, _p(x), _p(w_gate), _p(e_bias),
                                    _p(w_up), _p(w_up_scale), _p(w_down), _p(w_down_scale),
                                    _p(ws_up), _p(ws_up_scale), _p(ws_down), _p(ws_down_scale),
                                    _p(y), _p(topk_idx), _p(topk_w), _p(expert_counts),
                                    _stream()), "moe_forward_static")
    return y


STATIC_SCRATCH_BYTES = 64 << 20  # MOE_STATIC_SCRATCH_BYTES


def block_workspace_size(cfg: MoeConfig, tokens: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_block_workspace_size(ctypes.byref(cfg), tokens, ctypes.byref(n)),
           "moe_block_workspace_size")
    return n.value


def quantize_rows(x, q=None, scale=None):
    """Per-row e4m3 codes and fp32 scales of x [rows, cols] (fp32 or bf16):
    moe_quantize_rows."""
    rows, cols = x.shape
    dt = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}.get(x.dtype)
    if dt is None:
        raise TypeError(f"quantize_rows takes fp32 or bf16 rows, not {x.dtype}")
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device) if q is None else q
    scale = torch.empty(rows, dtype=torch.float32, device=x.device) if scale is None else scale
    _check(lib().moe_quantize_rows(dt, rows, cols, _p(x), _p(q), _p(scale), _stream()),
           "moe_quantize_rows")
    return q, scale


def rmsnorm(cfg: MoeConfig, x, weight, eps: float, out=None):
    """The block's RMSNorm of rows x (see moe.h)."""
    out = torch.empty_like(x) if out is None else out
    _check(lib().moe_rmsnorm(ctypes.byref(cfg), x.shape[0], _p(x), _p(weight), float(eps),
                             _p(out), _stream()), "moe_rmsnorm")
    return out


def block_forward(cfg: MoeConfig, x, norm_weight, eps: float, w_gate, e_bias, w_up, w_down,
                  ws_up, ws_down, w_up_scale=None, w_down_scale=None, ws_up_scale=None,
                  ws_down_scale=None, ws=None, out=None, topk_idx=None, topk_w=None,
                  expert_counts=None, stage_events=None):
    """out = x + MoE(RMSNorm(x)): moe_block_forward (moe_block_forward_timed with
    ``stage_events``).  ``out`` may be ``x`` itself."""
    T = x.shape[0]
    out = torch.empty_like(x) if out is None else out
    if ws is None:
        ws = workspace(block_workspace_size(cfg, T), x)
    args = [ctypes.byref(cfg), T, _p(x), _p(norm_weight), float(eps), _p(w_gate), _p(e_bias),
            _p(w_up), _p(w_up_scale), _p(w_down), _p(w_down_scale), _p(ws_up), _p(ws_up_scale),
            _p(ws_down), _p(ws_down_scale), _p(out), _p(topk_idx), _p(topk_w),
            _p(expert_counts), _p(ws), ws.numel(), _stream()]
    if stage_events is None:
        _check(lib().moe_block_forward(*args), "moe_block_forward")
    else:
        _check(lib().moe_block_forward_timed(*args, stage_events.array),
               "moe_block_forward_timed")
    return out


class StageEvents:
    """One start/stop event pair per stage of moe_forward_timed."""

    def __init__(self):
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(STAGES))]
        for e in self.events:
            e.record()  # materialise the underlying hipEvent_t
        torch.cuda.synchronize()
        self.array = (ctypes.c_void_p * len(self.events))(
            *[ctypes.c_void_p(e.cuda_event) for e in self.events])
    def elapsed_ms(self, stages):
        """{stage: ms} of the listed stages (those that ran; call after a sync)."""
        return {s: self.events[2 * STAGES.index(s)].elapsed_time(
            self.events[2 * STAGES.index(s) + 1]) for s in stages}


def stages_of(wl, block: bool = False, tokens: int = None):
    """The stages moe_forward (or, with ``block``, moe_block_forward) runs for
    a workload, in launch order, as the library reports them
    (moe_forward_stage_mask)."""
    cfg = config_from(wl)
    mask = ctypes.c_uint32()
    _check(lib().moe_forward_stage_mask(ctypes.byref(cfg), tokens or wl.tokens,
                                        ctypes.byref(mask)), "moe_forward_stage_mask")
    st = ["norm"] if block else []
    return st + [s for i, s in enumerate(STAGES) if s != "norm" and (mask.value >> i) & 1]


class MoELayer:
    """Device-resident weights of one MoE layer plus a reusable workspace.

    ``layer(x)`` runs the whole forward through ``moe_forward``; the routing
    of the last call is kept in ``topk_idx`` / ``topk_w`` / ``expert_counts``.
    """

    def __init__(self, wl, tensors: dict, device="cuda", max_tokens: int = None):
        self.wl = wl
        self.cfg = config_from(wl)
        self.device = torch.device(device)
        self.t = {k: to_device(v, device, k, wl) for k, v in tensors.items()
                  if v is not None and k != "x"}
        self.max_tokens = max_tokens or wl.tokens
        # (the block's workspace holds the layer's and the normalised rows)
        self.ws = torch.empty(block_workspace_size(self.cfg, self.max_tokens),
                              dtype=torch.uint8, device=self.device)
        T, k = self.max_tokens, wl.top_k
        self.topk_idx = torch.empty((T, k), dtype=torch.int32, device=self.device)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=self.device)
        self.expert_counts = torch.empty((wl.n_experts,), dtype=torch.int32, device=self.device)

    def __call__(self, x, y=None, stage_events=None):
        T = x.shape[0]
        if T > self.max_tokens:
            raise ValueError(f"{T} tokens exceed the workspace sized for {self.max_tokens}")
        t = self.t
        return forward(self.cfg, x, t["w_gate"], t["e_bias"], t["w_up"], t["w_down"],
                       t.get("ws_up"), t.get("ws_down"),
                       t.get("w_up_scale", t.get("w_up_bscale")),
                       t.get("w_down_scale", t.get("w_down_bscale")), ws=self.ws, y=y,
                       topk_idx=self.topk_idx[:T], topk_w=self.topk_w[:T],
                       expert_counts=self.expert_counts, stage_events=stage_events,
                       ws_up_scale=t.get("ws_up_bscale"), ws_down_scale=t.get("ws_down_bscale"))

    def block(self, x, out=None, stage_events=None):
        """out = x + layer(RMSNorm(x)) (moe_block_forward); ``out`` may be ``x``."""
        T = x.shape[0]
        if T > self.max_tokens:
            raise ValueError(f"{T} tokens exceed the workspace sized for {self.max_tokens}")
        t = self.t
        return block_forward(self.cfg, x, t["norm_w"], self.wl.norm_eps, t["w_gate"],
                             t["e_bias"], t["w_up"], t["w_down"], t.get("ws_up"),
                             t.get("ws_down"), t.get("w_up_scale", t.get("w_up_bscale")),
                             t.get("w_down_scale", t.get("w_down_bscale")),
                             t.get("ws_up_bscale"), t.get("ws_down_bscale"), ws=self.ws, out=out,
                             topk_idx=self.topk_idx[:T], topk_w=self.topk_w[:T],
                             expert_counts=self.expert_counts, stage_events=stage_events)


class GraphStep:
    """One MoELayer forward captured in a HIP graph (torch.cuda.CUDAGraph).

    moe_forward allocates nothing and records no memset, so the captured
    launch sequence replays as is; ``replay()`` recomputes ``y`` from the
    current contents of ``x``.
    """

    def __init__(self, layer: MoELayer, x, y, block: bool = False):
        self.x, self.y = x, y

        def step():
            if block:  # the block around the layer: y = x + layer(RMSNorm(x))
                layer.block(x, out=y)
            else:
                layer(x, y=y)

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            step()

    def replay(self):
        self.graph.replay()
        return self.y


def to_device(a, device, name: str, wl):
    """numpy storage array (fp32 / bf16 bits / fp8 codes) -> device tensor."""
    import numpy as np
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to(device)
