"""How far e4m3 rounding flips of h may move an fp8 expert row's output.

In the fp8 expert path h = relu(W_up a)^2 is quantised per row to e4m3 in
fp32 (s = amax / 448, q = nearest-even e4m3 of h / s).  The GPU accumulates
W_up a in fp32 in its own order and the oracle in fp64, so where an element
of h / s lies within a hair of a rounding midpoint the two sides can pick
neighbouring codes.  A quantised code is an integer that floating point
decides: both sides decide in the same fp32 arithmetic, but not from bitwise
equal inputs, so the comparison allows for it instead of demanding it.

An element is "near" when its oracle value h / s is within a relative
distance DELTA of a midpoint.  DELTA = 1e-4 is several times the relative
difference of fp32 and fp64 dot products at these lengths (flips seen on the
GPU sat within 3e-5).  A flip moves h_j by the code step at that midpoint
times s, and output i of the row by |W_down[i, j]| times that.  A row's
allowance is the largest change over its outputs if every near element
flipped at once; it is zero for rows with no near element, which then meet
the plain gate.

Everything here is computed from the oracle's codecs and quantiser and from
the inputs, never from GPU results.
"""

from __future__ import annotations

import numpy as np

import oracle
from non_gated_relu_amd.synthetic import bf16_bits_to_f32

DELTA = 1e-4


def _grid():
    v = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    return np.unique(np.abs(v[np.isfinite(v)]))  # 0 ... 448


def near_midpoint(v: np.ndarray, delta: float = DELTA):
    """(mask of |v| within relative delta of an e4m3 rounding midpoint,
    the code step across that midpoint)."""
    grid = _grid()
    mids = (grid[1:] + grid[:-1]) / 2
    steps = np.diff(grid)
    v = np.abs(np.asarray(v, np.float64))
    i = np.searchsorted(mids, v)
    lo = np.clip(i - 1, 0, mids.size - 1)
    hi = np.clip(i, 0, mids.size - 1)
    d_lo, d_hi = np.abs(v - mids[lo]), np.abs(v - mids[hi])
    nearest = np.where(d_lo <= d_hi, lo, hi)
    dist = np.minimum(d_lo, d_hi)
    near = (v > 0) & (dist < delta * v)
    return near, steps[nearest]


def row_allowance(x_bits, rows, mats, w_up, w_up_scale, w_down, w_down_scale,
                  delta: float = DELTA) -> np.ndarray:
    """Allowance of each routed row (token rows[p] through expert mats[p])."""
    rows = np.asarray(rows, np.int64)
    mats = np.asarray(mats, np.int64)
    xq, xs = oracle.quantize_rows(bf16_bits_to_f32(x_bits))
    xd = oracle.e4m3_decode(xq) * xs.astype(np.float64)[:, None]
    out = np.zeros(rows.size)
    for m in np.unique(mats):
        sel = np.flatnonzero(mats == m)
        wu = oracle.e4m3_decode(w_up[m]) * w_up_scale[m].astype(np.float64)[:, None]
        wd = np.abs(oracle.e4m3_decode(w_down[m]) * w_down_scale[m].astype(np.float64)[:, None])
        h = (np.maximum(xd[rows[sel]] @ wu.T, 0.0) ** 2).astype(np.float32)
        s = (h.max(axis=1) / np.float32(448.0)).astype(np.float32)
        s[s == 0] = np.float32(1.0)
        v = (h / s[:, None]).astype(np.float32)
        near, step = near_midpoint(v, delta)
        dh = np.where(near, step * s.astype(np.float64)[:, None], 0.0)
        out[sel] = (dh @ wd.T).max(axis=1)
    return out


def token_allowance(row_allow, topk_w, slot_rows) -> np.ndarray:
    """Allowance of each token's layer output: sum_j |w_tj| times the
    allowance of its routed row.  slot_rows[t, j] indexes row_allow."""
    return (np.abs(np.asarray(topk_w, np.float64)) * np.asarray(row_allow)[slot_rows]).sum(axis=1)
