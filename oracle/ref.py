"""Reference results in fp64 — oracle side (TEST INFRASTRUCTURE).

The GPU path reaches, up to fp32 rounding, exactly the value of "dequantize,
then dot product". This module is that definition written out:

    y[m][n] = sum_k w'[n][k] * x[m][k]

with ``x`` the fp16 activations widened exactly to fp64 and ``w'`` the
dequantized weights of ``formats.dequantize``. Each product d*q*x has at most
30 significant bits, so it is exact in fp64, and the fp64 sum error (about
K * 2^-53 * sum|w'x|) is far below the tolerance. The sum is a library matrix
product (numpy/BLAS dgemm) over row chunks, so a vocabulary-sized head never
materialises as one fp64 array.

Acceptance bound for a GPU result (per output):
    |y - y_ref| <= 2e-3 * sum_k |w'[n][k] * x[m][k]| + 1e-6

Decode context (Kinetic docs, "What makes it fast"): a dense model reads all
of its weights once per token, and several guessed tokens are checked in one
pass over the weights, so y has M columns that share one weight pass; a
mixture of experts reads only the experts a token is routed to.
"""
from __future__ import annotations

import numpy as np

from . import formats as F

REL_TOL = 2e-3
ABS_TOL = 1e-6
ROW_CHUNK = 16384


def gemv(fmt: str, fields: dict, x16: np.ndarray, rows: slice | None = None):
    """fp64 y[M][N] and sum|w'x| [M][N] for fp16 activations x16 [M][K].
    ``rows`` restricts the computation to a row slice of the matrix."""
    x = np.asarray(x16, dtype=np.float16).astype(np.float64)
    if x.ndim == 1:
        x = x[None, :]
    n_total = F.rows_of(fields)
    r0, r1, _ = (rows or slice(0, n_total)).indices(n_total)
    ys, absd = [], []
    for c0 in range(r0, r1, ROW_CHUNK):
        c1 = min(r1, c0 + ROW_CHUNK)
        w = F.dequantize(fmt, fields, slice(c0, c1))      # fp64 [n, K]
        ys.append(x @ w.T)
        absd.append(np.abs(x) @ np.abs(w).T)
    if not ys:
        m = x.shape[0]
        return np.zeros((m, 0)), np.zeros((m, 0))
    return np.concatenate(ys, axis=1), np.concatenate(absd, axis=1)


def tolerance(abs_dot: np.ndarray) -> np.ndarray:
    return REL_TOL * np.asarray(abs_dot) + ABS_TOL


def within_tolerance(y_gpu, y_ref, abs_dot) -> np.ndarray:
    return np.abs(np.asarray(y_gpu, np.float64) - y_ref) <= tolerance(abs_dot)


def error_ratio(y_gpu, y_ref, abs_dot) -> float:
    """max |y - y_ref| / sum|w'x|, reported so regressions show up long before
    the bound is reached."""
    d = np.abs(np.asarray(y_gpu, np.float64) - y_ref)
    den = np.maximum(np.asarray(abs_dot), 1e-300)
    return float(np.max(d / den)) if d.size else 0.0


def argmax_lowest(y: np.ndarray) -> np.ndarray:
    """Index of the largest value per column; the lowest index wins ties."""
    y = np.asarray(y)
    if y.ndim == 1:
        return np.int64(np.argmax(y))
    return np.argmax(y, axis=-1)


def top2_gap(y: np.ndarray) -> np.ndarray:
    """Largest minus second-largest value per column (argmax robustness)."""
    y = np.asarray(y, np.float64)
    part = -np.partition(-y, 1, axis=-1)
    return part[..., 0] - part[..., 1]


# ---------------------------------------------------------------- experts ---

def silu(z: np.ndarray) -> np.ndarray:
    """z / (1 + e^-z) in fp64."""
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu_h16(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """h = fp16(silu(gate) * up): the gated-FFN activation between the gate/up
    and down projections of one expert, rounded to fp16 (RNE) because it is
    the next GEMV's fp16 input."""
    return (silu(gate) * np.asarray(up, np.float64)).astype(np.float16)


def moe_gemv(fmt: str, expert_fields, x16: np.ndarray, route_ids: np.ndarray,
             route_w: np.ndarray | None, x_per_slot: bool):
    """Routed-expert GEMV.

    x16 is [M][K] (x_per_slot False: every slot of token m reads x[m]) or
    [M][top_k][K] (True: slot j of token m reads x[m][j]).
    route_w None: per-slot outputs y[M][top_k][N].
    route_w given: y[M][N] = sum_j route_w[m][j] * (W_{id[m][j]} x_{m,j}),
    summed in slot order j = 0..top_k-1.
    Returns (y, sum of |terms|) with the same shape.
    """
    ids = np.asarray(route_ids)
    m_tokens, top_k = ids.shape
    # experts no token is routed to may be absent (None)
    n = next(F.rows_of(f) for f in expert_fields if f is not None)
    per = np.zeros((m_tokens, top_k, n))
    per_abs = np.zeros((m_tokens, top_k, n))
    for t in range(m_tokens):
        for j in range(top_k):
            xv = x16[t, j] if x_per_slot else x16[t]
            y, a = gemv(fmt, expert_fields[int(ids[t, j])], xv[None, :])
            per[t, j], per_abs[t, j] = y[0], a[0]
    if route_w is None:
        return per, per_abs
    r = np.asarray(route_w, np.float32).astype(np.float64)
    out = np.zeros((m_tokens, n))
    out_abs = np.zeros((m_tokens, n))
    for j in range(top_k):                       # fixed slot order
        out = out + r[:, j:j + 1] * per[:, j]
        out_abs = out_abs + np.abs(r[:, j:j + 1]) * per_abs[:, j]
    return out, out_abs


def moe_ffn(fmt: str, gate_fields, up_fields, down_fields, x16, route_ids, route_w,
            h_override: np.ndarray | None = None):
    """Routed-expert FFN for decode tokens: per token m and slot j with expert
    e = route_ids[m][j]: g = Gate_e x_m, u = Up_e x_m, h = fp16(silu(g)*u),
    then y[m] = sum_j route_w[m][j] * Down_e h, in slot order.

    ``h_override`` ([M][top_k][inter] fp16) feeds a given h to the down
    projection instead of the oracle's own, so the down GEMV can be checked
    on exactly the GPU's input. Returns (y, abs, g, u, h)."""
    g, g_abs = moe_gemv(fmt, gate_fields, x16, route_ids, None, False)
    u, u_abs = moe_gemv(fmt, up_fields, x16, route_ids, None, False)
    h = swiglu_h16(g, u) if h_override is None else np.asarray(h_override, np.float16)
    y, y_abs = moe_gemv(fmt, down_fields, h, route_ids, route_w, True)
    return y, y_abs, (g, g_abs), (u, u_abs), h
