"""Shortlist: an exact argmax over a Q8_0 output layer that scores only the
rows that can still win — oracle side (TEST INFRASTRUCTURE).

Kinetic docs, "What makes it fast" (the Shortlist paragraph): picking the next
token reads an output layer with up to a quarter of a million rows; a small
copy of that layer gives a bound on every row's score, and exact scores are
computed only for the rows whose bound still lets them win. The pages give
neither the copy nor the bound; what follows is this library's reading, each
step written so it can be checked by hand.

Split of a Q8_0 quant q (int8, w' = d q) into a high and a low part:
    v  = floor(q / 8) + 16        0..31  (five bits)
    ql = q - 8 (v - 16)           0..7   (the low three bits of q)
so that w' = 8 d (v - 16) + d ql exactly.

Bound copy of an N x K Q8_0 matrix (K a multiple of 256, nb = K / 32 blocks
per row): per row, 22 nb bytes in three planes, rows back to back, then one
fp32 per row:
    d plane       nb x fp16, the Q8_0 block scales (bit copies), little-endian
    fifth bits    nb x uint32 little-endian, bit j = bit 4 of v_j
    nibbles       nb x 16 bytes, byte j = (v_j & 15) | (v_{j+16} & 15) << 4
    E_n           after all rows: N x fp32 little-endian, the smallest fp32
                  that is >= ||e_n||_2, e_j = d_b (ql_j - 3.5) over the row
The planes hold 22 of Q8_0's 34 bytes per block (65 %).

Bounds for activations x (fp16, one column), per row n, in real arithmetic:
    yhat_n = sum_b d_b [ 8 sum_j (v_j - 16) x_j + 3.5 sum_j x_j ]
             (the low part replaced by the middle of its range)
    y_n - yhat_n = sum_j e_j x_j, so |y_n - yhat_n| <= ||e_n||_2 ||x||_2
             (Cauchy-Schwarz) <= r_n = E_n ||x||_2
    T_n    = sum_b |d_b| sum_j |x_j|
    s_n    = T_n / 4 + r_n / 256 + 2^-80   (room for fp32 rounding on the
             GPU, where yhat and the exact scores are fp32 sums)
    u_n = yhat_n + r_n + s_n  >=  y_n  >=  l_n = yhat_n - r_n - s_n
Pivot: c, the row with the largest l (lowest index on ties).
Shortlist: the rows n with u_n >= y_c. Any other row scores below row c, so it
is not the argmax; ties with the maximum are kept (u_n >= y_n = max >= y_c).
Result: the argmax of y over the shortlist (lowest index on ties), which is the
argmax over all N rows.
"""
from __future__ import annotations

import math

import numpy as np

from . import formats as F
from . import ref as R

SPLIT_CENTRE = 3.5      # middle of the low part's range 0..7
ABS_SLACK = 2.0 ** -80


def bound_copy_bytes(n: int, k: int) -> int:
    if n <= 0 or k <= 0 or k % 256:
        raise ValueError("need N > 0 and K a positive multiple of 256")
    return n * (22 * (k // 32) + 4)


def split_quants(q: np.ndarray):
    """int8 quants -> (v 0..31, ql 0..7) with q = 8 (v - 16) + ql."""
    qi = np.asarray(q).astype(np.int64)
    v = np.floor_divide(qi, 8) + 16
    ql = qi - 8 * (v - 16)
    return v.astype(np.uint8), ql.astype(np.uint8)


def _exact_sum_sign(terms) -> int:
    """Sign of the exact sum of doubles (math.fsum rounds the exact sum
    correctly, so its sign is exact)."""
    s = math.fsum(terms)
    return (s > 0) - (s < 0)


def residual_norm_up(d_row: np.ndarray, ql_row: np.ndarray) -> np.float32:
    """Smallest fp32 f >= sqrt(S), S = sum_b d_b^2 sum_j (ql_j - 3.5)^2, for one
    row (d_row fp16 [nb], ql_row [nb][32]). Every term d^2 (2 ql - 7)^2 / 4 is
    exact in fp64 (a 22-bit d^2 times an integer below 2^11, over 4), and f*f
    of an fp32 f is exact too, so f*f >= S is decided exactly through fsum."""
    d = np.asarray(d_row, np.float16).astype(np.float64)
    Q = ((2 * np.asarray(ql_row, np.int64) - 7) ** 2).sum(axis=-1)
    terms = [float(t) for t in (d * d) * (Q.astype(np.float64) / 4.0)]
    S = math.fsum(terms)
    if not math.isfinite(S):
        raise ValueError("non-finite residual norm")
    neg = [-t for t in terms]

    def covers(f):
        ff = float(f)
        return _exact_sum_sign([ff * ff] + neg) >= 0

    f = np.float32(math.sqrt(S))
    up, down = np.float32(np.inf), np.float32(0.0)
    while not covers(f):
        f = np.nextafter(f, up)
    while f > 0 and covers(np.nextafter(f, down)):
        f = np.nextafter(f, down)
    return np.float32(f)


def encode_bound_copy(q8_fields: dict) -> np.ndarray:
    """Q8_0 block fields (d fp16 [N][nb], q int8 [N][nb][32]) -> bound copy
    bytes (uint8 [bound_copy_bytes(N, K)])."""
    d = np.asarray(q8_fields["d"], np.float16)
    q = np.asarray(q8_fields["q"], np.int8)
    n, nb, _ = q.shape
    if nb % 8:
        raise ValueError("K must be a multiple of 256")
    if not np.all(np.isfinite(d)):
        raise ValueError("non-finite block scale")
    v, ql = split_quants(q)
    d_plane = F._f16_bytes(d).reshape(n, 2 * nb)
    fifth = F._high_bits(v).reshape(n, 4 * nb)
    nib = F._nibbles(v & 0x0F).reshape(n, 16 * nb)
    rows = np.concatenate([d_plane, fifth, nib], axis=1)
    E = np.array([residual_norm_up(d[i], ql[i]) for i in range(n)], dtype="<f4")
    return np.concatenate([rows.reshape(-1), E.view(np.uint8)])


def decode_bound_copy(buf: np.ndarray, n: int, k: int) -> dict:
    """Bound copy bytes -> {d fp16 [N][nb], v uint8 [N][nb][32], E fp32 [N]}."""
    nb = k // 32
    b = np.asarray(buf, np.uint8)
    assert b.size == bound_copy_bytes(n, k)
    rows = b[: n * 22 * nb].reshape(n, 22 * nb)
    d = F._bytes_f16(rows[:, : 2 * nb].reshape(n, nb, 2))
    fifth = F._unhigh_bits(rows[:, 2 * nb: 6 * nb].reshape(n, nb, 4))
    low = F._unnibble(rows[:, 6 * nb:].reshape(n, nb, 16))
    v = (low | (fifth << 4)).astype(np.uint8)
    E = b[n * 22 * nb:].view("<f4").astype(np.float32)
    return {"d": d, "v": v, "E": E}


def bound_terms(bound: dict, x16: np.ndarray) -> dict:
    """yhat, r, T, s, u, l per row (fp64) for one fp16 column x16 [K]."""
    x = np.asarray(x16, np.float16).astype(np.float64).reshape(-1)
    d = bound["d"].astype(np.float64)                          # [N, nb]
    v = bound["v"].astype(np.float64) - 16.0                   # [N, nb, 32]
    n, nb, _ = v.shape
    xb = x.reshape(nb, 32)
    hi = np.einsum("nbj,bj->nb", v, xb)                        # sum_j (v - 16) x
    sx = xb.sum(axis=1)                                        # sum_j x per block
    yhat = (d * (8.0 * hi + SPLIT_CENTRE * sx[None, :])).sum(axis=1)
    xnorm = math.sqrt(math.fsum(float(t) for t in x * x))
    r = bound["E"].astype(np.float64) * xnorm
    T = (np.abs(d) * np.abs(xb).sum(axis=1)[None, :]).sum(axis=1)
    s = T / 4.0 + r / 256.0 + ABS_SLACK
    return {"yhat": yhat, "r": r, "T": T, "s": s, "u": yhat + r + s, "l": yhat - r - s}


def shortlist_argmax(q8_fields: dict, bound: dict, x16: np.ndarray) -> dict:
    """The method step by step: bounds, pivot, shortlist, exact scores of the
    shortlisted rows, their argmax. Exact scores are oracle GEMV rows (fp64)."""
    t = bound_terms(bound, x16)
    c = int(R.argmax_lowest(t["l"]))
    y, _ = R.gemv("q8_0", q8_fields, np.asarray(x16)[None, :])   # exact scores (only kept rows are used)
    tau = float(y[0, c])
    keep = ~(t["u"] < tau)
    idx = np.flatnonzero(keep)
    best = int(idx[int(R.argmax_lowest(y[0, idx]))])
    return {"index": best, "pivot": c, "tau": tau, "keep": keep, "terms": t}
