"""Block formats, quantizer and dequantizer — oracle side (TEST INFRASTRUCTURE).

Every format cuts each row of an fp32 weight matrix ``W[N][K]`` into blocks of
32 consecutive weights along K and stores one block as a fixed number of bytes.
A packed row is its K/32 blocks back to back; a packed matrix is its rows back
to back (no padding).

Q8_0 (34 bytes): fp16 scale ``d`` then 32 int8 quants.
    d = fp16(max_j |w_j| / 127)          (fp32 divide, then fp16 round-to-nearest-even)
    q_j = clamp(round(w_j / d), -127, 127), or 0 for every j when d == 0
    dequantized weight w' = d * q
Q4_0 (18 bytes): fp16 scale ``d`` then 16 bytes of 4-bit quants.
    m = w_i for the FIRST index i that maximises |w_i| (the signed maximum)
    d = fp16(m / -8)
    q_j = clamp(round(w_j / d) + 8, 0, 15), or 8 for every j when d == 0
    w' = d * (q - 8)
affine4 gs32 (20 bytes): fp16 scale ``s``, fp16 bias ``b``, 16 bytes of quants.
    lo = min_j w_j, hi = max_j w_j   (first index on ties, so the sign of a zero is kept)
    s = fp16((hi - lo) / 15), b = fp16(lo)
    q_j = clamp(round((w_j - b) / s), 0, 15), or 0 for every j when s == 0
    w' = s * q + b
Q5_0 (22 bytes): fp16 scale ``d``, 4 bytes of fifth bits, 16 bytes of low nibbles.
    m = w_i for the FIRST index i that maximises |w_i| (the signed maximum)
    d = fp16(m / -16)
    q_j = clamp(round(w_j / d) + 16, 0, 31), or 16 for every j when d == 0
    w' = d * (q - 16)
Q5_1 (24 bytes): fp16 scale ``d``, fp16 minimum ``m``, 4 bytes of fifth bits,
16 bytes of low nibbles.
    lo = min_j w_j, hi = max_j w_j   (first index on ties)
    d = fp16((hi - lo) / 31), m = fp16(lo)
    q_j = clamp(round((w_j - m) / d), 0, 31), or 0 for every j when d == 0
    w' = d * q + m
All 4-bit nibble areas keep element j in the low nibble of byte j and element
j+16 in the high nibble (the 5-bit formats keep the low four bits of q there);
the 5-bit formats keep bit 4 of q_j in bit j of a little-endian 32-bit word
ahead of the nibbles. Scales and biases are little-endian fp16 ahead of the
quants.

Readings of points the definitions leave open (each is pinned by a hand-worked
block in tests/golden/):
* ``round`` is round-half-away-from-zero (C ``round``), evaluated exactly.
* ``q`` is computed with the STORED fp16 scale/bias (the same symbol names the
  stored value in ``w' = d*q``), after an fp32 subtraction/division.
* Zero or underflowing scales give q = 0 (Q8_0, affine4) or q = 8 (Q4_0).
* Non-finite weights, or a scale/bias that overflows fp16, are rejected.

The 4-bit formats are the ones the Kipp README, "How fast" contrasts (affine4
carries a bias term, Q4_0 is scale-only); Q8_0, Q4_0, Q5_0 and Q5_1 are among
the GGUF weight formats the Kinetic docs, "Supported models" list. The pages
print no layout or quantizer for any of them: the 5-bit definitions above are
this library's reading (Q5_0 is Q4_0 with sixteen levels either side of zero,
Q5_1 is affine4 with 31 steps, each with the fifth bits in a word of their
own), with the same rounding, tie and zero-scale rules as the 4-bit formats.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
BLOCK_BYTES = {"q8_0": 34, "q4_0": 18, "affine4": 20, "q5_0": 22, "q5_1": 24}
FORMATS = tuple(BLOCK_BYTES)


def packed_bytes(fmt: str, n: int, k: int) -> int:
    if fmt not in BLOCK_BYTES:
        raise ValueError(f"unknown format {fmt!r}")
    if n < 0 or k < 0 or k % BLOCK:
        raise ValueError("need n >= 0, k >= 0, k % 32 == 0")
    return n * (k // BLOCK) * BLOCK_BYTES[fmt]


def round_half_away(v) -> np.ndarray:
    """Round half away from zero, exactly. ``v`` is fp32 (or exact in fp64);
    the fp64 difference v - trunc(v) is exact, so the comparison with 0.5 is."""
    v = np.asarray(v, dtype=np.float64)
    t = np.trunc(v)
    frac = np.abs(v - t)
    return t + np.sign(v) * (frac >= 0.5)


def to_f16(v32) -> np.ndarray:
    """fp32 -> fp16, round to nearest even, subnormals kept (numpy's cast)."""
    return np.asarray(v32, dtype=np.float32).astype(np.float16)


def _blocks(W: np.ndarray) -> np.ndarray:
    W = np.asarray(W)
    if W.dtype != np.float32:
        raise TypeError("weights must be float32")
    if W.ndim != 2 or W.shape[1] % BLOCK:
        raise ValueError("weights must be [N][K] with K % 32 == 0")
    if not np.all(np.isfinite(W)):
        raise ValueError("non-finite weight")
    n, k = W.shape
    return W.reshape(n, k // BLOCK, BLOCK)


def _first_index_value(B: np.ndarray, key: np.ndarray, pick_max: bool) -> np.ndarray:
    """Value of B at the first index (along the last axis) where ``key`` is
    extremal. np.argmax/np.argmin return the first occurrence."""
    idx = np.argmax(key, axis=-1) if pick_max else np.argmin(key, axis=-1)
    return np.take_along_axis(B, idx[..., None], axis=-1)[..., 0]


def _check_finite16(*arrs):
    for a in arrs:
        if not np.all(np.isfinite(a.astype(np.float32))):
            raise ValueError("scale or bias overflows fp16")


def quantize(fmt: str, W: np.ndarray) -> dict:
    """Quantize fp32 W[N][K]. Returns the block fields:
    q8_0: {"d": f16[N,B], "q": int8[N,B,32]}
    q4_0: {"d": f16[N,B], "q": uint8[N,B,32] (0..15)}
    affine4: {"s": f16[N,B], "b": f16[N,B], "q": uint8[N,B,32] (0..15)}
    q5_0: {"d": f16[N,B], "q": uint8[N,B,32] (0..31)}
    q5_1: {"d": f16[N,B], "m": f16[N,B], "q": uint8[N,B,32] (0..31)}
    with B = K/32."""
    X = _blocks(W)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        if fmt == "q8_0":
            a = np.max(np.abs(X), axis=-1)                       # fp32
            d = to_f16(a / np.float32(127.0))                    # fp32 divide, fp16 RNE
            _check_finite16(d)
            d32 = d.astype(np.float32)
            ratio = X / d32[..., None]                           # fp32 divide
            q = np.clip(round_half_away(ratio), -127, 127)
            q = np.where((d32 == 0)[..., None], 0, q).astype(np.int8)
            return {"d": d, "q": q}
        if fmt == "q4_0":
            m = _first_index_value(X, np.abs(X), pick_max=True)  # signed max
            d = to_f16(m / np.float32(-8.0))
            _check_finite16(d)
            d32 = d.astype(np.float32)
            ratio = X / d32[..., None]
            q = np.clip(round_half_away(ratio) + 8, 0, 15)
            q = np.where((d32 == 0)[..., None], 8, q).astype(np.uint8)
            return {"d": d, "q": q}
        if fmt == "affine4":
            lo = _first_index_value(X, X, pick_max=False)
            hi = _first_index_value(X, X, pick_max=True)
            s = to_f16((hi - lo) / np.float32(15.0))             # fp32 subtract, divide
            b = to_f16(lo)
            _check_finite16(s, b)
            s32 = s.astype(np.float32)
            b32 = b.astype(np.float32)
            ratio = (X - b32[..., None]) / s32[..., None]        # fp32 subtract, divide
            q = np.clip(round_half_away(ratio), 0, 15)
            q = np.where((s32 == 0)[..., None], 0, q).astype(np.uint8)
            return {"s": s, "b": b, "q": q}
        if fmt == "q5_0":
            m = _first_index_value(X, np.abs(X), pick_max=True)  # signed max
            d = to_f16(m / np.float32(-16.0))
            _check_finite16(d)
            d32 = d.astype(np.float32)
            ratio = X / d32[..., None]
            q = np.clip(round_half_away(ratio) + 16, 0, 31)
            q = np.where((d32 == 0)[..., None], 16, q).astype(np.uint8)
            return {"d": d, "q": q}
        if fmt == "q5_1":
            lo = _first_index_value(X, X, pick_max=False)
            hi = _first_index_value(X, X, pick_max=True)
            d = to_f16((hi - lo) / np.float32(31.0))
            m = to_f16(lo)
            _check_finite16(d, m)
            d32 = d.astype(np.float32)
            m32 = m.astype(np.float32)
            ratio = (X - m32[..., None]) / d32[..., None]
            q = np.clip(round_half_away(ratio), 0, 31)
            q = np.where((d32 == 0)[..., None], 0, q).astype(np.uint8)
            return {"d": d, "m": m, "q": q}
    raise ValueError(f"unknown format {fmt!r}")


def _nibbles(q: np.ndarray) -> np.ndarray:
    """uint8[..., 32] quants (0..15) -> uint8[..., 16] bytes, element j in the
    low nibble of byte j and element j+16 in the high nibble."""
    return (q[..., :16] | (q[..., 16:] << 4)).astype(np.uint8)


def _unnibble(nb: np.ndarray) -> np.ndarray:
    return np.concatenate([nb & 0x0F, nb >> 4], axis=-1).astype(np.uint8)


def _high_bits(q: np.ndarray) -> np.ndarray:
    """uint8[..., 32] 5-bit quants -> uint8[..., 4]: bit j of the
    little-endian 32-bit word is bit 4 of q_j."""
    h = ((q.astype(np.uint64) >> 4) & 1) << np.arange(32, dtype=np.uint64)
    word = h.sum(axis=-1).astype(np.uint32)
    return np.stack([((word >> (8 * i)) & 0xFF).astype(np.uint8) for i in range(4)], axis=-1)


def _unhigh_bits(b4: np.ndarray) -> np.ndarray:
    word = sum(b4[..., i].astype(np.uint32) << (8 * i) for i in range(4))
    return ((word[..., None] >> np.arange(32, dtype=np.uint32)) & 1).astype(np.uint8)


def _f16_bytes(h: np.ndarray) -> np.ndarray:
    u = h.astype(np.float16).view(np.uint16)
    return np.stack([(u & 0xFF).astype(np.uint8), (u >> 8).astype(np.uint8)], axis=-1)


def _bytes_f16(b2: np.ndarray) -> np.ndarray:
    u = b2[..., 0].astype(np.uint16) | (b2[..., 1].astype(np.uint16) << 8)
    return u.view(np.float16)


def encode(fmt: str, fields: dict) -> np.ndarray:
    """Block fields -> packed bytes uint8[N, B * block_bytes]."""
    if fmt == "q8_0":
        parts = [_f16_bytes(fields["d"]), fields["q"].view(np.uint8)]
    elif fmt == "q4_0":
        parts = [_f16_bytes(fields["d"]), _nibbles(fields["q"])]
    elif fmt == "affine4":
        parts = [_f16_bytes(fields["s"]), _f16_bytes(fields["b"]), _nibbles(fields["q"])]
    elif fmt == "q5_0":
        parts = [_f16_bytes(fields["d"]), _high_bits(fields["q"]), _nibbles(fields["q"] & 0x0F)]
    elif fmt == "q5_1":
        parts = [_f16_bytes(fields["d"]), _f16_bytes(fields["m"]), _high_bits(fields["q"]),
                 _nibbles(fields["q"] & 0x0F)]
    else:
        raise ValueError(f"unknown format {fmt!r}")
    blk = np.concatenate(parts, axis=-1)
    n, nb, bb = blk.shape
    assert bb == BLOCK_BYTES[fmt]
    return np.ascontiguousarray(blk.reshape(n, nb * bb))


def decode(fmt: str, packed: np.ndarray, n: int, k: int) -> dict:
    """Packed bytes -> block fields (inverse of encode)."""
    bb = BLOCK_BYTES[fmt]
    blk = np.asarray(packed, dtype=np.uint8).reshape(n, k // BLOCK, bb)
    if fmt == "q8_0":
        return {"d": _bytes_f16(blk[..., 0:2]), "q": blk[..., 2:34].view(np.int8)}
    if fmt == "q4_0":
        return {"d": _bytes_f16(blk[..., 0:2]), "q": _unnibble(blk[..., 2:18])}
    if fmt == "affine4":
        return {"s": _bytes_f16(blk[..., 0:2]), "b": _bytes_f16(blk[..., 2:4]),
                "q": _unnibble(blk[..., 4:20])}
    if fmt == "q5_0":
        return {"d": _bytes_f16(blk[..., 0:2]),
                "q": (_unnibble(blk[..., 6:22]) | (_unhigh_bits(blk[..., 2:6]) << 4)).astype(np.uint8)}
    if fmt == "q5_1":
        return {"d": _bytes_f16(blk[..., 0:2]), "m": _bytes_f16(blk[..., 2:4]),
                "q": (_unnibble(blk[..., 8:24]) | (_unhigh_bits(blk[..., 4:8]) << 4)).astype(np.uint8)}
    raise ValueError(f"unknown format {fmt!r}")


def pack(fmt: str, W: np.ndarray) -> np.ndarray:
    return encode(fmt, quantize(fmt, W))


def dequantize(fmt: str, fields: dict, rows: slice | None = None) -> np.ndarray:
    """Block fields -> fp64 W'[N][K] (optionally a row slice)."""
    sl = rows if rows is not None else slice(None)
    q = fields["q"][sl].astype(np.float64)
    if fmt == "q8_0":
        w = fields["d"][sl].astype(np.float64)[..., None] * q
    elif fmt == "q4_0":
        w = fields["d"][sl].astype(np.float64)[..., None] * (q - 8.0)
    elif fmt == "affine4":
        w = (fields["s"][sl].astype(np.float64)[..., None] * q
             + fields["b"][sl].astype(np.float64)[..., None])
    elif fmt == "q5_0":
        w = fields["d"][sl].astype(np.float64)[..., None] * (q - 16.0)
    elif fmt == "q5_1":
        w = (fields["d"][sl].astype(np.float64)[..., None] * q
             + fields["m"][sl].astype(np.float64)[..., None])
    else:
        raise ValueError(f"unknown format {fmt!r}")
    n, nb, _ = w.shape
    return w.reshape(n, nb * BLOCK)


def rows_of(fields: dict) -> int:
    return fields["q"].shape[0]

