"""Host models of index arithmetic in the matrix-core kernels (no GPU): the
small integer division, and the column-major x staging by DMA (below).

The division: the teams and K-chunked kernels split a workgroup's wave index by the waves per
tile, and a K split's group range by the split count, as
floor((a + 1/2) * rcp(b)) in fp32 instead of an integer division sequence.
The quotient (a + 1/2) / b lies at least 1 / (2 b) from an integer; the test
checks exhaustively that fp32 rounding of the sum and the product, with the
hardware reciprocal anywhere within 2 ulp of 1 / b, never moves it across one,
for every a the kernels can pass (wave < 16; split bound at most
8 x 2^20 / 128 = 2^16) and a margin beyond.
"""
import numpy as np

A_MAX = 1 << 17          # twice the largest argument the kernels pass
B_MAX = 16               # waves per tile, K splits (at most 8)


def _div_small_model(a, b, ulps):
    r = np.float32(1.0) / np.float32(b)
    r = (r.view(np.int32) + np.int32(ulps)).view(np.float32)
    t = (a.astype(np.float32) + np.float32(0.5)) * r      # fp32 sum and product, round to nearest
    assert t.dtype == np.float32
    return np.trunc(t).astype(np.int64)


def test_div_small_exact_for_every_argument():
    a = np.arange(A_MAX + 1, dtype=np.int64)
    for b in range(1, B_MAX + 1):
        want = a // b
        for ulps in (-2, -1, 0, 1, 2):
            got = _div_small_model(a, b, ulps)
            bad = np.nonzero(got != want)[0]
            assert bad.size == 0, (b, ulps, int(a[bad[0]]))


def test_model_catches_a_truncated_quotient():
    """Without the half offset the same model fails (a multiple of b times a
    reciprocal rounded down lands just below the integer), so the check above
    is not vacuous."""
    a = np.arange(1, 4096, dtype=np.int64)
    b = 3
    r = np.float32(1.0) / np.float32(b)
    r = (r.view(np.int32) - np.int32(1)).view(np.float32)
    t = np.trunc(a.astype(np.float32) * r).astype(np.int64)
    assert np.any(t != a // b)


# ----------------------------------------------------------------------------
# Host model of the matrix-core teams kernel's column-major x staging by DMA:
# piece p (16 bytes, x[c][8 (k8_0 + p) .. +7]) of column c at slot
# c P + (p ^ (c & 15)), P = 16 pieces per 4-block group; a wave instruction
# fills 64 consecutive slots, and lane (n, g) of an operand read takes
# x[c][32 b + 4 g .. +3] and x[c][32 b + 16 + 4 g .. +3] of block b (column
# c = min(n, M - 1)) as two 8-byte halves.

def _stage_cm(M, ngroups):
    """slot -> (column, piece) as the staging loop writes it (each slot once)."""
    P = 16 * ngroups
    seen = {}
    for base in range(0, M * P, 64):              # one wave instruction per run
        for lane in range(64):
            s = base + lane
            if s >= M * P:
                continue
            c = s // P
            p = (s - c * P) ^ (c & 15)
            assert 0 <= p < P
            assert s not in seen
            seen[s] = (c, p)
    assert len(seen) == M * P
    return seen


def test_cm_staging_covers_every_piece_once():
    for M in (1, 2, 3, 4, 5, 8, 13, 16):
        for ngroups in (1, 2, 19, 20, 32):
            slots = _stage_cm(M, ngroups)
            assert sorted(slots.values()) == [(c, p) for c in range(M) for p in range(16 * ngroups)]


def test_cm_operand_reads_find_their_elements():
    """Every operand half a lane reads holds the x elements the matrix-core
    product pairs with that lane group's weights."""
    for M in (1, 4, 5, 8, 16):
        ngroups = 3
        P = 16 * ngroups
        slots = _stage_cm(M, ngroups)
        for b in range(4 * ngroups):
            for lane in range(64):
                n, g = lane & 15, lane >> 4
                c = min(n, M - 1)
                for part, first in ((0, 32 * b + 4 * g), (1, 32 * b + 16 + 4 * g)):
                    p0 = 4 * b + 2 * part + (g >> 1)
                    slot = c * P + (p0 ^ (c & 15))
                    col, piece = slots[slot]
                    assert col == c
                    # bytes 8 (g & 1) .. +7 of the piece: elements 8 piece + 4 (g & 1) .. +3
                    assert 8 * piece + 4 * (g & 1) == first


def test_cm_operand_reads_use_distinct_bank_groups():
    """The 16 lanes of one lane group read 16 different columns' halves at one
    block: with 16-byte slots over 64 four-byte banks, their 8-byte reads fall
    in distinct 16-byte bank groups (column stride P is a multiple of 16
    slots, the XOR with the column spreads them)."""
    for ngroups in (2, 20, 32):
        P = 16 * ngroups
        for b in range(4 * ngroups):
            for g in range(4):
                for part in (0, 1):
                    p0 = 4 * b + 2 * part + (g >> 1)
                    groups = [((c * P + (p0 ^ (c & 15))) % 16) for c in range(16)]
                    assert len(set(groups)) == 16
