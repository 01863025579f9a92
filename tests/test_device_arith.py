"""Host model of the matrix-core kernels' small integer division (no GPU).

The teams and K-chunked kernels split a workgroup's wave index by the waves per
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
