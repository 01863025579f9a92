"""kq_gemv_argmax_noalloc through the C ABI: the allocation-free variant of
kq_gemv_argmax (partials in the library's static per-device scratch array).
Checked against kq_gemv_argmax with a caller workspace (y bit for bit, the
same argmax) and against the oracle, on two calls in a row where the second
is smaller (the scratch keeps the first call's contents), for the fused
one-column path and the two-pass path; and the host-side size check."""
import numpy as np
import pytest

import block_quantized_gemv_kq_amd as kq
from oracle import ref as R
from synth import inputs as S
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def _with_workspace(fmt, Wd, xd, N, K, M):
    y = U.empty_dev((M, N))
    out = U.empty_dev((M,), "int32")
    wsb = kq.kq_gemv_argmax_workspace_bytes(fmt, N, K, M)
    ws = U.empty_dev((wsb // 4 + 2,))
    kq.kq_gemv_argmax(fmt, Wd, xd, y, N, K, M, out, ws, wsb)
    return U.to_host(y), U.to_host(out)


def _noalloc(fmt, Wd, xd, N, K, M):
    y = U.empty_dev((M, N))
    y.fill_(float("nan"))
    out = U.empty_dev((M,), "int32")
    out.fill_(-7)
    kq.kq_gemv_argmax_noalloc(fmt, Wd, xd, y, N, K, M, out)
    return U.to_host(y), U.to_host(out)


# (fmt, N, K, M) of the first call, then a smaller second call
CASES = [
    (("q8_0", 40000, 2560, 1), ("q8_0", 3000, 1024, 1)),       # fused one-column path
    (("affine4", 20000, 2560, 1), ("affine4", 777, 2560, 1)),
    (("q4_0", 9000, 1024, 5), ("q4_0", 2100, 512, 3)),          # GEMV + two-pass argmax
    (("q8_0", 12000, 2560, 16), ("q8_0", 12000, 2560, 1)),
]


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_matches_workspace_entry(first, second):
    for i, (fmt, N, K, M) in enumerate((first, second)):
        print(f"noalloc call {i}: {fmt} N={N} K={K} M={M}", flush=True)
        W = S.weights((61, N, K, i), N, K)
        packed, fields = U.quantize_both(fmt, W)
        x = S.activations((62, N, K, i), K, M)
        Wd, xd = U.to_dev(packed), U.to_dev(x)
        y_ws, am_ws = _with_workspace(fmt, Wd, xd, N, K, M)
        y_na, am_na = _noalloc(fmt, Wd, xd, N, K, M)
        assert np.array_equal(y_na.view(np.uint32), y_ws.view(np.uint32)), "y differs from kq_gemv_argmax"
        assert np.array_equal(am_na, am_ws)
        yr, ad = R.gemv(fmt, fields, x)
        U.assert_parity(y_na, yr, ad, f"noalloc {fmt} {N}x{K} M={M}")
        gaps = R.top2_gap(yr)
        pinned = gaps > 4 * np.max(np.abs(y_na - yr), axis=1)
        assert np.all(am_na[pinned] == R.argmax_lowest(yr)[pinned])


def test_noalloc_rejects_shapes_beyond_the_scratch():
    """Checked on the host before any HIP call (fake device addresses)."""
    L = kq.lib()
    N = 5_000_000   # two-pass partials of 64 columns: 64 * 2442 * 8 B > 1 MiB
    st = L.kq_gemv_argmax_noalloc(0, 0x10000, 0x10000, 0x10000, N, 2560, 64, 0x10000, None)
    assert st == kq.KQ_ERR_ARG and "static scratch" in kq.last_error()
