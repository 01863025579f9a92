"""GPU parity at the size limits, through the C ABI:

* the longest rows the boundary accepts (K = KQ_MAX_K = 2^20 inputs) in every
  format, on the kernels that take them (register-x VALU at one to three
  columns, the K-chunked matrix-core kernel beyond), against the oracle;
* weights past 4 GiB in one call (2^21 Q8_0 rows of 2048, 2^22 affine4
  rows): 1024 seeded rows repeated on the device, so every repeat must give
  the first one's bits (a row offset or output index that wrapped at 32 bits
  would break that) and the first one is checked against the oracle, at one
  and at eight columns, and the argmax of the repeated output layer is the
  first maximum (lowest index on ties).
"""
import numpy as np
import pytest

import block_quantized_gemv_kq_amd as kq
from oracle import ref as R
from synth import inputs as S
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

FMTS = ("q8_0", "q4_0", "affine4", "q5_0", "q5_1")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", (1, 3, 8, 17))
def test_longest_rows(fmt, M):
    N, K = 5, kq.KQ_MAX_K
    W = S.weights((120, N, K), N, K)
    x = S.activations((120, K, M), K, M)
    packed, fields = U.quantize_both(fmt, W)
    del W
    y = U.gemv_gpu(fmt, U.to_dev(packed), x, N, K)
    yr, ad = R.gemv(fmt, fields, x)
    U.assert_parity(y, yr, ad, f"{fmt} N={N} K=2^20 M={M}")


def test_longest_rows_64_columns():
    fmt, N, K, M = "q4_0", 3, 1 << 20, 64
    W = S.weights((121, N, K), N, K)
    x = S.activations((121, K, M), K, M)
    packed, fields = U.quantize_both(fmt, W)
    del W
    y = U.gemv_gpu(fmt, U.to_dev(packed), x, N, K)
    yr, ad = R.gemv(fmt, fields, x)
    U.assert_parity(y, yr, ad, f"{fmt} N={N} K=2^20 M={M}")


@pytest.fixture(scope="module", params=[("q8_0", 2048, 1 << 21), ("affine4", 2048, 1 << 22)],
                ids=["q8_0", "affine4"])
def past_4gib(request):
    fmt, K, N = request.param
    torch = U.torch_cuda()
    base = 1024
    W = S.weights((122, kq.FORMATS[fmt], K), base, K)
    packed, fields = U.quantize_both(fmt, W)
    del W
    row = packed.reshape(base, -1)
    assert N * row.shape[1] > 4 << 30, "the matrix must pass 4 GiB"
    big = U.to_dev(row).repeat(N // base, 1)
    torch.cuda.synchronize()
    yield fmt, K, N, base, big, fields
    del big
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M", (1, 8))
def test_weights_past_4gib(past_4gib, M):
    fmt, K, N, base, big, fields = past_4gib
    x = S.activations((123, K, M), K, M)
    y = U.gemv_gpu(fmt, big, x, N, K)
    tiles = y.reshape(M, N // base, base)
    first = tiles[:, :1, :]
    assert np.array_equal(tiles.view(np.uint32), np.broadcast_to(first, tiles.shape).view(np.uint32)), \
        "a repeat of the first 1024 rows gave other bits"
    yr, ad = R.gemv(fmt, fields, x)
    U.assert_parity(np.ascontiguousarray(first[:, 0, :]), yr, ad, f"{fmt} past 4 GiB M={M}")


def test_argmax_past_4gib(past_4gib):
    fmt, K, N, base, big, fields = past_4gib
    x = S.activations((124, K, 1), K, 1)
    y = U.empty_dev((1, N))
    out = U.empty_dev((1,), "int32")
    wsb = kq.kq_gemv_argmax_workspace_bytes(fmt, N, K, 1)
    ws = U.empty_dev((wsb // 4 + 2,))
    kq.kq_gemv_argmax(fmt, big, U.to_dev(x), y, N, K, 1, out, ws, wsb)
    idx = int(U.to_host(out)[0])
    yg = U.to_host(y)[0]
    # every repeat ties with the first 1024 rows: the lowest index is among them
    assert idx < base and idx == int(R.argmax_lowest(yg)), idx
    yr, ad = R.gemv(fmt, fields, x)
    U.assert_parity(yg[None, :base], yr, ad, f"{fmt} argmax layer past 4 GiB")
    if float(R.top2_gap(yr[0])) > 4 * float(np.max(np.abs(yg[:base] - yr[0]))):
        assert idx == int(R.argmax_lowest(yr[0]))
