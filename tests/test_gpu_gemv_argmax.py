"""GPU tests of kq_gemv_argmax through the C ABI: the GEMV with the argmax of
every column, fused into the GEMV kernel for one column (partials per
workgroup, one reduction kernel) and as GEMV + kq_argmax beyond. Checked
against the oracle and against kq_gemv + kq_argmax (bit for bit) on small
shapes and on the 4B-shaped Q8_0 lm_head, and on planted ties and NaN rows
inside one workgroup and across workgroups."""
import numpy as np
import pytest

import block_quantized_gemv_kq_amd as kq
from oracle import ref as R
from synth import inputs as S
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def _gemv_argmax(fmt, Wdev, xd, N, K, M):
    y = U.empty_dev((M, N))
    out = U.empty_dev((M,), "int32")
    wsb = kq.kq_gemv_argmax_workspace_bytes(fmt, N, K, M)
    ws = U.empty_dev((wsb // 4 + 2,))
    kq.kq_gemv_argmax(fmt, Wdev, xd, y, N, K, M, out, ws, wsb)
    return U.to_host(y), U.to_host(out)


def _gemv_then_argmax(fmt, Wdev, xd, N, K, M):
    y = U.empty_dev((M, N))
    kq.kq_gemv(fmt, Wdev, xd, y, N, K, M)
    out = U.empty_dev((M,), "int32")
    wsb = kq.kq_argmax_workspace_bytes(N, M)
    ws = U.empty_dev((wsb // 4 + 2,))
    kq.kq_argmax(y, N, M, out, ws, wsb)
    return U.to_host(y), U.to_host(out)


@pytest.mark.parametrize("fmt", ("q8_0", "q4_0", "affine4"))
@pytest.mark.parametrize("N,K", [(1000, 1024), (37, 96), (4099, 2560), (150, 9728)])
@pytest.mark.parametrize("M", (1, 2, 3, 5))
def test_matches_gemv_then_argmax(fmt, N, K, M):
    W = S.weights((85, N, K), N, K)
    x = S.activations((85, K), K, M)
    packed, fields = U.quantize_both(fmt, W)
    Wdev, xd = U.to_dev(packed), U.to_dev(x)
    y1, a1 = _gemv_argmax(fmt, Wdev, xd, N, K, M)
    y2, a2 = _gemv_then_argmax(fmt, Wdev, xd, N, K, M)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    assert np.array_equal(a1, a2)
    yr, ad = R.gemv(fmt, fields, x)
    U.assert_parity(y1, yr, ad, f"{fmt} gemv_argmax N={N} K={K} M={M}")


def _q8_rows(N, K, seed):
    """Packed Q8_0 rows of small random weights (host bytes, [N][K/32*34])."""
    W = S.weights((86, seed, N, K), N, K)
    return kq.kq_pack("q8_0", W).reshape(N, -1).copy()


def _big_row(K):
    """A Q8_0 row with d = 1 and every q = 127 (each block: fp16 1.0, 32 x 0x7f)."""
    blk = np.zeros(34, np.uint8)
    blk[:2] = np.frombuffer(np.float16(1.0).tobytes(), np.uint8)
    blk[2:] = 127
    return np.tile(blk, K // 32)


@pytest.mark.parametrize("M", (1, 3))
def test_ties_and_nan_rows(M):
    """Rows 3, 7 (one workgroup) and 2700 (another) are the same large row:
    the lowest index wins. A NaN scale on row 3 makes its score NaN, which
    never wins, so row 7 does. Column m of x is all ones scaled by m + 1."""
    N, K = 5000, 256
    rows = _q8_rows(N, K, 0)
    big = _big_row(K)
    for r in (3, 7, 2700):
        rows[r] = big
    x = np.stack([np.full(K, np.float16(m + 1)) for m in range(M)]).view(np.uint16)
    xd = U.to_dev(x)
    _, am = _gemv_argmax("q8_0", U.to_dev(rows.reshape(-1)), xd, N, K, M)
    assert list(am) == [3] * M
    rows[3, :2] = np.frombuffer(np.float16(np.nan).tobytes(), np.uint8)
    y, am = _gemv_argmax("q8_0", U.to_dev(rows.reshape(-1)), xd, N, K, M)
    assert np.all(np.isnan(y[:, 3]))
    assert list(am) == [7] * M


@pytest.fixture(scope="module")
def lm_head_dev():
    st = S.QWEN3_4B_AFFINE4
    h = st.head
    W = S.weights(st.weight_seed(st.layers, 0), h.n, h.k)
    Wdev = U.to_dev(kq.kq_pack(h.fmt, W))
    del W
    return h, Wdev


@pytest.mark.parametrize("M", (1, 2, 3, 8))
def test_lm_head_shape(lm_head_dev, M):
    """The 4B-shaped Q8_0 lm_head (151936 x 2560; kq_gemv + kq_argmax at this
    shape are pinned to the oracle by the workload tests): the same scores,
    bit for bit, and the same argmax, fused (M = 1) or not."""
    h, Wdev = lm_head_dev
    xd = U.to_dev(S.activations((S.VERIFY_WORKLOAD_ID, 36, 0), h.k, M))
    y1, a1 = _gemv_argmax(h.fmt, Wdev, xd, h.n, h.k, M)
    y2, a2 = _gemv_then_argmax(h.fmt, Wdev, xd, h.n, h.k, M)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    assert np.array_equal(a1, a2)
