"""GPU tests of kq_gemv_ws, the K split of the matrix-core teams kernel into
a caller's workspace (partial sums per split, then a fixed-order sum): parity
with the fp64 oracle on every format, ragged rows, rows of 2-byte-aligned
blocks and forced split counts; run-to-run determinism; and the plain kq_gemv
result where no split applies."""
import numpy as np
import pytest

import block_quantized_gemv_kq_amd as kq
from oracle import ref as R
from synth import inputs as S
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

FMTS = ("q8_0", "q4_0", "affine4", "q5_0", "q5_1")


def _case(fmt, N, K, M, seed):
    W = S.weights((88, seed, N, K), N, K)
    x = S.activations((88, seed, K), K, M)
    packed, fields = U.quantize_both(fmt, W)
    return packed, fields, x


def _gemv_ws(fmt, Wd, x, N, K):
    M = x.shape[0]
    need = kq.kq_gemv_workspace_bytes(fmt, N, K, M)
    ws = U.empty_dev(((need + 15) // 4 + 4,)) if need else None
    if ws is not None:
        ws.fill_(float("nan"))          # partials must be written before they are summed
    xd = U.to_dev(x)
    y = U.empty_dev((M, N))
    y.fill_(float("nan"))
    kq.kq_gemv_ws(fmt, Wd, xd, y, N, K, M, ws, need)
    return U.to_host(y), need


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(2560, 9728), (77, 9728), (300, 6176), (33, 8192)])
@pytest.mark.parametrize("M", (4, 8, 13, 16))
@pytest.mark.parametrize("xdma", ("0", "1"))
def test_split_parity(fmt, N, K, M, xdma):
    """xdma: x of each split by DMA into column-major LDS, or through registers."""
    packed, fields, x = _case(fmt, N, K, M, 1)
    Wd = U.to_dev(packed)
    with U.tuning({"mfma_xdma": xdma}):
        y, need = _gemv_ws(fmt, Wd, x, N, K)
        y2, _ = _gemv_ws(fmt, Wd, x, N, K)
    assert need > 0, "this shape is expected to split"
    yr, ad = R.gemv(fmt, fields, x)
    U.assert_parity(y, yr, ad, f"{fmt} split N={N} K={K} M={M} xdma={xdma}")
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), "not deterministic run to run"


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("splits", ("2", "3", "5", "8"))
@pytest.mark.parametrize("N,K,M", [(40, 2048, 8), (130, 4160, 5), (16, 1024, 16)])
@pytest.mark.parametrize("xdma", ("0", "1"))
def test_forced_split_counts(fmt, splits, N, K, M, xdma):
    """Any split count (uneven group ranges, one or two groups per split,
    ragged rows, a partial last group) meets the bar, with x of each split
    staged through registers or by DMA; where one split's x would need more
    staging threads than its workgroup has, the call does not split
    (workspace 0) and is kq_gemv."""
    packed, fields, x = _case(fmt, N, K, M, 2)
    Wd = U.to_dev(packed)
    with U.tuning({"mfma_split": splits, "mfma_xdma": xdma}):
        y, need = _gemv_ws(fmt, Wd, x, N, K)
    assert need in (0, int(splits) * M * N * 4)
    if (N, K, M, splits) != (16, 1024, 16, "8"):
        assert need > 0
    yr, ad = R.gemv(fmt, fields, x)
    U.assert_parity(y, yr, ad, f"{fmt} {splits} splits N={N} K={K} M={M}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K,M", [(2560, 4096, 8), (19456, 2560, 8), (2560, 9728, 1), (333, 9728, 32)])
def test_no_split_is_kq_gemv(fmt, N, K, M):
    """Where kq_gemv_workspace_bytes is 0 the call is kq_gemv, bit for bit."""
    assert kq.kq_gemv_workspace_bytes(fmt, N, K, M) == 0
    packed, fields, x = _case(fmt, N, K, M, 3)
    Wd = U.to_dev(packed)
    y, _ = _gemv_ws(fmt, Wd, x, N, K)
    y0 = U.gemv_gpu(fmt, Wd, x, N, K)
    assert np.array_equal(y.view(np.uint32), y0.view(np.uint32))
