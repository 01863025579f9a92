"""GPU parity of kq_gemv against the fp64 oracle, through the C ABI.

Bar: |y - y_ref| <= 2e-3 * sum|w'x| + 1e-6 per output, plus closed-form
probes (unit vectors give w' exactly, y(2x) == 2 y(x) bitwise), run-to-run
bitwise determinism, and row/column independence.
"""
import numpy as np
import pytest

import block_quantized_gemv_kq_amd as kq
from oracle import formats as F
from oracle import ref as R
from synth import inputs as S
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

FMTS = ("q8_0", "q4_0", "affine4", "q5_0", "q5_1")
M_LIST = (1, 2, 3, 4, 7, 8, 9, 15, 16, 17, 32, 48, 64)


def _case(fmt, N, K, M, seed):
    W = S.weights((80, seed, N, K), N, K)
    x = S.activations((80, seed, K), K, M)
    packed, fields = U.quantize_both(fmt, W)
    return packed, fields, x


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", M_LIST)
def test_parity_small(fmt, M):
    N, K = 333, 1024                  # several tiles and a ragged tail
    packed, fields, x = _case(fmt, N, K, M, 0)
    y = U.gemv_gpu(fmt, U.to_dev(packed), x, N, K)
    yr, ad = R.gemv(fmt, fields, x)
    U.assert_parity(y, yr, ad, f"{fmt} M={M}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(1, 64), (5, 128), (64, 256), (77, 2560), (130, 4096), (41, 9728),
                                 (3, 32), (9, 96), (17, 160)])
@pytest.mark.parametrize("M", (1, 5, 16))
def test_parity_shapes(fmt, N, K, M):
    packed, fields, x = _case(fmt, N, K, M, 1)
    y = U.gemv_gpu(fmt, U.to_dev(packed), x, N, K)
    yr, ad = R.gemv(fmt, fields, x)
    U.assert_parity(y, yr, ad, f"{fmt} N={N} K={K} M={M}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("K", (32, 96, 160, 2592))
@pytest.mark.parametrize("M", (2, 17))
def test_mfma_odd_block_counts(fmt, K, M):
    """Rows whose length is an odd number of blocks leave Q4_0/Q8_0/Q5_0
    blocks only 2-byte aligned; the matrix-core path realigns them in
    registers."""
    N = 45
    packed, fields, x = _case(fmt, N, K, M, 6)
    y = U.gemv_gpu(fmt, U.to_dev(packed), x, N, K)
    yr, ad = R.gemv(fmt, fields, x)
    U.assert_parity(y, yr, ad, f"{fmt} mfma N={N} K={K} M={M}")


@pytest.mark.parametrize("fmt", FMTS)
def test_generic_path_parity(fmt):
    N, K, M = 70, 1024, 3
    packed, fields, x = _case(fmt, N, K, M, 2)
    y = U.gemv_gpu(fmt, U.to_dev(packed), x, N, K, path="generic")
    yr, ad = R.gemv(fmt, fields, x)
    U.assert_parity(y, yr, ad, f"{fmt} generic")


@pytest.mark.parametrize("fmt", FMTS)
def test_unit_vectors_exact(fmt):
    """x = e_k gives y[n] = w'[n][k] exactly (w' is representable in fp32 for
    these value ranges): pins nibble order and block indexing."""
    N, K = 96, 512
    W = S.weights((81, 0, 0, 0), N, K)
    packed, fields = U.quantize_both(fmt, W)
    Wd = F.dequantize(fmt, fields)
    ks = [0, 1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 200, 255, 256, 500, 511]
    x = np.zeros((len(ks), K), np.float16)
    for i, k in enumerate(ks):
        x[i, k] = 1.0
    Wdev = U.to_dev(packed)
    for m0 in range(0, len(ks), 4):            # VALU path, 4 columns at a time
        y = U.gemv_gpu(fmt, Wdev, x[m0:m0 + 4], N, K)
        for i in range(y.shape[0]):
            assert np.array_equal(y[i].astype(np.float64), Wd[:, ks[m0 + i]]), (fmt, ks[m0 + i])
    y = U.gemv_gpu(fmt, Wdev, x, N, K)       # all columns in one call
    for i, k in enumerate(ks):
        assert np.array_equal(y[i].astype(np.float64), Wd[:, k]), (fmt, k, "M=16")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", (1, 3, 16))
def test_scale_by_two_bitwise_and_deterministic(fmt, M):
    N, K = 300, 2560
    packed, fields, x = _case(fmt, N, K, M, 3)
    Wdev = U.to_dev(packed)
    y1 = U.gemv_gpu(fmt, Wdev, x, N, K)
    y1b = U.gemv_gpu(fmt, Wdev, x, N, K)
    assert np.array_equal(y1.view(np.uint32), y1b.view(np.uint32)), "not deterministic"
    x2 = (x.astype(np.float32) * 2).astype(np.float16)
    y2 = U.gemv_gpu(fmt, Wdev, x2, N, K)
    assert np.array_equal(y2, 2 * y1)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", (2, 4, 8, 16))
def test_columns_match_single_column_runs(fmt, M):
    """Each column of an M-column call equals its own M=1 call within the
    tolerance (both are within it of the oracle; different M may take
    different kernels, so the summation order, and the last bits, differ)."""
    N, K = 200, 2048
    packed, fields, x = _case(fmt, N, K, M, 4)
    Wdev = U.to_dev(packed)
    y = U.gemv_gpu(fmt, Wdev, x, N, K)
    _, ad = R.gemv(fmt, fields, x)
    for m in range(M):
        y1 = U.gemv_gpu(fmt, Wdev, x[m:m + 1], N, K)
        assert np.all(np.abs(y[m] - y1[0]) <= 2 * R.tolerance(ad[m])), (fmt, m)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("path", ("lds", "valu", "generic", "mfma"))
@pytest.mark.parametrize("M", (1, 3))
def test_every_path_parity(fmt, path, M):
    """Each kernel path on the same shapes (the dispatcher would pick only one)."""
    for N, K in ((300, 2560), (17, 9728), (64, 4096)):
        packed, fields, x = _case(fmt, N, K, M, 5)
        y = U.gemv_gpu(fmt, U.to_dev(packed), x, N, K, path=path)
        yr, ad = R.gemv(fmt, fields, x)
        U.assert_parity(y, yr, ad, f"{fmt} {path} N={N} K={K} M={M}")


@pytest.mark.parametrize("fmt", FMTS)
def test_row_concatenation_bitwise(fmt):
    K = 1024
    Wa = S.weights((82, 0, 0, 0), 100, K)
    Wb = S.weights((82, 1, 0, 0), 61, K)
    x = S.activations((82, 0, 0), K, 2)
    pa = kq.kq_pack(fmt, Wa)
    pb = kq.kq_pack(fmt, Wb)
    pab = kq.kq_pack(fmt, np.concatenate([Wa, Wb]))
    assert np.array_equal(pab, np.concatenate([pa, pb]))
    ya = U.gemv_gpu(fmt, U.to_dev(pa), x, 100, K)
    yb = U.gemv_gpu(fmt, U.to_dev(pb), x, 61, K)
    yab = U.gemv_gpu(fmt, U.to_dev(pab), x, 161, K)
    assert np.array_equal(yab, np.concatenate([ya, yb], axis=1))


def test_single_q8_0_workload():
    """The single 1024 x 1024 Q8_0 GEMV (weights seed 0, activation seed 1)."""
    w = S.SINGLE_Q8_0
    W = S.weights(w.weight_seed, w.n, w.k)
    x = S.activation_column(w.act_seed, w.k)[None, :]
    packed, fields = U.quantize_both("q8_0", W)
    y = U.gemv_gpu("q8_0", U.to_dev(packed), x, w.n, w.k)
    yr, ad = R.gemv("q8_0", fields, x)
    ratio = U.assert_parity(y, yr, ad, "single q8_0")
    assert ratio < 1e-4
    assert int(np.argmax(y[0])) == int(R.argmax_lowest(yr[0]))


def test_zero_and_constant_weights():
    K = 256
    W = np.zeros((8, K), np.float32)
    W[1] = 0.5
    W[2] = -3.0
    W[3, ::3] = -0.0
    x = S.activations((83, 0, 0), K, 2)
    for fmt in FMTS:
        packed, fields = U.quantize_both(fmt, W)
        y = U.gemv_gpu(fmt, U.to_dev(packed), x, 8, K)
        yr, ad = R.gemv(fmt, fields, x)
        U.assert_parity(y, yr, ad, f"{fmt} constant rows")
        assert np.all(y[:, 0] == 0.0)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("variant", ("pers", "pers_tpw3", "teams", "teams_sx", "teams_x0", "teams_x1", "teams_xdma",
                                     "chunk", "chunk_whole", "direct"))
@pytest.mark.parametrize("N,K,M", [(1000, 2560, 8), (37, 96, 5), (300, 4128, 16), (16, 32, 2), (529, 640, 13),
                                   (300, 4128, 40), (77, 9728, 33)])
def test_mfma_variants_parity(fmt, variant, N, K, M):
    """Each matrix-core kernel (the dispatcher picks one by shape: persistent
    waves for many tiles, split-K teams with x staged in LDS with or without
    block sums, K-chunked staging for many columns or long rows, per-wave
    activation loads) on ragged rows, partial groups and odd block counts;
    pers_tpw3 gives each wave three tiles. Past 16 columns only the chunked
    and per-wave kernels apply; with fewer than 256 row tiles the chunked
    kernel runs one workgroup per 16 columns (chunk), or one for all columns
    of a tile (chunk_whole)."""
    packed, fields, x = _case(fmt, N, K, M, 9)
    env = {"mfma_variant": {"pers_tpw3": "pers", "teams_x0": "teams", "teams_x1": "teams",
                            "teams_xdma": "teams"}.get(variant, variant)}
    if variant == "pers_tpw3":
        env["mfma_pers_tpw"] = "3"
    if variant == "teams_x0":          # weights issued before x is written (the other load order)
        env["mfma_xf"] = "0"
    if variant == "teams_x1":          # x written before the weights are issued, at any grid size
        env["mfma_xf"] = "1"
    if variant == "teams_xdma":        # x by DMA into column-major LDS (without block sums), or through registers
        env["mfma_xdma"] = "1"
    with U.tuning(env):
        y = U.gemv_gpu(fmt, U.to_dev(packed), x, N, K, path="mfma")
        y2 = U.gemv_gpu(fmt, U.to_dev(packed), x, N, K, path="mfma")
    yr, ad = R.gemv(fmt, fields, x)
    U.assert_parity(y, yr, ad, f"{fmt} {variant} N={N} K={K} M={M}")
    assert np.array_equal(y, y2), "not deterministic run to run"


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("variant", ("teams", "teams_sx"))
@pytest.mark.parametrize("N,K,M", [(1000, 2560, 8), (37, 96, 5), (300, 4128, 16), (529, 640, 13), (2560, 4096, 8),
                                   (6144, 2560, 7), (160, 9728, 12), (1000, 2560, 4), (300, 4128, 3), (37, 96, 2),
                                   (6144, 2560, 4), (2560, 9728, 4)])
def test_teams_x_dma_same_bits(fmt, variant, N, K, M):
    """The teams kernel, with block sums in LDS or an MFMA against ones per
    block, gives the same bits whether x is staged by DMA in column-major
    order or through registers in operand order (the same operands, block
    sums, products and sums in the same order)."""
    packed, fields, x = _case(fmt, N, K, M, 19)
    Wd = U.to_dev(packed)
    with U.tuning({"mfma_variant": variant, "mfma_xdma": "1"}):
        y1 = U.gemv_gpu(fmt, Wd, x, N, K, path="mfma")
    with U.tuning({"mfma_variant": variant, "mfma_xdma": "0"}):
        y0 = U.gemv_gpu(fmt, Wd, x, N, K, path="mfma")
    yr, ad = R.gemv(fmt, fields, x)
    U.assert_parity(y1, yr, ad, f"{fmt} {variant} x by DMA N={N} K={K} M={M}")
    assert np.array_equal(y1.view(np.uint32), y0.view(np.uint32))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K,M", [(50, 2048, 17), (130, 1024, 64), (4000, 256, 48), (4096, 512, 33)])
def test_chunk_column_groups(fmt, N, K, M):
    """Past 16 columns the chunked kernel runs one workgroup per tile and 16
    columns below 256 row tiles (a grid y of column groups, the last one
    partial) and one per tile for all columns from 256 tiles on (4096 rows):
    parity with the oracle either way, and run-to-run determinism."""
    packed, fields, x = _case(fmt, N, K, M, 11)
    y = U.gemv_gpu(fmt, U.to_dev(packed), x, N, K, path="mfma")
    y2 = U.gemv_gpu(fmt, U.to_dev(packed), x, N, K, path="mfma")
    yr, ad = R.gemv(fmt, fields, x)
    U.assert_parity(y, yr, ad, f"{fmt} chunk column groups N={N} K={K} M={M}")
    assert np.array_equal(y, y2), "not deterministic run to run"


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K,M", [(6144, 2560, 1), (2560, 4096, 1), (2560, 9728, 1), (19456, 2560, 1), (333, 1024, 2),
                                   (77, 9728, 2), (1000, 640, 3), (151936 // 16, 2560, 1)])
def test_lds_x_dma_same_bits(fmt, N, K, M):
    """The one-column LDS kernel gives the same bits whether x goes through
    registers or is copied by DMA ahead of the weight loads (the same padded
    layout, block sums and products)."""
    packed, fields, x = _case(fmt, N, K, M, 23)
    Wd = U.to_dev(packed)
    with U.tuning({"lds_xdma": "1"}):
        y1 = U.gemv_gpu(fmt, Wd, x, N, K, path="lds")
    y0 = U.gemv_gpu(fmt, Wd, x, N, K, path="lds")
    yr, ad = R.gemv(fmt, fields, x)
    U.assert_parity(y1, yr, ad, f"{fmt} lds x by DMA N={N} K={K} M={M}")
    assert np.array_equal(y1.view(np.uint32), y0.view(np.uint32))


@pytest.mark.parametrize("fmt", ("q8_0", "q4_0", "affine4", "q5_0", "q5_1"))
@pytest.mark.parametrize("wpg", ("8", "12", "16"))
def test_lds_waves_per_workgroup(fmt, wpg):
    """The one-column LDS kernel at every workgroup size the launcher may pick:
    within the oracle's bar and bitwise equal to 4 waves per workgroup (each
    lane's sum and the per-workgroup staging do not depend on it)."""
    for N, K, g in ((333, 1024, None), (2560, 4096, None), (17, 9728, None), (300, 2560, "16"), (1, 64, None)):
        packed, fields, x = _case(fmt, N, K, 1, 13)
        Wd = U.to_dev(packed)
        extra = {"valu_g": g} if g else {}
        with U.tuning({"lds_wpg": wpg, **extra}):
            y = U.gemv_gpu(fmt, Wd, x, N, K, path="lds")
        with U.tuning({"lds_wpg": "4", **extra}):
            y4 = U.gemv_gpu(fmt, Wd, x, N, K, path="lds")
        yr, ad = R.gemv(fmt, fields, x)
        U.assert_parity(y, yr, ad, f"{fmt} wpg={wpg} N={N} K={K}")
        assert np.array_equal(y.view(np.uint32), y4.view(np.uint32)), (fmt, wpg, N, K)


@pytest.mark.parametrize("fmt", ("q8_0", "affine4"))
@pytest.mark.parametrize("N", (2560, 6144, 5000))
def test_lds_workgroup_size_argmax(fmt, N):
    """kq_gemv_argmax at one column where the launcher picks 12 waves per
    workgroup (2560 x 2560 affine4: two units per lane) or 4: y equals
    kq_gemv's, the index is the first maximum of y, and y meets the bar."""
    K = 2560
    packed, fields, x = _case(fmt, N, K, 1, 14)
    Wd = U.to_dev(packed)
    xd = U.to_dev(x)
    wsb = kq.kq_gemv_argmax_workspace_bytes(fmt, N, K, 1)
    ws = U.empty_dev(((max(wsb, 4) + 3) // 4,))
    y = U.empty_dev((1, N))
    out = U.empty_dev((1,), "int32")
    kq.kq_gemv_argmax(fmt, Wd, xd, y, N, K, 1, out, ws, wsb)
    yh = U.to_host(y)
    y1 = U.gemv_gpu(fmt, Wd, x, N, K)
    yr, ad = R.gemv(fmt, fields, x)
    U.assert_parity(yh, yr, ad, f"{fmt} balanced argmax N={N}")
    assert np.array_equal(yh.view(np.uint32), y1.view(np.uint32))
    assert int(U.to_host(out)[0]) == int(np.argmax(yh[0]))
