"""GPU tests of the 5-bit formats (Q5_0, Q5_1) through the C ABI: packer bytes
equal the oracle's (every case packs through kq_pack and checks), parity of
kq_gemv with the fp64 oracle on every kernel path these formats take (the
one-column LDS-staged and register-x kernels, the matrix-core kernels from 4
columns on, the generic kernel for 2-byte-aligned Q5_0 rows at one column),
unit vectors giving w' exactly (which
pins the fifth-bit and nibble order on the GPU), the output-layer argmax,
batch-invariant columns, and the routed-expert FFN."""
import numpy as np
import pytest

import block_quantized_gemv_kq_amd as kq
from oracle import formats as F
from oracle import ref as R
from synth import inputs as S
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

FMTS = ("q5_0", "q5_1")


def _case(fmt, N, K, M, seed):
    W = S.weights((86, seed, N, K), N, K)
    x = S.activations((86, seed, K), K, M)
    packed, fields = U.quantize_both(fmt, W)
    return packed, fields, x


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(333, 1024), (77, 2560), (130, 4096), (41, 9728), (5, 64), (3, 32), (9, 96),
                                 (17, 45056)])
@pytest.mark.parametrize("M", (1, 2, 3, 4, 8, 9, 16, 48))
def test_parity(fmt, N, K, M):
    packed, fields, x = _case(fmt, N, K, M, 1)
    y = U.gemv_gpu(fmt, U.to_dev(packed), x, N, K)
    yr, ad = R.gemv(fmt, fields, x)
    ratio = U.assert_parity(y, yr, ad, f"{fmt} N={N} K={K} M={M}")
    assert ratio < 1e-4


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("path", ("lds", "valu", "generic", "mfma"))
@pytest.mark.parametrize("M", (1, 3, 5))
def test_every_path(fmt, path, M):
    for N, K in ((300, 2560), (17, 9728), (64, 4096)):
        packed, fields, x = _case(fmt, N, K, M, 2)
        y = U.gemv_gpu(fmt, U.to_dev(packed), x, N, K, path=path)
        yr, ad = R.gemv(fmt, fields, x)
        U.assert_parity(y, yr, ad, f"{fmt} {path} N={N} K={K} M={M}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("path", (None, "valu", "generic", "mfma"))
def test_unit_vectors_exact(fmt, path):
    """x = e_k gives y[n] = w'[n][k] bit for bit: w' = d(q - 16) or dq + m is
    exact in fp32, so every fifth bit and nibble lands on its element."""
    N, K = 40, 128
    packed, fields, _ = _case(fmt, N, K, 1, 3)
    Wd = F.dequantize(fmt, fields)
    Wdev = U.to_dev(packed)
    for k in (0, 1, 15, 16, 17, 31, 32, 63, 64, 95, 127):
        x = np.zeros((1, K), np.float16)
        x[0, k] = 1.0
        y = U.gemv_gpu(fmt, Wdev, x, N, K, path=path)
        assert np.array_equal(y[0].astype(np.float64), Wd[:, k]), (fmt, path, k)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("variant", ("teams", "teams_sx", "pers", "chunk", "direct"))
def test_unit_vectors_exact_matrix_cores(fmt, variant):
    """Sixteen columns at once, column m = e_k for k over every element slot
    of a block (both nibble halves, every fifth-bit position) and block
    boundaries: each matrix-core kernel gives y[m][n] = w'[n][k_m] bit for bit
    (1024 + q and the fix-up terms are exact in fp32), so the fifth bits reach
    the right halves of the operand in every lane group."""
    N, K = 40, 128
    packed, fields, _ = _case(fmt, N, K, 1, 5)
    Wd = F.dequantize(fmt, fields)
    Wdev = U.to_dev(packed)
    for ks in ((0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15),
               (16, 17, 18, 19, 20, 21, 22, 23, 24, 25, 26, 27, 28, 29, 30, 31),
               (32, 47, 48, 63, 64, 79, 80, 95, 96, 100, 111, 112, 113, 119, 126, 127)):
        x = np.zeros((16, K), np.float16)
        for m, k in enumerate(ks):
            x[m, k] = 1.0
        with U.tuning({"mfma_variant": variant}):
            y = U.gemv_gpu(fmt, Wdev, x, N, K, path="mfma")
        for m, k in enumerate(ks):
            assert np.array_equal(y[m].astype(np.float64), Wd[:, k]), (fmt, variant, k)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", (1, 4))
def test_argmax(fmt, M):
    N, K = 50000, 1024
    packed, fields, x = _case(fmt, N, K, M, 4)
    Wdev, xd = U.to_dev(packed), U.to_dev(x)
    y = U.empty_dev((M, N))
    out = U.empty_dev((M,), "int32")
    wsb = kq.kq_gemv_argmax_workspace_bytes(fmt, N, K, M)
    ws = U.empty_dev((wsb // 4 + 2,))
    kq.kq_gemv_argmax(fmt, Wdev, xd, y, N, K, M, out, ws, wsb)
    yh, am = U.to_host(y), U.to_host(out)
    yr, ad = R.gemv(fmt, fields, x)
    U.assert_parity(yh, yr, ad, f"{fmt} argmax M={M}")
    gaps = R.top2_gap(yr)
    assert np.all(gaps > 4 * np.max(np.abs(yh - yr), axis=1)), "argmax not pinned by this seed"
    assert np.array_equal(am, R.argmax_lowest(yr))


@pytest.mark.parametrize("fmt", FMTS)
def test_invariant_columns(fmt):
    N, K = 301, 2560
    packed, fields, x = _case(fmt, N, K, 16, 5)
    Wdev = U.to_dev(packed)

    def run(xs):
        xd = U.to_dev(xs)
        y = U.empty_dev((xs.shape[0], N))
        kq.kq_gemv_invariant(fmt, Wdev, xd, y, N, K, xs.shape[0])
        return U.to_host(y)
    ref = np.stack([run(x[m:m + 1])[0] for m in range(16)])
    for M in (2, 5, 8, 16):
        y = run(x[:M])
        assert np.array_equal(y.view(np.uint32), ref[:M].view(np.uint32)), M
    yr, ad = R.gemv(fmt, fields, x)
    U.assert_parity(ref, yr, ad, f"{fmt} invariant")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", (1, 4))
def test_moe_ffn(fmt, M):
    """A small routed-expert layer (16 experts, hidden 512, FFN 256, top-4):
    y within tolerance of the oracle fed the GPU's own h, and h within one
    fp16 ulp-scale of the oracle's (the SwiGLU reading)."""
    E, hidden, inter, top_k = 16, 512, 256, 4
    gate = [U.quantize_both(fmt, S.weights((87, e, 0), inter, hidden)) for e in range(E)]
    up = [U.quantize_both(fmt, S.weights((87, e, 1), inter, hidden)) for e in range(E)]
    down = [U.quantize_both(fmt, S.weights((87, e, 2), hidden, inter)) for e in range(E)]
    x = S.activations((87, M), hidden, M)
    ids, rw = S.route_table(87, M, E, top_k)
    Wg = U.to_dev(np.concatenate([g[0].reshape(-1) for g in gate]))
    Wu = U.to_dev(np.concatenate([u[0].reshape(-1) for u in up]))
    Wdn = U.to_dev(np.concatenate([d[0].reshape(-1) for d in down]))
    y = U.empty_dev((M, hidden))
    h = U.empty_dev((M, top_k, inter), "float16")
    wsb = kq.kq_moe_ffn_workspace_bytes(hidden, inter, M, top_k)
    ws = U.empty_dev((wsb // 4 + 4,))
    kq.kq_moe_ffn(fmt, Wg, Wu, Wdn, U.to_dev(x), U.to_dev(ids), U.to_dev(rw), y, h, hidden, inter, M, top_k, E,
                  ws, wsb)
    yh, hh = U.to_host(y), U.to_host(h)
    yr, ya, (g, ga), (u, ua), h_ref = R.moe_ffn(fmt, [f for _, f in gate], [f for _, f in up],
                                                [f for _, f in down], x, ids, rw, h_override=hh)
    U.assert_parity(yh, yr, ya, f"{fmt} moe y M={M}")
    # h = fp16(silu(g) u): the GPU's g and u are within tolerance, so h is
    # within a few fp16 ulps of the oracle's own
    _, _, _, _, h_own = R.moe_ffn(fmt, [f for _, f in gate], [f for _, f in up], [f for _, f in down], x, ids, rw)
    assert np.max(np.abs(hh.astype(np.float64) - h_own.astype(np.float64))) <= 4 * 2.0 ** -10 * (
        1 + np.max(np.abs(h_own.astype(np.float64))))
