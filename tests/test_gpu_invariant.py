"""GPU tests of kq_gemv_invariant through the C ABI: column m of an M-column
call has the same bits as a one-column kq_gemv_invariant call on x[m] (the
batch rule of the Kinetic docs, "What makes it fast"), on every kernel the
entry point takes (persistent waves, split-K teams, K-chunked, the generic
kernel for 2-byte-aligned rows), at small and at decode sizes, for M from 1
to 64; plus parity with the oracle and run-to-run determinism."""
import numpy as np
import pytest

import block_quantized_gemv_kq_amd as kq
from oracle import ref as R
from synth import inputs as S
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

FMTS = ("q8_0", "q4_0", "affine4")
M_LIST = (1, 2, 3, 4, 5, 8, 13, 16, 48, 64)


def _run(entry, fmt, Wdev, x16, N, K):
    M = x16.shape[0]
    xd = U.to_dev(x16)
    y = U.empty_dev((M, N))
    y.fill_(float("nan"))
    getattr(kq, entry)(fmt, Wdev, xd, y, N, K, M)
    return U.to_host(y)


def _single_columns(fmt, Wdev, x16, N, K, entry="kq_gemv_invariant"):
    return np.stack([_run(entry, fmt, Wdev, x16[m:m + 1], N, K)[0] for m in range(x16.shape[0])])


# (N, K): x of 8 columns staged in LDS (the split-K teams kernel, K = 2048),
# rows too long for that (the K-chunked kernel, K = 45056), blocks that are
# not whole 2-block units (Q4_0 / Q8_0 at K = 96: the generic kernel; affine4
# there is one partial group), and more than 4096 row tiles (persistent waves).
SHAPES = [(133, 2048), (37, 45056), (29, 96), (65601, 256)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", SHAPES)
def test_columns_bitwise_equal_single_column_calls(fmt, N, K):
    W = S.weights((81, N, K), N, K)
    x = S.activations((81, K), K, max(M_LIST))
    packed, fields = U.quantize_both(fmt, W)
    Wdev = U.to_dev(packed)
    ref = _single_columns(fmt, Wdev, x, N, K)
    yr, ad = R.gemv(fmt, fields, x)
    U.assert_parity(ref, yr, ad, f"{fmt} one-column calls N={N} K={K}")
    for M in M_LIST:
        y = _run("kq_gemv_invariant", fmt, Wdev, x[:M], N, K)
        assert np.array_equal(y.view(np.uint32), ref[:M].view(np.uint32)), (fmt, N, K, M)
        U.assert_parity(y, yr[:M], ad[:M], f"{fmt} invariant N={N} K={K} M={M}")


@pytest.mark.parametrize("fmt", FMTS)
def test_deterministic_and_parity(fmt):
    N, K, M = 301, 2560, 9
    W = S.weights((82, N, K), N, K)
    x = S.activations((82, K), K, M)
    packed, fields = U.quantize_both(fmt, W)
    Wdev = U.to_dev(packed)
    y1 = _run("kq_gemv_invariant", fmt, Wdev, x, N, K)
    y2 = _run("kq_gemv_invariant", fmt, Wdev, x, N, K)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    yr, ad = R.gemv(fmt, fields, x)
    U.assert_parity(y1, yr, ad, f"{fmt} invariant M={M}")


@pytest.mark.parametrize("fmt", FMTS)
def test_two_and_three_columns_of_kq_gemv_are_invariant(fmt):
    """kq_gemv itself takes the one-column kernels for 2 and 3 columns of
    whole-unit rows that fit LDS staging: its columns are bit-identical too."""
    N, K = 150, 2560
    W = S.weights((83, N, K), N, K)
    x = S.activations((83, K), K, 3)
    packed, _ = U.quantize_both(fmt, W)
    Wdev = U.to_dev(packed)
    ref = _single_columns(fmt, Wdev, x, N, K, entry="kq_gemv")
    for M in (2, 3):
        y = _run("kq_gemv", fmt, Wdev, x[:M], N, K)
        assert np.array_equal(y.view(np.uint32), ref[:M].view(np.uint32)), (fmt, M)


@pytest.mark.parametrize("N,K", [(6144, 2560), (2560, 4096), (2560, 9728), (19456, 2560)])
def test_decode_shapes_m8(N, K):
    """The 4B-shaped affine4 layer matrices at M = 8 (the verify width) and
    M = 16: every output of every column bit-identical to the one-column
    calls."""
    fmt = "affine4"
    rng = np.random.default_rng(N * 7 + K)
    nb = kq.kq_packed_bytes(fmt, N, K)
    # random packed bytes with finite scales: scale/bias fields are fp16 values in [-1, 1)
    packed = rng.integers(0, 256, size=(N, nb // N), dtype=np.uint8)
    blocks = packed.reshape(N, K // 32, 20)
    hdr = (rng.random((N, K // 32, 2)) * 2 - 1).astype(np.float16) * np.float16(0.05)
    blocks[:, :, :4] = hdr.view(np.uint8).reshape(N, K // 32, 4)
    Wdev = U.to_dev(packed.reshape(-1))
    x = S.activations((84, N, K), K, 16)
    ref = _single_columns(fmt, Wdev, x, N, K)
    assert np.all(np.isfinite(ref))
    for M in (8, 16):
        y = _run("kq_gemv_invariant", fmt, Wdev, x[:M], N, K)
        assert np.array_equal(y.view(np.uint32), ref[:M].view(np.uint32)), M


def test_lm_head_shape_m8():
    """The 151936 x 2560 Q8_0 output layer (persistent waves) at M = 8 and
    48: columns bit-identical to one-column calls (random packed bytes with
    finite scales)."""
    fmt, N, K = "q8_0", 151936, 2560
    rng = np.random.default_rng(85)
    nb = kq.kq_packed_bytes(fmt, N, K)
    packed = rng.integers(0, 256, size=(N, nb // N), dtype=np.uint8)
    blocks = packed.reshape(N, K // 32, 34)
    blocks[:, :, :2] = ((rng.random((N, K // 32, 1)) * 2 - 1).astype(np.float16) * np.float16(0.002)).view(np.uint8)
    Wdev = U.to_dev(packed.reshape(-1))
    x = S.activations((85, N, K), K, 48)
    ref = np.stack([_run("kq_gemv_invariant", fmt, Wdev, x[m:m + 1], N, K)[0] for m in (0, 7, 31, 47)])
    for M in (8, 48):
        y = _run("kq_gemv_invariant", fmt, Wdev, x[:M], N, K)
        cols = [m for m in (0, 7, 31, 47) if m < M]
        assert np.array_equal(y[cols].view(np.uint32), ref[:len(cols)].view(np.uint32)), M
