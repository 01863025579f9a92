"""GPU tests of kq_shortlist_argmax through the C ABI: the argmax of a Q8_0
output layer from its bound copy and exact scores of the rows the bounds keep.

* the index equals kq_gemv_argmax's (the kept rows are scored with kq_gemv's
  per-row arithmetic) and the oracle's argmax, where the oracle's top-2 gap
  pins it;
* every row's upper bound u (left in the workspace) is at least the score
  kq_gemv gives that row, and u is within tolerance of the oracle's bound;
* ties (lowest index), an all-zero column (every row kept, index 0), a NaN in
  x (every score NaN: every row kept, index 0), a column that makes one row
  stand out (few rows kept), ragged and one-row shapes, K up to 16384;
* the 4B-shaped 151936 x 2560 head at the bench's launch configuration.
"""
import numpy as np
import pytest

import block_quantized_gemv_kq_amd as kq
from oracle import formats as F
from oracle import ref as R
from oracle import shortlist as SL
from synth import inputs as S
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def _upload(packed, N, K):
    copy = kq.kq_shortlist_pack(packed, N, K)
    return U.to_dev(packed.reshape(-1)), U.to_dev(copy)


def _shortlist(Wd, Cd, xd, N, K):
    wsb = kq.kq_shortlist_workspace_bytes(N, K)
    ws = U.empty_dev((wsb // 4 + 64,))
    ws.fill_(float("nan"))
    out = U.empty_dev((1,), "int32")
    kept = U.empty_dev((1,), "int32")
    kq.kq_shortlist_argmax(Wd, Cd, xd, N, K, ws, wsb, out, kept)
    return int(U.to_host(out)[0]), int(U.to_host(kept)[0]), U.to_host(ws)[:N]


def _gemv_argmax(Wd, xd, N, K):
    y = U.empty_dev((1, N))
    out = U.empty_dev((1,), "int32")
    wsb = kq.kq_gemv_argmax_workspace_bytes("q8_0", N, K, 1)
    ws = U.empty_dev((wsb // 4 + 2,))
    kq.kq_gemv_argmax("q8_0", Wd, xd, y, N, K, 1, out, ws, wsb)
    return U.to_host(y)[0], int(U.to_host(out)[0])


def _check(packed, x16, N, K, fields=None, oracle=True):
    Wd, Cd = _upload(packed, N, K)
    xd = U.to_dev(x16.reshape(1, K))
    idx, kept, u = _shortlist(Wd, Cd, xd, N, K)
    y, ref_idx = _gemv_argmax(Wd, xd, N, K)
    assert idx == ref_idx, (idx, ref_idx)
    assert 1 <= kept <= N
    finite = np.isfinite(y)
    assert np.all(u[finite] >= y[finite]), "an upper bound below the row's score"
    if oracle:
        fields = fields if fields is not None else F.decode("q8_0", packed, N, K)
        yr, ad = R.gemv("q8_0", fields, x16.reshape(1, K))
        U.assert_parity(y[None, :], yr, ad, f"q8_0 N={N} K={K}")
        gap = float(R.top2_gap(yr[0])) if N > 1 else np.inf
        err = float(np.max(np.abs(y - yr[0])))
        if gap > 4 * err:
            assert idx == int(R.argmax_lowest(yr[0]))
        bound = SL.decode_bound_copy(kq.kq_shortlist_pack(packed, N, K), N, K)
        t = SL.bound_terms(bound, x16.reshape(-1))
        tol = 2e-3 * (135.5 * t["T"] + t["r"] + t["s"]) + 1e-6
        assert np.all(np.abs(u - t["u"]) <= tol), "bound differs from the oracle's"
    return idx, kept


@pytest.mark.parametrize("N,K", [(1, 256), (37, 256), (1000, 512), (4099, 2560), (20000, 2560), (300, 16384),
                                 (777, 768)])
@pytest.mark.parametrize("seed", (0, 1))
def test_matches_gemv_argmax_and_oracle(N, K, seed):
    W = S.weights((93, seed, N, K), N, K)
    packed = kq.kq_pack("q8_0", W)
    x = S.activations((93, seed, K), K, 1)[0]
    _check(packed, x, N, K)


def _big_row(K):
    blk = np.zeros(34, np.uint8)
    blk[:2] = np.frombuffer(np.float16(1.0).tobytes(), np.uint8)
    blk[2:] = 127
    return np.tile(blk, K // 32)


def test_ties_lowest_index():
    N, K = 5000, 256
    rows = kq.kq_pack("q8_0", S.weights((94, N, K), N, K)).reshape(N, -1).copy()
    for r in (2700, 7, 3):
        rows[r] = _big_row(K)
    x = np.full(K, np.float16(1.0))
    idx, kept = _check(rows.reshape(-1), x, N, K)
    assert idx == 3 and kept >= 3


def test_zero_column_keeps_every_row():
    N, K = 3000, 512
    packed = kq.kq_pack("q8_0", S.weights((95, N, K), N, K))
    idx, kept = _check(packed, np.zeros(K, np.float16), N, K)
    assert idx == 0 and kept == N


def test_nan_in_x_keeps_every_row():
    N, K = 2000, 256
    packed = kq.kq_pack("q8_0", S.weights((96, N, K), N, K))
    x = S.activations((96, K), K, 1)[0].copy()
    x[17] = np.float16(np.nan)
    Wd, Cd = _upload(packed, N, K)
    xd = U.to_dev(x.reshape(1, K))
    idx, kept, _ = _shortlist(Wd, Cd, xd, N, K)
    y, ref_idx = _gemv_argmax(Wd, xd, N, K)
    assert np.all(np.isnan(y))
    assert idx == ref_idx == 0 and kept == N


def test_peaked_column_keeps_few_rows():
    """x from row 4321's own weights gives it a score far above the rest."""
    N, K = 30000, 2560
    packed = kq.kq_pack("q8_0", S.weights((97, N, K), N, K))
    w = F.dequantize("q8_0", F.decode("q8_0", packed, N, K), slice(4321, 4322))[0]
    x = (w / np.abs(w).max() * 4.0).astype(np.float16)
    idx, kept = _check(packed, x, N, K)
    assert idx == 4321
    assert kept < N // 100


def test_repeatable():
    N, K = 20000, 2560
    packed = kq.kq_pack("q8_0", S.weights((98, N, K), N, K))
    Wd, Cd = _upload(packed, N, K)
    xd = U.to_dev(S.activations((98, K), K, 1))
    first = _shortlist(Wd, Cd, xd, N, K)
    for _ in range(3):
        again = _shortlist(Wd, Cd, xd, N, K)
        assert again[:2] == first[:2]
        assert np.array_equal(again[2].view(np.uint32), first[2].view(np.uint32))


@pytest.fixture(scope="module")
def head_dev():
    st = S.QWEN3_4B_AFFINE4
    h = st.head
    W = S.weights(st.weight_seed(st.layers, 0), h.n, h.k)
    packed = kq.kq_pack(h.fmt, W)
    del W
    Wd, Cd = _upload(packed, h.n, h.k)
    return h, packed, Wd, Cd


@pytest.mark.parametrize("col", (0, 1, 2))
def test_lm_head(head_dev, col):
    """The 4B-shaped Q8_0 head: the index of kq_gemv_argmax and of the oracle,
    every bound above its row's score, and about 3 % of the rows kept."""
    h, packed, Wd, Cd = head_dev
    x = S.activations((S.VERIFY_WORKLOAD_ID, 36, col), h.k, 1)
    xd = U.to_dev(x)
    idx, kept, u = _shortlist(Wd, Cd, xd, h.n, h.k)
    y, ref_idx = _gemv_argmax(Wd, xd, h.n, h.k)
    assert idx == ref_idx
    assert np.all(u >= y)
    assert kept < h.n // 10
    fields = F.decode("q8_0", packed, h.n, h.k)
    yr, ad = R.gemv("q8_0", fields, x)
    U.assert_parity(y[None, :], yr, ad, "lm_head")
    assert float(R.top2_gap(yr[0])) > 4 * float(np.max(np.abs(y - yr[0])))
    assert idx == int(R.argmax_lowest(yr[0]))
    print(f"lm_head column {col}: kept {kept} of {h.n} rows ({100.0 * kept / h.n:.2f} %)")
