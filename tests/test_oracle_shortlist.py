"""Pins for the Shortlist oracle (oracle/shortlist.py), checked against values
fixed by hand and by mathematics, never against the oracle itself:

* hand-worked bound-copy rows (tests/golden/shortlist/): bytes and norm
* the quant split q = 8 (v - 16) + ql over every int8
* the residual norm against exact rational arithmetic (Fractions)
* |y - yhat| <= E ||x||_2 in exact arithmetic, and its equality case
* yhat in closed form for block-constant activations
* the shortlisted argmax against the argmax of every exact score, including
  ties, an all-zero column and a column that makes one row stand out
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import ref as R
from oracle import shortlist as SL
from tests import golden_blocks as G

ROWS = G.all_shortlist_rows()


def _q8(n, k, seed, scale=0.02):
    rng = np.random.default_rng(seed)
    W = rng.normal(0.0, scale, size=(n, k)).astype(np.float32)
    return F.quantize("q8_0", W)


def _x(k, seed):
    return np.random.default_rng(seed).standard_normal(k).astype(np.float16)


# ------------------------------------------------------------ check helpers
# Functions, so tests/test_oracle_mutations.py can run them on a broken oracle.

def check_golden_row(row) -> None:
    got = SL.encode_bound_copy(row["fields"])
    assert got.tobytes() == row["bytes"].tobytes(), (
        f"{row['name']}: {got.tobytes().hex(' ')} != {row['bytes'].tobytes().hex(' ')}")
    dec = SL.decode_bound_copy(row["bytes"], 1, row["k"])
    assert float(dec["E"][0]) == row["E"]


def check_split_every_int8() -> None:
    q = np.arange(-128, 128).astype(np.int8)
    v, ql = SL.split_quants(q)
    assert v.min() == 0 and v.max() == 31 and ql.min() == 0 and ql.max() == 7
    assert np.array_equal(8 * (v.astype(np.int64) - 16) + ql, q.astype(np.int64))
    spots = {-1: (15, 7), -8: (15, 0), -9: (14, 7), 0: (16, 0), 7: (16, 7), 8: (17, 0), 127: (31, 7), -127: (0, 1)}
    for qq, (vv, ll) in spots.items():
        a, b = SL.split_quants(np.array([qq], np.int8))
        assert (int(a[0]), int(b[0])) == (vv, ll), qq


def _exact_S(d_row, ql_row) -> Fraction:
    s = Fraction(0)
    for b in range(len(d_row)):
        db = Fraction(float(np.float16(d_row[b])))
        s += db * db * sum((Fraction(int(t)) - Fraction(7, 2)) ** 2 for t in ql_row[b])
    return s


def check_norm_is_least_fp32_above(d_row, q_row) -> None:
    _, ql = SL.split_quants(q_row)
    E = SL.residual_norm_up(d_row, ql)
    S = _exact_S(d_row, ql)
    assert Fraction(float(E)) ** 2 >= S
    below = np.nextafter(np.float32(E), np.float32(0))
    assert E == 0 or Fraction(float(below)) ** 2 < S


def check_bound_exact(fields, x16) -> None:
    """(y - yhat)^2 <= E^2 ||x||^2 for every row, in Fractions; y from the
    Q8_0 definition w' = d q, yhat from the split."""
    bound = SL.decode_bound_copy(SL.encode_bound_copy(fields), fields["q"].shape[0], fields["q"].shape[1] * 32)
    xs = [Fraction(float(t)) for t in np.asarray(x16, np.float16)]
    x2 = sum(t * t for t in xs)
    for n in range(fields["q"].shape[0]):
        y = yhat = Fraction(0)
        for b in range(fields["q"].shape[1]):
            db = Fraction(float(fields["d"][n, b]))
            xb = xs[32 * b:32 * b + 32]
            y += db * sum(int(fields["q"][n, b, j]) * xb[j] for j in range(32))
            yhat += db * (8 * sum((int(bound["v"][n, b, j]) - 16) * xb[j] for j in range(32))
                          + Fraction(7, 2) * sum(xb))
        E = Fraction(float(bound["E"][n]))
        assert (y - yhat) ** 2 <= E * E * x2, n
        t = SL.bound_terms(bound, x16)
        assert abs(float(yhat) - t["yhat"][n]) <= 1e-12 * (1 + t["T"][n] * 128)


def check_equality_case() -> None:
    """x equal to the residual e of one block (d = 1, so e_j = ql_j - 3.5 is
    an exact fp16): y - yhat = ||e||^2 and E ||x|| = E ||e|| is at most one
    fp32 rounding above it, so the radius is attained, not just respected."""
    k = 256
    q = np.zeros((1, 8, 32), np.int8)
    q[0, 3] = np.array([(5 * j) % 256 - 128 for j in range(32)], np.int8)
    d = np.zeros((1, 8), np.float16)
    d[0, 3] = 1.0
    fields = {"d": d, "q": q}
    _, ql = SL.split_quants(q)
    x = np.zeros(k, np.float16)
    x[96:128] = ql[0, 3].astype(np.float64) - 3.5
    bound = SL.decode_bound_copy(SL.encode_bound_copy(fields), 1, k)
    t = SL.bound_terms(bound, x)
    y = float(sum(int(a) * float(b) for a, b in zip(q[0, 3], x[96:128])))
    gap = y - t["yhat"][0]
    e2 = float(((ql[0, 3].astype(np.float64) - 3.5) ** 2).sum())
    assert gap == pytest.approx(e2, rel=1e-12)
    assert t["r"][0] >= gap and t["r"][0] <= gap * (1 + 2.0 ** -22)


def check_yhat_block_constant() -> None:
    """x = c on block b, 0 elsewhere: yhat = d_b c (8 sum_j (v_j - 16) + 3.5 * 32)."""
    fields = _q8(3, 512, seed=11)
    bound = SL.decode_bound_copy(SL.encode_bound_copy(fields), 3, 512)
    for b, c in ((0, 1.0), (7, -2.5), (15, 0.125)):
        x = np.zeros(512, np.float16)
        x[32 * b:32 * b + 32] = c
        t = SL.bound_terms(bound, x)
        for n in range(3):
            v = bound["v"][n, b].astype(np.int64) - 16
            want = float(fields["d"][n, b]) * c * (8 * int(v.sum()) + 3.5 * 32)
            assert t["yhat"][n] == pytest.approx(want, rel=1e-14, abs=1e-300)


def check_shortlist_argmax(fields, x16) -> dict:
    n, nb, _ = fields["q"].shape
    bound = SL.decode_bound_copy(SL.encode_bound_copy(fields), n, nb * 32)
    res = SL.shortlist_argmax(fields, bound, x16)
    y, _ = R.gemv("q8_0", fields, np.asarray(x16)[None, :])
    assert res["index"] == int(R.argmax_lowest(y[0])), (res["index"], int(R.argmax_lowest(y[0])))
    assert res["keep"][res["index"]] and res["keep"][res["pivot"]]
    t = res["terms"]
    assert np.all(t["u"] >= y[0]) and np.all(t["l"] <= y[0])
    return res


# ------------------------------------------------------------------ tests

@pytest.mark.parametrize("row", ROWS, ids=[r["name"] for r in ROWS])
def test_golden_rows(row):
    assert len(ROWS) >= 2
    check_golden_row(row)


def test_split_every_int8():
    check_split_every_int8()


@pytest.mark.parametrize("seed", range(6))
def test_norm_least_fp32_above(seed):
    fields = _q8(2, 256, seed=100 + seed, scale=[0.02, 1e-3, 3.0, 1e-6, 0.5, 40.0][seed])
    for n in range(2):
        check_norm_is_least_fp32_above(fields["d"][n], fields["q"][n])


def test_norm_special_scales():
    q = np.random.default_rng(5).integers(-127, 128, size=(8, 32)).astype(np.int8)
    for dv in (0.0, 2.0 ** -24, 65504.0, 6.1035e-05):
        d = np.full(8, dv, np.float16)
        check_norm_is_least_fp32_above(d, q)
    assert SL.residual_norm_up(np.zeros(8, np.float16), SL.split_quants(q)[1]) == 0


@pytest.mark.parametrize("seed", range(3))
def test_bound_exact(seed):
    fields = _q8(4, 256, seed=200 + seed)
    check_bound_exact(fields, _x(256, 300 + seed))


def test_equality_case():
    check_equality_case()


def test_yhat_block_constant():
    check_yhat_block_constant()


@pytest.mark.parametrize("n,k,seed", [(1, 256, 0), (7, 256, 1), (300, 512, 2), (2000, 256, 3), (5000, 768, 4)])
def test_shortlist_argmax_random(n, k, seed):
    check_shortlist_argmax(_q8(n, k, seed=400 + seed), _x(k, 500 + seed))


def test_shortlist_argmax_ties_lowest_index():
    fields = _q8(50, 256, seed=7)
    x = _x(256, 8)
    y, _ = R.gemv("q8_0", fields, x[None, :])
    top = int(R.argmax_lowest(y[0]))
    for dst in (3, 40):          # copies of the best row before and after it
        fields["d"][dst] = fields["d"][top]
        fields["q"][dst] = fields["q"][top]
    res = check_shortlist_argmax(fields, x)
    assert res["index"] == 3


def test_shortlist_argmax_zero_column():
    fields = _q8(64, 256, seed=9)
    res = check_shortlist_argmax(fields, np.zeros(256, np.float16))
    assert res["index"] == 0 and res["keep"].all()


def test_shortlist_prunes_a_peaked_column():
    """x built from one row's weights gives that row a score well above the
    rest: the shortlist keeps a small fraction of the rows."""
    fields = _q8(3000, 512, seed=12)
    w = F.dequantize("q8_0", fields, slice(1234, 1235))[0]
    x = (w / np.abs(w).max() * 4.0).astype(np.float16)
    res = check_shortlist_argmax(fields, x)
    assert res["index"] == 1234
    assert res["keep"].mean() < 0.02


def test_round_trip():
    fields = _q8(9, 768, seed=13)
    buf = SL.encode_bound_copy(fields)
    assert buf.size == SL.bound_copy_bytes(9, 768)
    dec = SL.decode_bound_copy(buf, 9, 768)
    v, ql = SL.split_quants(fields["q"])
    assert np.array_equal(dec["v"], v)
    assert np.array_equal(dec["d"].view(np.uint16), fields["d"].view(np.uint16))
    for n in range(9):
        assert dec["E"][n] == SL.residual_norm_up(fields["d"][n], ql[n])
