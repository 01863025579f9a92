"""Pins for the CPU oracle: checks against values fixed by the block
definitions and by mathematics, never against the oracle itself.

* hand-worked blocks (tests/golden/): packed bytes and exact dequantized values
* round-half-away-from-zero against exact rational rounding at every tie
* fp16 conversion spot checks (round-to-nearest-even, subnormals)
* exact (Fraction) dot products on small matrices
* closed forms: unit-vector probes, all-ones sums, SiLU identities
* quantize/dequantize round-trip invariants and idempotence
* routed-expert special cases
"""
from fractions import Fraction
import math

import numpy as np
import pytest

from oracle import formats as F
from oracle import ref as R
from synth import inputs as S
from tests import golden_blocks as G

BLOCKS = G.all_blocks()


# ------------------------------------------------------------ check helpers
# Written as functions so tests/test_oracle_mutations.py can re-run them on a
# deliberately broken oracle and see them fail.

def check_golden_block(blk) -> None:
    fmt = blk["format"]
    W = blk["weights"][None, :]
    got = F.pack(fmt, W)[0]
    assert got.tobytes() == blk["bytes"].tobytes(), (
        f"{blk['name']}: bytes {got.tobytes().hex(' ')} != {blk['bytes'].tobytes().hex(' ')}")
    fields = F.decode(fmt, blk["bytes"], 1, 32)
    wq = F.dequantize(fmt, fields)[0]
    assert np.array_equal(wq, blk["dequant"]), f"{blk['name']}: dequant {wq} != {blk['dequant']}"


def check_unit_vectors(fmt: str, seed: int = 3) -> None:
    """x = e_k gives y[n] = w'[n][k]; checked against the hand-worked blocks
    stacked as rows (their w' are known exactly)."""
    rows = [b for b in BLOCKS if b["format"] == fmt]
    packed = np.stack([b["bytes"] for b in rows])
    fields = F.decode(fmt, packed, len(rows), 32)
    expect = np.stack([b["dequant"] for b in rows])          # [n, 32]
    for k in range(32):
        x = np.zeros((1, 32), np.float16)
        x[0, k] = 1.0
        y, _ = R.gemv(fmt, fields, x)
        assert np.array_equal(y[0], expect[:, k]), f"{fmt} column {k}"


def check_ones_sum(fmt: str) -> None:
    """x = all ones gives the exact sum of each block's w' (computed here in
    Fractions from the hand-derived dequant values)."""
    rows = [b for b in BLOCKS if b["format"] == fmt]
    packed = np.stack([b["bytes"] for b in rows])
    fields = F.decode(fmt, packed, len(rows), 32)
    y, _ = R.gemv(fmt, fields, np.ones((1, 32), np.float16))
    for i, b in enumerate(rows):
        exact = sum(Fraction(float(v)) for v in b["dequant"])
        assert Fraction(float(y[0, i])) == exact, b["name"]


def _exact_wprime(fmt, fields):
    """w' in Fractions from the block fields, for small matrices only."""
    q = fields["q"]
    n, nb, _ = q.shape
    out = [[None] * (nb * 32) for _ in range(n)]
    for r in range(n):
        for b in range(nb):
            for j in range(32):
                qq = int(q[r, b, j])
                if fmt == "q8_0":
                    v = Fraction(float(fields["d"][r, b])) * qq
                elif fmt == "q4_0":
                    v = Fraction(float(fields["d"][r, b])) * (qq - 8)
                elif fmt == "q5_0":
                    v = Fraction(float(fields["d"][r, b])) * (qq - 16)
                elif fmt == "q5_1":
                    v = Fraction(float(fields["d"][r, b])) * qq + Fraction(float(fields["m"][r, b]))
                else:
                    v = Fraction(float(fields["s"][r, b])) * qq + Fraction(float(fields["b"][r, b]))
                out[r][b * 32 + j] = v
    return out


def check_exact_small_gemv(fmt: str, n: int, k: int, m: int, seed: int) -> None:
    """Fraction-exact y on a non-square matrix vs the fp64 oracle, within the
    fp64 summation bound K * 2^-52 * sum|w'x|."""
    W = S.weights((99, seed, 0, 0), n, k)
    x = S.activations((99, seed, 0), k, m)
    fields = F.quantize(fmt, W)
    y, absd = R.gemv(fmt, fields, x)
    wp = _exact_wprime(fmt, fields)
    for c in range(m):
        xf = [Fraction(float(v)) for v in x[c]]
        for r in range(n):
            exact = sum(wp[r][kk] * xf[kk] for kk in range(k))
            absx = sum(abs(wp[r][kk] * xf[kk]) for kk in range(k))
            assert abs(Fraction(float(y[c, r])) - exact) <= Fraction(k) * Fraction(2) ** -52 * absx + Fraction(1, 10**300)
            assert abs(float(absd[c, r]) - float(absx)) <= 1e-12 * float(absx) + 1e-300


def check_acceptance_bound() -> None:
    """The bar every GPU result is held to, per output: |y - y_ref| <=
    2e-3 * sum_k |w'[n][k] x[m][k]| + 1e-6. Points worked by hand: at
    sum|w'x| = 1000 the bound is 2.000001, at 0 it is 1e-6, at 0.5 it is
    0.001001; differences just inside pass and just outside fail, in both
    directions."""
    cases = [  # (sum|w'x|, y_ref, y_gpu, inside?)
        (1000.0, 0.0, 2.0000009, True), (1000.0, 0.0, 2.0000011, False),
        (1000.0, 5.0, 5.0 - 2.0000009, True), (1000.0, 5.0, 5.0 - 2.0000011, False),
        (0.0, 0.0, 0.9e-6, True), (0.0, 0.0, 1.1e-6, False), (0.0, 3.0, 3.0 - 1.1e-6, False),
        (0.5, 1.0, 1.0 + 0.00100099, True), (0.5, 1.0, 1.0 + 0.00100101, False),
    ]
    a = np.array([c[0] for c in cases])
    ref = np.array([c[1] for c in cases])
    gpu = np.array([c[2] for c in cases])
    expect = np.array([c[3] for c in cases])
    got = R.within_tolerance(gpu, ref, a)
    assert np.array_equal(got, expect), f"acceptance {got} != {expect}"
    assert abs(float(R.tolerance(np.array([1000.0]))[0]) - 2.000001) < 1e-12
    assert abs(float(R.tolerance(np.array([0.0]))[0]) - 1e-6) < 1e-18


def check_error_ratio() -> None:
    """max |y - y_ref| / sum|w'x| on a hand-worked case: differences 0.1,
    0 and 0.03 over sums 10, 4 and 1 give ratios 0.01, 0 and 0.03."""
    r = R.error_ratio(np.array([1.0, 2.0, -0.03]), np.array([1.1, 2.0, 0.0]), np.array([10.0, 4.0, 1.0]))
    assert abs(r - 0.03) < 1e-12, r


def check_abs_dot(fmt: str) -> None:
    """The sum in the bound is of |w'x| term by term, not |sum w'x|: with x
    alternating +1/-1 it equals sum_k |w'[n][k]| exactly (Fractions of the
    hand-derived dequant values of the golden blocks)."""
    rows = [b for b in BLOCKS if b["format"] == fmt]
    packed = np.stack([b["bytes"] for b in rows])
    fields = F.decode(fmt, packed, len(rows), 32)
    x = np.array([[1.0 if k % 2 == 0 else -1.0 for k in range(32)]], np.float16)
    _, absd = R.gemv(fmt, fields, x)
    for i, b in enumerate(rows):
        exact = sum(abs(Fraction(float(v))) for v in b["dequant"])
        assert Fraction(float(absd[0, i])) == exact, f"{b['name']}: {absd[0, i]} != {float(exact)}"


# ------------------------------------------------------------ the pins

@pytest.mark.parametrize("blk", BLOCKS, ids=lambda b: b["name"])
def test_golden_block(blk):
    check_golden_block(blk)


@pytest.mark.parametrize("fmt", F.FORMATS)
def test_unit_vectors(fmt):
    check_unit_vectors(fmt)


@pytest.mark.parametrize("fmt", F.FORMATS)
def test_ones_sum(fmt):
    check_ones_sum(fmt)


def test_round_half_away_ties():
    """Every k + 0.5 for k in [-128, 127] and its fp32 neighbours, against
    exact rational rounding: sign(v) * floor(|v| + 1/2)."""
    vals = []
    for k in range(-128, 128):
        t = np.float32(k + 0.5)
        vals += [t, np.nextafter(t, np.float32(np.inf)), np.nextafter(t, np.float32(-np.inf))]
    vals += [np.float32(0.5 - 2.0 ** -25), np.float32(-(0.5 - 2.0 ** -25)), np.float32(0.0), np.float32(-0.0)]
    got = F.round_half_away(np.array(vals, np.float32))
    for v, g in zip(vals, got):
        fv = Fraction(float(v))
        sign = 1 if fv >= 0 else -1
        exact = sign * math.floor(abs(fv) + Fraction(1, 2))
        assert g == exact, (float(v), g, exact)


def test_fp16_conversion_spot_checks():
    """numpy's fp32->fp16 cast is the oracle's fp16(); pin its rounding."""
    cases = [
        (1.0 + 2.0 ** -11, 1.0),                   # tie -> even (mantissa 0)
        (1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -9),   # tie -> even (mantissa 2)
        (1.0 + 2.0 ** -11 + 2.0 ** -20, 1.0 + 2.0 ** -10),
        (65504.0, 65504.0),
        (65519.0, 65504.0),
        (2.0 ** -24, 2.0 ** -24),                  # smallest subnormal
        (1.5 * 2.0 ** -24, 2.0 ** -23),            # tie -> even subnormal
        (2.0 ** -25, 0.0),                         # tie -> even (zero)
        (1.4 * 2.0 ** -24, 2.0 ** -24),
        (-2.0 ** -14, -2.0 ** -14),                # smallest normal
    ]
    for v, want in cases:
        got = float(F.to_f16(np.float32(v)))
        assert got == want, (v, got, want)
    assert np.isinf(F.to_f16(np.float32(65520.0)))


@pytest.mark.parametrize("fmt", F.FORMATS)
@pytest.mark.parametrize("n,k,m,seed", [(3, 32, 1, 1), (5, 96, 2, 2), (8, 64, 3, 3)])
def test_exact_small_gemv(fmt, n, k, m, seed):
    check_exact_small_gemv(fmt, n, k, m, seed)


def test_gemv_matches_textbook_dgemv():
    """Special case that reduces to a library routine: the oracle equals a
    plain fp64 matrix-vector product of the dequantized matrix."""
    W = S.weights((98, 0, 0, 0), 40, 256)
    x = S.activations((98, 0, 0), 256, 2)
    for fmt in F.FORMATS:
        fields = F.quantize(fmt, W)
        y, _ = R.gemv(fmt, fields, x)
        Wd = F.dequantize(fmt, fields)
        for c in range(2):
            ref = np.array([math.fsum(Wd[r] * x[c].astype(np.float64)) for r in range(40)])
            np.testing.assert_allclose(y[c], ref, rtol=0, atol=1e-15 * np.abs(Wd).sum(1).max() * 4)


def test_acceptance_bound():
    check_acceptance_bound()


def test_error_ratio():
    check_error_ratio()


@pytest.mark.parametrize("fmt", F.FORMATS)
def test_abs_dot_is_termwise(fmt):
    check_abs_dot(fmt)


def test_packed_bytes_match_block_sizes():
    """Block sizes as the workloads state them (Q8_0 34, Q4_0 18, affine4 20
    bytes per 32 weights), and the 1024 x 1024 Q8_0 matrix at 1,114,112 B."""
    assert F.packed_bytes("q8_0", 1024, 1024) == 1024 * 32 * 34 == 1114112
    assert F.packed_bytes("q4_0", 3, 64) == 3 * 2 * 18
    assert F.packed_bytes("affine4", 5, 96) == 5 * 3 * 20
    W = S.weights((77,), 3, 64)
    for fmt in F.FORMATS:
        assert F.encode(fmt, F.quantize(fmt, W)).nbytes == F.packed_bytes(fmt, 3, 64)


# ------------------------------------------------------------ invariants

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_q8_0_roundtrip(seed):
    W = S.weights((97, seed, 0, 0), 64, 512)
    f = F.quantize("q8_0", W)
    q = f["q"].astype(np.int32)
    d = f["d"].astype(np.float64)
    assert np.all(np.abs(q) <= 127)
    assert np.all(np.max(np.abs(q), axis=-1) == 127)           # normal scales
    err = np.abs(W.reshape(64, 16, 32).astype(np.float64) - d[..., None] * q)
    assert np.all(err <= d[..., None] / 2 * (1 + 2.0 ** -10) + 2.0 ** -23 * np.abs(W.reshape(64, 16, 32)))
    assert np.array_equal(F.pack("q8_0", F.dequantize("q8_0", f).astype(np.float32)), F.encode("q8_0", f))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_q4_0_roundtrip(seed):
    W = S.weights((96, seed, 0, 0), 64, 512)
    f = F.quantize("q4_0", W)
    q = f["q"].astype(np.int32)
    d = f["d"].astype(np.float64)
    X = W.reshape(64, 16, 32).astype(np.float64)
    assert q.min() >= 0 and q.max() <= 15
    istar = np.argmax(np.abs(X), axis=-1)
    assert np.all(np.take_along_axis(q, istar[..., None], -1) == 0)
    err = np.abs(X - d[..., None] * (q - 8))
    # Elements of the opposite sign to the signed maximum can reach w/d = 8(1+2^-11)
    # (d is m/-8 rounded to fp16); they clamp to q = 15 with error up to |d|(1 + 2^-8).
    clamped = (q == 15) & (X / d[..., None] > 7.5)
    bound = np.abs(d)[..., None] / 2 * (1 + 2.0 ** -10)
    assert np.all((err <= bound) | (clamped & (err <= (1 + 2.0 ** -8) * np.abs(d)[..., None])))
    assert np.array_equal(F.pack("q4_0", F.dequantize("q4_0", f).astype(np.float32)), F.encode("q4_0", f))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_affine4_roundtrip(seed):
    W = S.weights((95, seed, 0, 0), 64, 512)
    f = F.quantize("affine4", W)
    q = f["q"].astype(np.int32)
    s = f["s"].astype(np.float64)[..., None]
    b = f["b"].astype(np.float64)[..., None]
    X = W.reshape(64, 16, 32).astype(np.float64)
    lo = X.min(-1, keepdims=True)
    assert q.min() >= 0 and q.max() <= 15
    assert np.all(np.take_along_axis(q, np.argmin(X, -1)[..., None], -1) == 0)
    assert np.all(np.take_along_axis(q, np.argmax(X, -1)[..., None], -1) == 15)
    err = np.abs(X - (s * q + b))
    assert np.all(err <= s / 2 * (1 + 2.0 ** -9) + np.abs(b - lo) + 1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_q5_0_roundtrip(seed):
    W = S.weights((93, seed, 0, 0), 64, 512)
    f = F.quantize("q5_0", W)
    q = f["q"].astype(np.int32)
    d = f["d"].astype(np.float64)
    X = W.reshape(64, 16, 32).astype(np.float64)
    assert q.min() >= 0 and q.max() <= 31
    istar = np.argmax(np.abs(X), axis=-1)
    assert np.all(np.take_along_axis(q, istar[..., None], -1) == 0)
    err = np.abs(X - d[..., None] * (q - 16))
    # as Q4_0 with 16 levels: the opposite side of the signed maximum can
    # reach w/d = 16(1+2^-11) and clamps to q = 31
    clamped = (q == 31) & (X / d[..., None] > 15.5)
    bound = np.abs(d)[..., None] / 2 * (1 + 2.0 ** -10)
    assert np.all((err <= bound) | (clamped & (err <= (1 + 2.0 ** -8) * np.abs(d)[..., None])))
    assert np.array_equal(F.pack("q5_0", F.dequantize("q5_0", f).astype(np.float32)), F.encode("q5_0", f))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_q5_1_roundtrip(seed):
    W = S.weights((92, seed, 0, 0), 64, 512)
    f = F.quantize("q5_1", W)
    q = f["q"].astype(np.int32)
    d = f["d"].astype(np.float64)[..., None]
    m = f["m"].astype(np.float64)[..., None]
    X = W.reshape(64, 16, 32).astype(np.float64)
    lo = X.min(-1, keepdims=True)
    assert q.min() >= 0 and q.max() <= 31
    assert np.all(np.take_along_axis(q, np.argmin(X, -1)[..., None], -1) == 0)
    assert np.all(np.take_along_axis(q, np.argmax(X, -1)[..., None], -1) == 31)
    err = np.abs(X - (d * q + m))
    assert np.all(err <= d / 2 * (1 + 2.0 ** -9) + np.abs(m - lo) + 1e-12)


def test_fifth_bits_word_layout():
    """Bit j of the little-endian word after the scale(s) is bit 4 of q_j:
    q with only element 9 at 16 (Q5_0) gives the word 0x00000200."""
    f = {"d": np.array([[1.0]], np.float16), "q": np.full((1, 1, 32), 0, np.uint8)}
    f["q"][0, 0, 9] = 16
    b = F.encode("q5_0", f)[0]
    assert b[2:6].tolist() == [0x00, 0x02, 0x00, 0x00]
    assert b[6:22].tolist() == [0] * 16
    assert np.array_equal(F.decode("q5_0", b, 1, 32)["q"], f["q"])


def test_encode_decode_inverse():
    W = S.weights((94, 0, 0, 0), 7, 160)
    for fmt in F.FORMATS:
        f = F.quantize(fmt, W)
        p = F.encode(fmt, f)
        assert p.shape == (7, 5 * F.BLOCK_BYTES[fmt])
        f2 = F.decode(fmt, p, 7, 160)
        for key in f:
            assert np.array_equal(f[key].view(np.uint8), f2[key].view(np.uint8)), (fmt, key)


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        F.quantize("q8_0", np.full((1, 32), np.nan, np.float32))
    with pytest.raises(ValueError):
        F.quantize("affine4", np.full((1, 32), 70000.0, np.float32))
    with pytest.raises(ValueError):
        F.quantize("q8_0", np.zeros((1, 33), np.float32))
    with pytest.raises(TypeError):
        F.quantize("q8_0", np.zeros((1, 32), np.float64))


def test_scale_invariance_of_gemv():
    """y(2x) == 2 y(x) exactly: every product and partial sum scales by a power of two."""
    W = S.weights((93, 0, 0, 0), 16, 128)
    x = S.activations((93, 0, 0), 128, 1)
    for fmt in F.FORMATS:
        f = F.quantize(fmt, W)
        y1, _ = R.gemv(fmt, f, x)
        y2, _ = R.gemv(fmt, f, (x.astype(np.float32) * 2).astype(np.float16))
        assert np.array_equal(y2, 2 * y1)


def test_argmax_lowest_index_on_ties():
    y = np.array([1.0, 3.0, 2.0, 3.0])
    assert R.argmax_lowest(y) == 1
    assert list(R.argmax_lowest(np.stack([y, y[::-1]]))) == [1, 0]
    assert R.top2_gap(np.array([0.5, 2.0, 1.5])) == pytest.approx(0.5)


# ------------------------------------------------------------ experts

def test_silu_identities():
    z = np.linspace(-20, 20, 401)
    s = R.silu(z)
    np.testing.assert_allclose(s - R.silu(-z), z, rtol=0, atol=1e-13)   # silu(z) - silu(-z) = z
    assert R.silu(np.array([0.0]))[0] == 0.0
    assert R.silu(np.array([1.0]))[0] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert abs(R.silu(np.array([50.0]))[0] - 50.0) < 1e-15 * 50


def test_swiglu_rounds_to_fp16():
    g = np.array([0.0, 1.0, -3.0, 10.0])
    u = np.array([5.0, 2.0, 1.5, -0.25])
    h = R.swiglu_h16(g, u)
    assert h.dtype == np.float16
    want = [0.0, 2.0 / (1 + math.exp(-1.0)), 1.5 * -3.0 / (1 + math.exp(3.0)), -0.25 * 10 / (1 + math.exp(-10.0))]
    for a, b in zip(h, want):
        assert float(a) == float(np.float16(b))


def _tiny_experts(fmt, n_exp, n, k, seed):
    return [F.quantize(fmt, S.weights((92, seed, e, 0), n, k)) for e in range(n_exp)]


def test_moe_top1_unit_weight_is_plain_gemv():
    ex = _tiny_experts("q4_0", 4, 24, 64, 0)
    x = S.activations((92, 0, 0), 64, 3)
    ids = np.array([[2], [0], [2]], np.int32)
    y, _ = R.moe_gemv("q4_0", ex, x, ids, np.ones((3, 1), np.float32), False)
    for t in range(3):
        yr, _ = R.gemv("q4_0", ex[ids[t, 0]], x[t:t + 1])
        assert np.array_equal(y[t], yr[0])


def test_moe_identical_experts_convex_weights():
    f = F.quantize("q8_0", S.weights((92, 1, 0, 0), 16, 64))
    ex = [f] * 5
    x = S.activations((92, 1, 0), 64, 2)
    ids = np.array([[0, 3, 1], [4, 2, 0]], np.int32)
    rw = np.array([[0.5, 0.25, 0.25], [0.125, 0.375, 0.5]], np.float32)   # exact, sum to 1
    y, _ = R.moe_gemv("q8_0", ex, x, ids, rw, False)
    yr, _ = R.gemv("q8_0", f, x)
    np.testing.assert_allclose(y, yr, rtol=1e-15, atol=1e-15)


def test_moe_weighted_sum_exact_small():
    """Down-projection style call (x per slot, weighted sum) against a
    Fraction-exact sum in slot order."""
    ex = _tiny_experts("affine4", 3, 4, 32, 2)
    x = S.activations((92, 2, 0), 32, 4).reshape(2, 2, 32)
    ids = np.array([[1, 2], [0, 1]], np.int32)
    rw = np.array([[0.75, 0.25], [0.5, 0.5]], np.float32)
    y, _ = R.moe_gemv("affine4", ex, x, ids, rw, True)
    for t in range(2):
        for r in range(4):
            exact = Fraction(0)
            for j in range(2):
                wp = _exact_wprime("affine4", ex[ids[t, j]])
                exact += Fraction(float(rw[t, j])) * sum(
                    wp[r][kk] * Fraction(float(x[t, j, kk])) for kk in range(32))
            assert abs(Fraction(float(y[t, r])) - exact) <= Fraction(1, 2 ** 40) * (1 + abs(exact))


def test_moe_ffn_matches_dense_per_expert_path():
    """All tokens routed to the same experts: the routed FFN equals the dense
    gate/up -> SwiGLU -> down computation per expert, weighted."""
    fmt = "q4_0"
    gate = _tiny_experts(fmt, 3, 32, 64, 10)
    up = _tiny_experts(fmt, 3, 32, 64, 11)
    down = _tiny_experts(fmt, 3, 64, 32, 12)
    x = S.activations((92, 3, 0), 64, 2)
    ids = np.array([[2, 0], [2, 0]], np.int32)
    rw = np.array([[0.625, 0.375], [0.625, 0.375]], np.float32)
    y, _, _, _, _ = R.moe_ffn(fmt, gate, up, down, x, ids, rw)
    for t in range(2):
        acc = np.zeros(64)
        for j, e in enumerate(ids[t]):
            g = F.dequantize(fmt, gate[e]) @ x[t].astype(np.float64)
            u = F.dequantize(fmt, up[e]) @ x[t].astype(np.float64)
            h = (g / (1 + np.exp(-g)) * u).astype(np.float16).astype(np.float64)
            acc = acc + float(rw[t, j]) * (F.dequantize(fmt, down[e]) @ h)
        np.testing.assert_allclose(y[t], acc, rtol=1e-12, atol=1e-12)


def test_route_table_shape_and_normalisation():
    ids, rw = S.route_table(5, 16, 128, 8)
    assert ids.shape == (16, 8) and rw.shape == (16, 8)
    for t in range(16):
        assert len(set(ids[t].tolist())) == 8
        assert abs(float(rw[t].astype(np.float64).sum()) - 1.0) < 1e-6
    assert ids.min() >= 0 and ids.max() < 128
