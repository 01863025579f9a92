"""The library's host packer (kq_pack, C++) against the oracle: packed bytes
must be identical (bit-exact), for seeded matrices and for edge blocks."""
import numpy as np
import pytest

import block_quantized_gemv_kq_amd as kq
from oracle import formats as F
from synth import inputs as S
from tests import golden_blocks as G

FMTS = ("q8_0", "q4_0", "affine4")


@pytest.mark.parametrize("blk", G.all_blocks(), ids=lambda b: b["name"])
def test_golden_blocks_through_c_packer(blk):
    got = kq.kq_pack(blk["format"], blk["weights"][None, :])[0]
    assert got.tobytes() == blk["bytes"].tobytes()
    back = kq.kq_unpack(blk["format"], blk["bytes"], 1, 32)[0]
    assert np.array_equal(back.astype(np.float64), blk["dequant"])


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("seed", [0, 1])
def test_seeded_matrix_bytes_identical(fmt, seed):
    W = S.weights((91, seed, 0, 0), 257, 1024)
    assert np.array_equal(kq.kq_pack(fmt, W, n_threads=4), F.pack(fmt, W))


def _edge_blocks():
    """Blocks that stress every branch: zero/constant blocks, signed zeros,
    |w| ties of opposite sign, exact .5 quotients, tiny (subnormal-scale)
    blocks, huge blocks near the fp16 limit, single spikes."""
    rng = np.random.default_rng(1234)
    rows = []
    rows.append(np.zeros(32))
    rows.append(-np.zeros(32))
    z = np.zeros(32)
    z[::2] = -0.0
    rows.append(z)
    rows.append(np.full(32, 0.37))
    rows.append(np.full(32, -1.5))
    t = np.zeros(32)
    t[3], t[17] = 0.5, -0.5
    rows.append(t)
    t = np.zeros(32)
    t[0], t[31] = -0.25, 0.25
    rows.append(t)
    rows.append(np.arange(32) - 15.5)
    rows.append((np.arange(32) - 16) * 2.0 ** -20)
    rows.append(rng.standard_normal(32) * 1e-7)
    rows.append(rng.standard_normal(32) * 1e-5)
    rows.append(rng.standard_normal(32) * 3e3)
    rows.append(np.linspace(-60000, 60000, 32))
    s = np.zeros(32)
    s[7] = 1.0
    rows.append(s)
    s = np.zeros(32)
    s[7] = -1.0
    rows.append(s)
    for k in range(8):
        rows.append(np.round(rng.standard_normal(32) * 8) / 8)  # many exact ties
        rows.append(rng.uniform(-1, 1, 32) * 10.0 ** rng.integers(-6, 4))
    return np.stack(rows).astype(np.float32)


@pytest.mark.parametrize("fmt", FMTS)
def test_edge_blocks_bytes_identical(fmt):
    E = _edge_blocks()
    W = E.reshape(-1, 64) if E.shape[0] % 2 == 0 else E
    assert np.array_equal(kq.kq_pack(fmt, W), F.pack(fmt, W))


@pytest.mark.parametrize("fmt", FMTS)
def test_unpack_matches_oracle_dequant(fmt):
    W = S.weights((90, 0, 0, 0), 33, 320)
    p = kq.kq_pack(fmt, W)
    back = kq.kq_unpack(fmt, p, 33, 320)
    ref = F.dequantize(fmt, F.decode(fmt, p, 33, 320))
    assert np.array_equal(back.astype(np.float64), ref)


def test_q4_1_is_the_affine4_block():
    """Q4_1 read as Q5_1 with four bits is the affine4 gs32 block: the same
    enum value, the same bytes from the packer, the affine4 golden blocks
    under the Q4_1 name."""
    assert kq.KQ_Q4_1 == kq.KQ_AFFINE4_G32 and kq.FORMATS["q4_1"] == kq.KQ_AFFINE4_G32
    assert kq.kq_block_bytes("q4_1") == 20
    W = S.weights((92, 0, 0, 0), 33, 512)
    assert np.array_equal(kq.kq_pack("q4_1", W), kq.kq_pack("affine4", W))
    for blk in G.all_blocks():
        if blk["format"] == "affine4":
            assert kq.kq_pack("q4_1", blk["weights"][None, :])[0].tobytes() == blk["bytes"].tobytes()


def test_multithreaded_pack_identical():
    W = S.weights((89, 0, 0, 0), 1000, 2048)
    a = kq.kq_pack("affine4", W, n_threads=1)
    b = kq.kq_pack("affine4", W, n_threads=7)
    assert np.array_equal(a, b)


def test_fp16_conversion_exhaustive_near_range():
    """The packer's own fp32->fp16 against numpy's cast, on EVERY fp32 bit
    pattern whose exponent lies in or near fp16's range (underflow to zero,
    subnormals, normals, overflow), both signs, plus a stride over all 2^32
    patterns. Checked one exponent at a time to bound memory."""
    mant = np.arange(0, 1 << 23, dtype=np.uint32)
    chunks = [np.uint32(e) << np.uint32(23) | mant for e in range(95, 146)]
    chunks.append(np.arange(0, 1 << 32, 4099, dtype=np.uint64).astype(np.uint32))
    for u in chunks:
        for sign in (np.uint32(0), np.uint32(0x80000000)):
            f = (u | sign).view(np.float32)
            f = f[~np.isnan(f)]
            with np.errstate(over="ignore"):
                want = f.astype(np.float16).view(np.uint16)
            got = kq.kq_f32_to_f16(f)
            bad = np.nonzero(got != want)[0]
            assert bad.size == 0, f"{bad.size} mismatches, first {f[bad[0]]!r}: {got[bad[0]]:#x} vs {want[bad[0]]:#x}"


# ------------------------------------------------------- Shortlist bound copy
from oracle import shortlist as SL  # noqa: E402


@pytest.mark.parametrize("row", G.all_shortlist_rows(), ids=lambda r: r["name"])
def test_shortlist_golden_rows_through_c_packer(row):
    q8 = F.encode("q8_0", row["fields"])
    got = kq.kq_shortlist_pack(q8, 1, row["k"])
    assert got.tobytes() == row["bytes"].tobytes()


def _raw_q8(n, k, seed):
    """Q8_0 bytes with every int8 (including -128) and scales across fp16's
    range: subnormal, tiny, ordinary, huge, zero."""
    rng = np.random.default_rng(seed)
    nb = k // 32
    d = rng.choice(np.array([0.0, 2.0 ** -24, 3 * 2.0 ** -20, 1e-3, 0.02, 1.0, 300.0, 65504.0], np.float16),
                   size=(n, nb))
    q = rng.integers(-128, 128, size=(n, nb, 32)).astype(np.int8)
    return F.encode("q8_0", {"d": d, "q": q}), {"d": d, "q": q}


@pytest.mark.parametrize("n,k,seed", [(3, 256, 0), (17, 512, 1), (64, 2560, 2), (5, 16384, 3)])
def test_shortlist_copy_bytes_identical(n, k, seed):
    q8, fields = _raw_q8(n, k, seed)
    got = kq.kq_shortlist_pack(q8, n, k)
    assert got.tobytes() == SL.encode_bound_copy(fields).tobytes()


def test_shortlist_copy_of_seeded_layer_identical():
    W = S.weights((92, 0, 0, 0), 300, 2560)
    q8 = kq.kq_pack("q8_0", W)
    got = kq.kq_shortlist_pack(q8, 300, 2560)
    assert got.tobytes() == SL.encode_bound_copy(F.decode("q8_0", q8, 300, 2560)).tobytes()


def test_shortlist_pack_multithreaded_identical():
    q8, _ = _raw_q8(4096, 512, 9)
    one = kq.kq_shortlist_pack(q8, 4096, 512, n_threads=1)
    many = kq.kq_shortlist_pack(q8, 4096, 512, n_threads=8)
    assert one.tobytes() == many.tobytes()
