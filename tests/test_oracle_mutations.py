"""Planted mistakes in the oracle (on the CPU): each plausible slip must make
at least one pin in tests/test_oracle.py fail. This shows the pins can tell a
wrong oracle from a right one."""
import numpy as np
import pytest

from oracle import formats as F
from oracle import ref as R
from tests import test_oracle as T


def _fails(check, *args) -> bool:
    try:
        check(*args)
    except AssertionError:
        return True
    return False


def _any_golden_fails(fmt=None) -> bool:
    return any(_fails(T.check_golden_block, b) for b in T.BLOCKS if fmt is None or b["format"] == fmt)


def test_half_even_rounding_is_caught(monkeypatch):
    monkeypatch.setattr(F, "round_half_away", lambda v: np.round(np.asarray(v, np.float64)))
    assert _any_golden_fails("q8_0")


def test_naive_fp32_rounding_is_caught():
    # trunc(v + 0.5f) in fp32 rounds 0.5 - 2^-25 up to 1.
    v = np.float32(0.5 - 2.0 ** -25)
    assert np.trunc(v + np.float32(0.5)) == 1.0
    assert F.round_half_away(v) == 0.0


def test_swapped_nibble_order_is_caught(monkeypatch):
    monkeypatch.setattr(F, "_nibbles", lambda q: (q[..., 16:] | (q[..., :16] << 4)).astype(np.uint8))
    monkeypatch.setattr(F, "_unnibble", lambda nb: np.concatenate([nb >> 4, nb & 0x0F], -1).astype(np.uint8))
    assert _any_golden_fails("q4_0") and _any_golden_fails("affine4")


def test_sequential_nibble_pairs_are_caught(monkeypatch):
    monkeypatch.setattr(F, "_nibbles", lambda q: (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8))
    assert _any_golden_fails("q4_0")


def test_last_index_signed_max_is_caught(monkeypatch):
    orig = F._first_index_value

    def last(B, key, pick_max):
        rb, rk = B[..., ::-1], key[..., ::-1]
        return orig(rb, rk, pick_max)
    monkeypatch.setattr(F, "_first_index_value", last)
    assert _any_golden_fails("q4_0")


def test_positive_scale_q4_0_is_caught(monkeypatch):
    orig = F.to_f16
    monkeypatch.setattr(F, "to_f16", lambda v: np.abs(orig(v)))
    assert _any_golden_fails("q4_0")


def test_fp32_scale_for_quants_is_caught(monkeypatch):
    # quants computed from the unrounded fp32 scale/bias (the stored bytes are
    # still rounded to fp16 by encode)
    monkeypatch.setattr(F, "to_f16", lambda v: np.asarray(v, np.float32))
    assert _any_golden_fails("affine4")


def test_dropped_q4_0_offset_is_caught(monkeypatch):
    orig = F.dequantize

    def bad(fmt, fields, rows=None):
        if fmt == "q4_0":
            f2 = dict(fields)
            f2["q"] = fields["q"].astype(np.int32) + 8     # w' = d*q instead of d*(q-8)
            return orig(fmt, f2, rows)
        return orig(fmt, fields, rows)
    monkeypatch.setattr(F, "dequantize", bad)
    assert _fails(T.check_unit_vectors, "q4_0")


def test_dropped_affine_bias_is_caught(monkeypatch):
    orig = F.dequantize

    def bad(fmt, fields, rows=None):
        if fmt == "affine4":
            f2 = dict(fields)
            f2["b"] = np.zeros_like(fields["b"])
            return orig(fmt, f2, rows)
        return orig(fmt, fields, rows)
    monkeypatch.setattr(F, "dequantize", bad)
    assert _fails(T.check_unit_vectors, "affine4")


def test_transposed_operand_is_caught(monkeypatch):
    orig = R.gemv

    def bad(fmt, fields, x16, rows=None):
        y, a = orig(fmt, fields, x16, rows)
        return y[:, ::-1], a[:, ::-1]          # rows scrambled
    monkeypatch.setattr(R, "gemv", bad)
    assert _fails(T.check_exact_small_gemv, "q8_0", 5, 96, 2, 2)


def test_wrong_sign_in_dot_is_caught(monkeypatch):
    orig = R.gemv

    def bad(fmt, fields, x16, rows=None):
        y, a = orig(fmt, fields, x16, rows)
        return -y, a
    monkeypatch.setattr(R, "gemv", bad)
    assert _fails(T.check_ones_sum, "affine4")


def test_dropped_block_is_caught(monkeypatch):
    orig = F.dequantize

    def bad(fmt, fields, rows=None):
        w = orig(fmt, fields, rows)
        if w.shape[1] > 32:
            w[:, -32:] = 0
        return w
    monkeypatch.setattr(F, "dequantize", bad)
    assert _fails(T.check_exact_small_gemv, "q4_0", 3, 64, 1, 1)


def test_loose_relative_tolerance_is_caught(monkeypatch):
    monkeypatch.setattr(R, "REL_TOL", 2e-2)
    assert _fails(T.check_acceptance_bound)


def test_loose_absolute_tolerance_is_caught(monkeypatch):
    monkeypatch.setattr(R, "ABS_TOL", 1e-3)
    assert _fails(T.check_acceptance_bound)


def test_dropped_relative_term_is_caught(monkeypatch):
    monkeypatch.setattr(R, "tolerance", lambda abs_dot: np.zeros_like(np.asarray(abs_dot, np.float64)) + R.ABS_TOL)
    assert _fails(T.check_acceptance_bound)


def test_strict_comparison_is_caught(monkeypatch):
    # a bound applied to twice the difference (e.g. a relative error taken
    # against the midpoint of y and y_ref) rejects results the bar accepts
    orig = R.tolerance
    monkeypatch.setattr(R, "tolerance", lambda abs_dot: orig(abs_dot) / 2)
    assert _fails(T.check_acceptance_bound)


def test_error_ratio_against_reference_magnitude_is_caught(monkeypatch):
    def bad(y_gpu, y_ref, abs_dot):
        d = np.abs(np.asarray(y_gpu, np.float64) - y_ref)
        return float(np.max(d / np.maximum(np.abs(y_ref), 1e-300)))
    monkeypatch.setattr(R, "error_ratio", bad)
    assert _fails(T.check_error_ratio)


def test_abs_of_sum_instead_of_sum_of_abs_is_caught(monkeypatch):
    orig = R.gemv

    def bad(fmt, fields, x16, rows=None):
        y, _ = orig(fmt, fields, x16, rows)
        return y, np.abs(y)
    monkeypatch.setattr(R, "gemv", bad)
    assert _fails(T.check_abs_dot, "affine4")


def test_reversed_fifth_bit_order_is_caught(monkeypatch):
    orig_h, orig_u = F._high_bits, F._unhigh_bits
    monkeypatch.setattr(F, "_high_bits", lambda q: orig_h(q[..., ::-1]))
    monkeypatch.setattr(F, "_unhigh_bits", lambda b4: orig_u(b4)[..., ::-1])
    assert _any_golden_fails("q5_0") and _any_golden_fails("q5_1")


def test_dropped_fifth_bit_is_caught(monkeypatch):
    orig = F.decode

    def bad(fmt, packed, n, k):
        f = orig(fmt, packed, n, k)
        if fmt in ("q5_0", "q5_1"):
            f = dict(f)
            f["q"] = f["q"] & 0x0F
        return f
    monkeypatch.setattr(F, "decode", bad)
    assert _any_golden_fails("q5_0") and _any_golden_fails("q5_1")


def test_q5_0_offset_15_is_caught(monkeypatch):
    orig = F.dequantize

    def bad(fmt, fields, rows=None):
        if fmt == "q5_0":
            f2 = dict(fields)
            f2["q"] = fields["q"].astype(np.int32) + 1      # w' = d*(q-15)
            return orig(fmt, f2, rows)
        return orig(fmt, fields, rows)
    monkeypatch.setattr(F, "dequantize", bad)
    assert _fails(T.check_unit_vectors, "q5_0")


def test_q5_1_dropped_minimum_is_caught(monkeypatch):
    orig = F.dequantize

    def bad(fmt, fields, rows=None):
        if fmt == "q5_1":
            f2 = dict(fields)
            f2["m"] = np.zeros_like(fields["m"])
            return orig(fmt, f2, rows)
        return orig(fmt, fields, rows)
    monkeypatch.setattr(F, "dequantize", bad)
    assert _fails(T.check_unit_vectors, "q5_1")


def test_q5_1_fifteen_steps_is_caught(monkeypatch):
    # the 4-bit step (hi - lo) / 15 planted in the 5-bit format
    orig = F.quantize

    def bad(fmt, W):
        if fmt != "q5_1":
            return orig(fmt, W)
        f = orig("affine4", W)
        return {"d": f["s"], "m": f["b"], "q": f["q"]}
    monkeypatch.setattr(F, "quantize", bad)
    assert _any_golden_fails("q5_1")


# ------------------------------------------------------------- Shortlist
from oracle import shortlist as SL  # noqa: E402
from tests import test_oracle_shortlist as TS  # noqa: E402


def test_shortlist_centre_4_is_caught(monkeypatch):
    monkeypatch.setattr(SL, "SPLIT_CENTRE", 4.0)
    assert _fails(TS.check_bound_exact, TS._q8(4, 256, seed=200), TS._x(256, 300))


def test_shortlist_norm_rounded_to_nearest_is_caught(monkeypatch):
    import math

    def nearest(d_row, ql_row):
        d = np.asarray(d_row, np.float16).astype(np.float64)
        Q = ((2 * np.asarray(ql_row, np.int64) - 7) ** 2).sum(axis=-1)
        return np.float32(math.sqrt(math.fsum((d * d) * (Q / 4.0))))
    monkeypatch.setattr(SL, "residual_norm_up", nearest)
    assert any(_fails(TS.check_golden_row, r) for r in TS.ROWS)


def test_shortlist_split_toward_zero_is_caught(monkeypatch):
    def trunc_split(q):
        qi = np.asarray(q).astype(np.int64)
        v = np.trunc(qi / 8).astype(np.int64) + 16
        return v.astype(np.uint8), (qi - 8 * (v - 16)).astype(np.uint8)
    monkeypatch.setattr(SL, "split_quants", trunc_split)
    assert _fails(TS.check_split_every_int8)


def test_shortlist_dropped_fifth_bit_is_caught(monkeypatch):
    monkeypatch.setattr(F, "_high_bits", lambda q: np.zeros(q.shape[:-1] + (4,), np.uint8))
    assert any(_fails(TS.check_golden_row, r) for r in TS.ROWS)


def test_shortlist_l1_radius_is_caught(monkeypatch):
    orig = SL.bound_terms

    def l1(bound, x16):
        t = orig(bound, x16)
        x = np.asarray(x16, np.float16).astype(np.float64)
        l2 = np.sqrt((x * x).sum())
        scale = np.abs(x).sum() / l2 if l2 else 1.0
        t["r"] = t["r"] * scale
        return t
    monkeypatch.setattr(SL, "bound_terms", l1)
    assert _fails(TS.check_equality_case)


def test_shortlist_dropped_centre_term_is_caught(monkeypatch):
    monkeypatch.setattr(SL, "SPLIT_CENTRE", 0.0)
    assert _fails(TS.check_yhat_block_constant)
