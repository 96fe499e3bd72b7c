"""Pins for the oracle's FP8 tier (ai-automate.fr, section on Minima-KV: recent
pages kept in FP8 beside low-bit older pages, merged by one online softmax):
the e4m3 encoder, formula F8 per token row, the record layout, and which
blocks attention reads through FP8."""
import math

import numpy as np
import pytest

from oracle import kivi


def _brute_e4m3(y):
    """Nearest finite e4m3 code by exhaustive search, ties to the even code."""
    best, bestd = None, None
    for c in range(256):
        if c & 0x7f == 0x7f:
            continue
        v = float(kivi.e4m3_value(np.array([c]))[0])
        if (v == 0.0) and (np.signbit(y) != bool(c & 0x80)):
            continue   # zero keeps the sign of y
        d = abs(v - y)
        if best is None or d < bestd or (d == bestd and c % 2 == 0 and best % 2 == 1):
            best, bestd = c, d
    return best


def test_e4m3_values_by_hand():
    v = kivi.e4m3_value(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x7e, 0xb8, 0x80]))
    assert list(v) == [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 448.0, -1.0, -0.0]


def test_e4m3_encoder_is_the_nearest_code():
    rng = np.random.default_rng(31)
    ys = list(rng.uniform(-448, 448, 300)) + list(rng.uniform(-0.05, 0.05, 300))
    # exact midpoints between neighbours, which must go to the even code
    mids = [(kivi.e4m3_value(np.array([c]))[0] + kivi.e4m3_value(np.array([c + 1]))[0]) / 2 for c in range(0, 0x7e)]
    ys += mids + [-m for m in mids] + [0.0, -0.0, 448.0, -448.0, 2.0 ** -10, 3 * 2.0 ** -11]
    got = kivi.e4m3_encode(np.array(ys))
    for y, c in zip(ys, got):
        assert c == _brute_e4m3(y), (y, c)


def test_f8_exact_when_the_scale_is_a_power_of_two():
    # row maximum 1.75 = 448 * 2^-8: the scale is exactly 2^-8 and every value
    # that is an e4m3 value times 2^-8 comes back unchanged
    rng = np.random.default_rng(32)
    codes = rng.integers(0, 0x7f, size=(6, 64))
    codes |= rng.integers(0, 2, size=(6, 64)) << 7
    x = (kivi.e4m3_value(codes) * 2.0 ** -8).astype(np.float32)
    x[:, 5] = 1.75
    c, s = kivi.quantize_fp8_rows(x)
    assert np.all(s == np.float16(2.0 ** -8))
    assert np.array_equal(kivi.e4m3_value(c) * 2.0 ** -8, x.astype(np.float64))


def test_f8_error_bound_and_extremes():
    rng = np.random.default_rng(33)
    x = (rng.standard_normal((50, 128)) * np.exp(rng.uniform(-6, 6, (50, 1)))).astype(np.float32)
    c, s = kivi.quantize_fp8_rows(x)
    xh = kivi.e4m3_value(c) * s.astype(np.float64)[:, None]
    a = np.abs(x).max(axis=1, keepdims=True).astype(np.float64)
    err = np.abs(xh - x)
    assert np.all(err <= 2.0 ** -4 * np.abs(x) + 2.0 ** -9 * s.astype(np.float64)[:, None] + 2.0 ** -10 * a)
    # the row maximum encodes to +-448
    i = np.argmax(np.abs(x), axis=1)
    assert np.all((c[np.arange(50), i] & 0x7f) == 0x7e)
    # an all-zero row: scale 0, codes 0
    c0, s0 = kivi.quantize_fp8_rows(np.zeros((1, 16), np.float32))
    assert s0[0] == 0 and not np.any(c0)


def test_fp8_record_layout():
    rng = np.random.default_rng(34)
    k = rng.standard_normal((32, 128)).astype(np.float32)
    v = rng.standard_normal((32, 128)).astype(np.float32)
    rec = kivi.fp8_record(k, v)
    spec = kivi.CacheSpec(1, 1, 1, 128, 2, 2, 32, 32, 8, 48, "f16", fp8_blocks=2)
    assert rec.size == kivi.fp8_record_bytes(spec) == 2 * 32 * 128 + 4 * 32
    kc, ks = kivi.quantize_fp8_rows(k)
    assert np.array_equal(rec[:4096], kc.ravel())
    assert np.array_equal(rec[4096:4160].view(np.float16), ks)
    assert np.array_equal(rec[4160:8256], kivi.quantize_fp8_rows(v)[0].ravel())


def test_fp8_window_blocks():
    spec = kivi.CacheSpec(1, 1, 1, 16, 2, 2, 16, 16, 8, 40, "f16", fp8_blocks=3)
    assert kivi.fp8_window(spec, 7) == (0, 0)
    assert kivi.fp8_window(spec, 8 + 16 * 2) == (0, 2)     # two blocks, both in FP8
    assert kivi.fp8_window(spec, 8 + 16 * 5) == (2, 5)     # five blocks, the last three in FP8


def test_fp8_blocks_are_read_exactly_when_representable():
    # identical keys: the output is the mean of the value rows. Value rows that
    # F8 reproduces exactly (scale 2^-8) come back exact through the FP8 tier,
    # and visibly not through the INT2 records.
    rng = np.random.default_rng(35)
    S, d, G, R = 8 + 16 * 3, 16, 16, 8
    codes = rng.integers(0, 0x7f, size=(S, d)) | (rng.integers(0, 2, size=(S, d)) << 7)
    V = (kivi.e4m3_value(codes) * 2.0 ** -8).astype(np.float32)
    V[:, 0] = 1.75
    # one key row for every token, itself exact through F8 (and constant channels are exact in INT2)
    krow = (kivi.e4m3_value(rng.integers(0, 0x7f, size=(1, d))) * 2.0 ** -8).astype(np.float32)
    krow[0, 0] = 1.75
    K = np.tile(krow, (S, 1))
    q = rng.standard_normal((1, 1, d)).astype(np.float16).astype(np.float32)
    mk = lambda W: kivi.CacheSpec(1, 1, 1, d, 2, 2, G, 16, R, R + G + 16, "f16", fp8_blocks=W)
    out = kivi.decode_attention(mk(3), q, K[None, None], V[None, None], [S])
    assert np.max(np.abs(out[0, 0] - V.astype(np.float64).mean(axis=0))) < 1e-13
    out0 = kivi.decode_attention(mk(0), q, K[None, None], V[None, None], [S])
    assert np.max(np.abs(out0[0, 0] - V.astype(np.float64).mean(axis=0))) > 1e-3
    # W = 1: only the newest block through FP8, the two older ones through INT2
    out1 = kivi.decode_attention(mk(1), q, K[None, None], V[None, None], [S])
    assert not np.allclose(out1, out, atol=1e-6) and not np.allclose(out1, out0, atol=1e-6)


def test_f8_divides_by_the_stored_fp16_scale():
    # the codes are those of x / s16 with s16 the stored fp16 scale (not the
    # unrounded max/448), each found by exhaustive search
    rng = np.random.default_rng(36)
    x = (rng.standard_normal((40, 16)) * np.exp(rng.uniform(-3, 3, (40, 1)))).astype(np.float32)
    c, s = kivi.quantize_fp8_rows(x)
    a = np.abs(x).max(axis=1)
    s16 = (a / np.float32(448)).astype(np.float32).astype(np.float16)
    assert np.array_equal(s, s16)
    changed = 0
    for r in range(40):
        y = np.clip(x[r] / np.float32(s16[r]), -448, 448).astype(np.float32)
        ref = [_brute_e4m3(float(t)) for t in y]
        assert list(c[r]) == ref
        y_unrounded = np.clip(x[r] / (a[r] / np.float32(448)), -448, 448).astype(np.float32)
        changed += sum(int(_brute_e4m3(float(t)) != rc) for t, rc in zip(y_unrounded, ref))
    assert changed > 0   # the fp16 rounding of the scale matters for some codes
