"""Pins of the oracle's fp8 query quantisation (the fp8-q scoring path).

The encoder is checked against things it does not compute itself: a brute
force nearest-value search over all finite e4m3fn values, the midpoints
between neighbouring codes (ties go to the even code), the format's half-ulp
error bound, and what the per-row scale guarantees (the row's largest
magnitude lands exactly on 448; an all-zero row stays zero).
"""
import numpy as np
import pytest

import oracle

FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
VALUES = oracle.e4m3fn_to_f64(FINITE)


def brute_nearest(x):
    """Code of the nearest finite e4m3fn value; ties -> even code (mantissa LSB 0),
    -0.0 -> code 0x80; past 448 -> 448."""
    out = np.empty(len(x), dtype=np.uint8)
    for i, v in enumerate(np.asarray(x, dtype=np.float64)):
        v = min(max(v, -448.0), 448.0)
        d = np.abs(VALUES - v)
        best = np.flatnonzero(d == d.min())
        best = [c for c in FINITE[best] if (c >> 7) == (1 if np.signbit(v) else 0)] or list(FINITE[best])
        even = [c for c in best if (c & 1) == 0]
        out[i] = (even or best)[0]
    return out


def test_encoder_matches_brute_force_nearest():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(3000) * 40.0,
        rng.standard_normal(1000) * 0.01,            # subnormal range
        rng.uniform(-460.0, 460.0, 1000),            # near and past the top
        np.array([0.0, -0.0, 2.0 ** -10, -(2.0 ** -10), 448.0, -448.0]),
    ]).astype(np.float32)
    np.testing.assert_array_equal(oracle.f32_to_e4m3fn_rne(x), brute_nearest(x))


def test_midpoints_round_to_the_even_code():
    pos = np.sort(VALUES[(VALUES > 0) & np.isfinite(VALUES)])
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (pos[:-1] + pos[1:]) / 2)   # exact in float32
    codes = oracle.f32_to_e4m3fn_rne(mids)
    assert np.all((codes & 1) == 0)
    got = oracle.e4m3fn_to_f64(codes)
    assert np.all((got == pos[:-1]) | (got == pos[1:]))


def test_quantised_rows_within_half_an_ulp_and_max_on_448():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((64, 8, 128)).astype(np.float32) * rng.uniform(0.01, 50.0, (64, 8, 1)).astype(np.float32)
    bits = (q.view(np.uint32) >> 16).astype(np.uint16)          # bf16 by truncation (any bf16 values will do)
    qf = oracle.bf16_bits_to_f64(bits)
    codes, s = oracle.quantize_q_e4m3(bits)
    assert codes.shape == bits.shape and s.shape == bits.shape[:-1] and s.dtype == np.float32
    deq = oracle.dequantize_q_e4m3(codes, s)
    x = qf / s[..., None].astype(np.float64)                     # the value that was rounded (up to 2^-24)
    normal = np.abs(x) >= 2.0 ** -6
    err = np.abs(deq / s[..., None] - x)
    assert np.all(err[normal] <= np.abs(x[normal]) * 2.0 ** -4 * (1 + 2.0 ** -20))
    assert np.all(err[~normal] <= 2.0 ** -10 * (1 + 2.0 ** -20))
    # the largest magnitude of each row is encoded as +-448 exactly
    am = np.argmax(np.abs(qf), axis=-1)
    top = np.take_along_axis(codes, am[..., None], axis=-1)[..., 0]
    assert np.all((top & 0x7F) == 0x7E)


def test_zero_row_and_representable_rows():
    codes, s = oracle.quantize_q_e4m3(np.zeros((3, 128), dtype=np.uint16))
    assert np.all(codes == 0) and np.all(s == 1.0)
    # a row that is already codes * s (with the max on 448) quantises back to the same codes
    rng = np.random.default_rng(8)
    c0 = rng.choice(FINITE[(FINITE & 0x7F) < 0x70], size=(4, 128)).astype(np.uint8)
    c0[:, 0] = 0x7E
    x = oracle.e4m3fn_to_f64(c0) * 2.0 ** -7                      # exact in bf16 (<= 4 significant bits)
    bits = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.all(oracle.bf16_bits_to_f64(bits) == x)
    codes, s = oracle.quantize_q_e4m3(bits)
    assert np.all(s == np.float32(2.0 ** -7))
    np.testing.assert_array_equal(codes, c0)


@pytest.mark.parametrize("bad", [0x10, 0x01])
def test_a_planted_encoder_mistake_is_caught(monkeypatch, bad):
    """Plant a mistake in the encoder (truncation instead of rounding, or a
    shifted subnormal step) and check that the brute-force pin fails."""
    real = oracle.f32_to_e4m3fn_rne

    def wrong(x):
        c = real(x)
        x64 = np.asarray(x, dtype=np.float64)
        if bad == 0x10:      # rounding toward zero in the normal range
            t = oracle.e4m3fn_to_f64(c)
            over = (np.abs(t) > np.abs(x64)) & (np.abs(x64) >= 2.0 ** -6) & ((c & 0x7F) > 0x08)
            c = np.where(over, c - 1, c).astype(np.uint8)
        else:                # subnormal codes off by one
            sub = (c & 0x7F) < 0x08
            c = np.where(sub & ((c & 0x7F) > 0), c - 1, c).astype(np.uint8)
        return c

    x = np.random.default_rng(9).standard_normal(2000).astype(np.float32) * np.float32(0.02 if bad == 0x01 else 30.0)
    assert not np.array_equal(wrong(x), brute_nearest(x))
