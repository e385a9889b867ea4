"""Pins for the oracle's element formats and MX quantizer.

The pages name the E2M1 payload, power-of-two (E8M0) block scales and FP8 operands
(gist.science summary: Problem Statement; Methodology 1 "Format Selection"; Methodology 2
"Gradient Formats") without defining them; the values below are the OCP Microscaling v1.0
definitions, written out as literal tables so that a wrong bias, bit order or subnormal rule
in the oracle fails here.
"""
import math
import random

import numpy as np
import pytest

# OCP MX v1.0: E2M1 magnitudes for codes 0..7 (bit 3 = sign).
E2M1_LITERAL = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]

# OCP FP8 E4M3 (FN): selected code points.
E4M3_POINTS = {
    0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5, 0x38: 1.0,
    0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x77: 240.0, 0x78: 256.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0,
}


def test_e2m1_table(orc):
    for c in range(8):
        assert orc.e2m1_decode(c) == E2M1_LITERAL[c]
        neg = orc.e2m1_decode(c | 8)
        assert neg == -E2M1_LITERAL[c] and math.copysign(1.0, neg) == -1.0


def test_e4m3_points_and_monotone(orc):
    for c, v in E4M3_POINTS.items():
        assert orc.e4m3_decode(c) == v, hex(c)
    assert math.isnan(orc.e4m3_decode(0x7F)) and math.isnan(orc.e4m3_decode(0xFF))
    assert math.copysign(1.0, orc.e4m3_decode(0x80)) == -1.0
    mags = [orc.e4m3_decode(c) for c in range(127)]
    assert all(b > a for a, b in zip(mags, mags[1:]))
    finite = [c for c in range(256) if not math.isnan(orc.e4m3_decode(c))]
    assert len(finite) == 254


def test_e8m0(orc):
    assert orc.e8m0_decode(127) == 1.0
    assert orc.e8m0_decode(0) == 2.0 ** -127
    assert orc.e8m0_decode(254) == 2.0 ** 127
    assert math.isnan(orc.e8m0_decode(255))


def test_round_trip_all_codes(orc):
    for c in range(16):
        assert orc.e2m1_encode(orc.e2m1_decode(c)) == c
    for c in range(256):
        v = orc.e4m3_decode(c)
        if not math.isnan(v):
            assert orc.e4m3_encode(v) == c, hex(c)


def _brute_nearest(x, values):
    """Brute force: nearest magnitude over every non-negative code; ties to the even code;
    the sign is kept; saturation at the largest magnitude."""
    sign = math.copysign(1.0, x) < 0
    a = abs(x)
    best, bestd = None, None
    for c, v in enumerate(values):
        d = abs(a - v)
        if best is None or d < bestd or (d == bestd and c % 2 == 0):
            best, bestd = c, d
    return best, sign


@pytest.mark.parametrize("fmt", ["e2m1", "e4m3"])
def test_encoder_matches_brute_force(orc, fmt):
    if fmt == "e2m1":
        values = E2M1_LITERAL
        enc, sbit, top = orc.e2m1_encode, 8, 6.0
    else:
        values = [orc.e4m3_decode(c) for c in range(127)]
        enc, sbit, top = orc.e4m3_encode, 128, 448.0
    rng = random.Random(7)
    xs = []
    # exact midpoints (ties) and their neighbours
    for a, b in zip(values, values[1:]):
        mid = 0.5 * (a + b)
        xs += [mid, math.nextafter(mid, 0.0), math.nextafter(mid, math.inf), -mid]
    xs += [rng.uniform(-1.5 * top, 1.5 * top) for _ in range(4000)]
    xs += [rng.uniform(-1, 1) * 2.0 ** rng.randint(-14, 2) for _ in range(2000)]
    xs += [0.0, -0.0, -1e-30, 1e-30, top, -top, 2 * top, 1e9, -1e9]
    for x in xs:
        mag, neg = _brute_nearest(x, values)
        if abs(x) > top:  # saturation
            mag = len(values) - 1
        want = mag | (sbit if neg else 0)
        assert enc(x) == want, (fmt, x)


def test_negative_underflow_keeps_sign(orc):
    assert orc.e2m1_encode(-0.1) == 8
    assert orc.e2m1_encode(-0.25) == 8  # tie at 0.25 rounds to zero, sign kept
    assert orc.e4m3_encode(-2.0 ** -11) == 0x80
    assert orc.e2m1_encode(-0.0) == 8


def test_mx_block_exponent_binades(orc):
    # floor(log2 amax) - emax, from the binade of amax
    for k in range(-120, 120, 7):
        for f in (1.0, 1.25, 1.999):
            amax = f * 2.0 ** k
            assert orc.mx_block_exponent(amax, orc.FMT_E2M1) == max(-127, min(127, k - 2))
            assert orc.mx_block_exponent(amax, orc.FMT_E4M3) == max(-127, min(127, k - 8))
            # the block max then lands in the top binade of the element format
            e = orc.mx_block_exponent(amax, orc.FMT_E2M1)
            if k - 2 > -127:
                assert 4.0 <= amax / 2.0 ** e < 8.0
    assert orc.mx_block_exponent(0.0, orc.FMT_E2M1) == -127
    assert orc.mx_block_exponent(2.0 ** -140, orc.FMT_E2M1) == -127
    assert orc.mx_block_exponent(2.0 ** 200, orc.FMT_E4M3) == 127


def _bf16(vals):
    from precision_attention_amd.inputs import f32_to_bf16_bits

    return f32_to_bf16_bits(np.asarray(vals, np.float32))


def test_mx_quantize_blocks_brute_force(orc):
    rng = np.random.default_rng(3)
    rows = []
    rows.append(rng.standard_normal(64).astype(np.float32))
    rows.append(np.zeros(64, np.float32))  # all-zero blocks: scale 2^-127, every code zero
    sub = np.float32(2.0 ** -130) * rng.standard_normal(64).astype(np.float32)  # bf16 subnormals
    rows.append(sub)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0] * 8, np.float32) * np.float32(0.5)
    rows.append(ties)
    rows.append(np.float32(1000.0) * rng.standard_normal(64).astype(np.float32))
    rows.append(-np.abs(rng.standard_normal(64).astype(np.float32)) * np.float32(1e-3))
    x = _bf16(np.stack(rows))  # [6, 64] bf16 bits
    xd = orc.bf16_to_f64(x)
    for fmt, vals, sbit in ((orc.FMT_E2M1, E2M1_LITERAL, 8), (orc.FMT_E4M3, None, 128)):
        if vals is None:
            vals = [orc.e4m3_decode(c) for c in range(127)]
        codes, scales = orc.mx_quantize(x, fmt, "d")
        assert codes.shape == (6, 64) and scales.shape == (6, 2)
        for r in range(6):
            for b in range(2):
                blk = xd[r, 32 * b:32 * b + 32]
                amax = np.max(np.abs(blk))
                emax = 2 if fmt == orc.FMT_E2M1 else 8
                e = -127 if amax == 0 else max(-127, min(127, math.floor(math.log2(amax)) - emax))
                assert scales[r, b] == e + 127
                for t in range(32):
                    y = blk[t] / 2.0 ** e
                    mag, neg = _brute_nearest(y, vals)
                    if abs(y) > vals[-1]:
                        mag = len(vals) - 1
                    assert codes[r, 32 * b + t] == (mag | (sbit if neg else 0)), (fmt, r, b, t, y)
    c0, s0 = orc.mx_quantize(x, orc.FMT_E2M1, "d")
    assert np.all(s0[1] == 0) and np.all(c0[1] == 0)


def test_mx_quantize_seq_axis_is_transpose(orc):
    rng = np.random.default_rng(5)
    x = _bf16(rng.standard_normal((2, 64, 96)).astype(np.float32))
    c1, s1 = orc.mx_quantize(x, orc.FMT_E4M3, "seq")
    c2, s2 = orc.mx_quantize(np.ascontiguousarray(np.swapaxes(x, -1, -2)), orc.FMT_E4M3, "d")
    assert c1.shape == (2, 64, 96) and s1.shape == (2, 2, 96)
    assert np.array_equal(c1, np.swapaxes(c2, -1, -2))
    assert np.array_equal(s1, np.swapaxes(s2, -1, -2))
    d1 = orc.mx_dequantize(c1, s1, orc.FMT_E4M3, "seq")
    xd = orc.bf16_to_f64(x)
    # FP8 with a per-32 scale: each element is within 1/8 of its block max (the top binade
    # [256, 512) * 2^e saturates at 448), and within half an E4M3 step below saturation
    blocks = np.abs(xd).reshape(2, 2, 32, 96).max(axis=2, keepdims=True)
    err = np.abs(d1 - xd).reshape(2, 2, 32, 96)
    assert np.all(err <= blocks * 2.0 ** -3)
    e = np.floor(np.log2(blocks)) - 8
    y = np.abs(xd).reshape(2, 2, 32, 96) / 2.0 ** e
    step = np.where(y >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 3), 2.0 ** -9)
    ok = y <= 448
    assert np.all((err / 2.0 ** e)[ok] <= 0.5 * step[ok])


def test_bf16_rounding_matches_float32_path(orc):
    from precision_attention_amd.inputs import f32_to_bf16_bits

    rng = np.random.default_rng(11)
    x = rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 20000).astype(np.float32)
    # float32 inputs are exact in binary64, so one rounding from either width agrees
    assert np.array_equal(orc.f64_to_bf16(x.astype(np.float64)), f32_to_bf16_bits(x))
    ties = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)], np.float64)
    # ties to even: 1+2^-8 -> 1.0 (0x3F80), 1+3*2^-8 -> 1+2^-6 (0x3F82)
    assert list(orc.f64_to_bf16(ties)) == [0x3F80, 0x3F82, 0xBF80]
