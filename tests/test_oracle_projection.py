"""Pins for the oracle's QKV projection with the MX quantization of its epilogue.

Reading (gist.science summary, Methodology 2 "Quantized Causal Backward", *Gradient Formats*;
Results, *Training Performance*): the projection epilogues publish the quantized Q, K, V and the
backward's FP8 views. The oracle forms X W^T in binary64 and MX-quantizes those values with no
intermediate bf16 rounding.

- Layout: with small integers every product and sum is exact, so Q, K and V must equal integer
  sums taken element by element over the stated weight layout (rows of Wq, then Wk, then Wv,
  head-major, D rows per head).
- Rounding point: an output of 2.5 + 2^-10 in an E2M1 block scaled by 2^0 must get the code of
  3.0, and 1.0625 + 2^-12 in an E4M3 block scaled by 2^0 the code of 1.125; rounding to bf16 first
  gives the ties 2.5 and 1.0625, hence 2.0 and 1.0.
- The binary64 MX quantizer on values off the bf16 grid, against a brute-force nearest search.
- Power-of-two scaling of X moves every block exponent by one and keeps every code.

Mutations of ``oracle/__init__.py`` applied one at a time, each of which made a test fail:
rounding Q, K, V to bf16 before the quantization; heads taken as the fastest-varying feature index
(D-major instead of head-major rows); V's rows taken before K's.
"""
import math

import numpy as np

from precision_attention_amd.inputs import f32_to_bf16_bits
from tests.test_oracle_formats import E2M1_LITERAL, _brute_nearest


def _bits(a):
    return f32_to_bf16_bits(np.asarray(a, np.float32))


def test_layout_exact_integers(orc):
    B, N, Dm, H, Hkv, D = 2, 64, 96, 4, 2, 32
    rng = np.random.default_rng(11)
    X = rng.integers(-8, 9, (B, N, Dm))
    W = rng.integers(-8, 9, ((H + 2 * Hkv) * D, Dm))
    q, k, v = orc.project_qkv(_bits(X), _bits(W), H, Hkv, D)
    assert q.shape == (B, H, N, D) and k.shape == (B, Hkv, N, D) and v.shape == (B, Hkv, N, D)
    Xl, Wl = X.tolist(), W.tolist()

    def dot(b, n, f):
        return sum(Xl[b][n][j] * Wl[f][j] for j in range(Dm))

    idx = rng.integers(0, 1 << 30, (300, 4))
    for r in idx:
        b, n, d = r[0] % B, r[1] % N, r[3] % D
        h, g = r[2] % H, r[2] % Hkv
        assert q[b, h, n, d] == dot(b, n, h * D + d)
        assert k[b, g, n, d] == dot(b, n, (H + g) * D + d)
        assert v[b, g, n, d] == dot(b, n, (H + Hkv + g) * D + d)


def test_no_intermediate_bf16_rounding(orc):
    """Token 0 has x = e0 + e1, token 1 has x = e2. Feature 0 of head 0 puts 4 in token 0's first
    32-feature block (E2M1 exponent 0), feature 7 puts 2.5 + 2^-10 beside it; feature 5 puts
    1.0625 + 2^-12 at token 0 and 256 at token 1 (E4M3 exponent 0 along the sequence)."""
    H, Hkv, D, Dm, N = 1, 1, 64, 64, 32
    X = np.zeros((1, N, Dm), np.float32)
    X[0, 0, 0] = X[0, 0, 1] = 1.0
    X[0, 1, 2] = 1.0
    W = np.zeros(((H + 2 * Hkv) * D, Dm), np.float32)
    W[0, 0] = 4.0
    W[7, 0], W[7, 1] = 2.5, 2.0 ** -10
    W[5, 0], W[5, 1], W[5, 2] = 1.0625, 2.0 ** -12, 256.0
    views, (q, _, _) = orc.project_qkv_views(_bits(X), _bits(W), H, Hkv, D, fp8_views=True)
    assert q[0, 0, 0, 7] == 2.5 + 2.0 ** -10 and q[0, 0, 0, 5] == 1.0625 + 2.0 ** -12
    # bf16 rounding would land on the ties
    assert orc.f64_to_bf16(np.array([2.5 + 2.0 ** -10]))[0] == _bits([2.5])[0]
    assert orc.f64_to_bf16(np.array([1.0625 + 2.0 ** -12]))[0] == _bits([1.0625])[0]
    codes, scales = views["q"]
    assert scales[0, 0, 0, 0] == 127
    assert codes[0, 0, 0, 7] == orc.e2m1_encode(3.0) != orc.e2m1_encode(2.0)
    codes8, scales8 = views["q8"]  # along the sequence: [B, H, N, D] codes, [B, H, N/32, D] scales
    assert scales8[0, 0, 0, 5] == 127
    assert codes8[0, 0, 0, 5] == orc.e4m3_encode(1.125) != orc.e4m3_encode(1.0)
    assert codes8[0, 0, 1, 5] == orc.e4m3_encode(256.0)


def test_f64_quantizer_brute_force(orc):
    rng = np.random.default_rng(12)
    x = rng.standard_normal((4, 64)) * np.array([[1.0], [37.0], [1e-3], [2.0 ** -120]])
    x[0, :32] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0] * 4) * (1 + 2.0 ** -40)
    for fmt, vals, sbit, emax in ((orc.FMT_E2M1, E2M1_LITERAL, 8, 2), (orc.FMT_E4M3, None, 128, 8)):
        if vals is None:
            vals = [orc.e4m3_decode(c) for c in range(127)]
        codes, scales = orc.mx_quantize(x, fmt, "d")
        for r in range(4):
            for b in range(2):
                blk = x[r, 32 * b:32 * b + 32]
                e = max(-127, min(127, math.floor(math.log2(np.max(np.abs(blk)))) - emax))
                assert scales[r, b] == e + 127
                for t in range(32):
                    y = blk[t] / 2.0 ** e
                    mag, neg = _brute_nearest(y, vals)
                    if abs(y) > vals[-1]:
                        mag = len(vals) - 1
                    assert codes[r, 32 * b + t] == (mag | (sbit if neg else 0)), (fmt, r, b, t, y)


def test_power_of_two_scaling(orc):
    B, N, Dm, H, Hkv, D = 1, 64, 64, 2, 1, 64
    rng = np.random.default_rng(13)
    X = rng.standard_normal((B, N, Dm)).astype(np.float32)
    W = (rng.standard_normal(((H + 2 * Hkv) * D, Dm)) / 8).astype(np.float32)
    a, _ = orc.project_qkv_views(_bits(X), _bits(W), H, Hkv, D, fp8_views=True)
    b, _ = orc.project_qkv_views(_bits(X * 2), _bits(W), H, Hkv, D, fp8_views=True)
    for name in a:
        assert np.array_equal(a[name][0], b[name][0]), name
        assert np.array_equal(a[name][1].astype(int) + 1, b[name][1].astype(int)), name
