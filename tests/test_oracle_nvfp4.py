"""Pins for the oracle's NVFP4-style quantization of Q and K and its Direct-P route.

Reading (gist.science summary, Methodology 1 "Format Selection": NVFP4 for Q and K): blocks of
16 along D with E2M1 elements and one E4M3 scale, s = RNE_E4M3(amax / 6 / 2^g) (saturating at
448), codes RNE_E2M1(x / (s 2^g)) (saturating, sign kept), the per-tensor scale 2^g a power of
two chosen by the caller. The route computes S from the represented values and runs Direct-P on
the integer-log2 anchor with MXFP4 V.

- Brute force in exact rational arithmetic (fractions.Fraction): the nearest E4M3 scale and the
  nearest E2M1 element by enumeration, ties to the even code, for random and hand-made blocks at
  several g.
- Hand cases: a block maximum of 6.375 makes the scale a tie (1.0625 between 1.0 and 1.125, to
  1.0) and the maximum then saturates to 6; an all-zero block; a block too small for the smallest
  E4M3 scale; a block whose scale saturates at 448.
- The represented values are exact in bf16.
- Route: on operands that both formats represent exactly (E2M1 values whose every 16- and 32-
  element block holds a 6), the NVFP4 route equals the MXFP4 anchored route bit for bit; V = 1
  gives O = 1.

Mutations of ``oracle/fp4attn_oracle.c`` applied one at a time, each of which made a test fail:
the scale taken from amax / 4 instead of amax / 6; the per-tensor scale left out of the element
quotient; the scale rounded up instead of to nearest; the block maximum taken over 8 of the 16
elements.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from precision_attention_amd.inputs import attention_inputs, f32_to_bf16_bits

E2M1 = [Fraction(v) for v in ("0", "1/2", "1", "3/2", "2", "3", "4", "6")]


def _e4m3_values(orc):
    return [Fraction(orc.e4m3_decode(c)) for c in range(127)]


def _nearest(v, grid):
    """Index of the nearest grid value to v >= 0 (ties to the even index), saturating."""
    best, bd = 0, None
    for i, g in enumerate(grid):
        d = abs(v - g)
        if bd is None or d < bd or (d == bd and i % 2 == 0):
            best, bd = i, d
    return best


def _brute(x, g, e4m3):
    """Scale code, element codes and represented values of one 16-element block."""
    xs = [Fraction(float(v)) for v in x]
    amax = max(abs(v) for v in xs)
    tg = Fraction(2) ** g
    sc = _nearest(amax / 6 / tg, e4m3)
    s = e4m3[sc]
    codes, vals = [], []
    for v in xs:
        if s == 0:
            c = 0
        else:
            c = _nearest(abs(v) / (s * tg), E2M1)
        sign = 8 if math.copysign(1.0, float(v)) < 0 else 0
        codes.append(c | sign)
        vals.append(float(E2M1[c] * s * tg) * (-1 if sign else 1))
    return sc, codes, vals


def _blocks():
    rng = np.random.default_rng(21)
    rows = [rng.standard_normal(16) for _ in range(6)]
    rows.append(rng.standard_normal(16) * 1000.0)
    rows.append(rng.standard_normal(16) * 1e-3)
    tie = np.zeros(16)
    tie[0], tie[1], tie[2] = 6.375, -3.1875, 0.53125  # amax / 6 = 1.0625: E4M3 tie between 1.0 and 1.125
    rows.append(tie)
    rows.append(np.zeros(16))
    rows.append(np.full(16, -2.0 ** -20))  # amax / 6 below half the smallest E4M3 scale
    rows.append(np.full(16, 6.0 * 448.0 * 3.0))  # the scale saturates at 448
    x = np.stack(rows)
    return orc_bf16_round(x)


def orc_bf16_round(x):
    return (f32_to_bf16_bits(x.astype(np.float32)).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("g", [0, -3, 5])
def test_nvfp4_brute_force(orc, g):
    x = _blocks()
    if g == 5:
        x = x * 32.0
    elif g == -3:
        x = x / 8.0
    codes, scales, xhat = orc.nvfp4_quantize(x, g)
    e4 = _e4m3_values(orc)
    for r in range(x.shape[0]):
        sc, cs, vs = _brute(x[r], g, e4)
        assert scales[r, 0] == sc, (r, scales[r, 0], sc)
        assert list(codes[r]) == cs, (r, list(codes[r]), cs)
        assert np.array_equal(xhat[r], np.array(vs)), r


def test_nvfp4_hand_cases(orc):
    x = _blocks()
    codes, scales, xhat = orc.nvfp4_quantize(x, 0)
    assert orc.e4m3_decode(int(scales[8, 0])) == 1.0                      # the tie rounds to even
    assert codes[8, 0] == orc.e2m1_encode(6.0) and xhat[8, 0] == 6.0     # 6.375 saturates to 6
    assert scales[9, 0] == 0 and np.all(codes[9] == 0) and np.all(xhat[9] == 0)
    assert scales[10, 0] == 0 and np.all(codes[10] == 8) and np.all(xhat[10] == 0)
    assert orc.e4m3_decode(int(scales[11, 0])) == 448.0
    assert np.all(xhat[11] == 6.0 * 448.0)


def test_nvfp4_values_exact_in_bf16(orc):
    x = attention_inputs(1, 2, 2, 256, 128, seed=4)["q"]
    _, _, xhat = orc.nvfp4_quantize(x, 0)
    back = (orc.f64_to_bf16(xhat).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(back, xhat)


def test_nvfp4_route_equals_mxfp4_on_common_values(orc):
    """E2M1 values with a 6 at the start of every 16-element block: NVFP4 scale 1 and MXFP4 scale
    2^0 both represent them exactly, so the two anchored routes see the same operands."""
    B, H, N, D = 1, 2, 256, 64
    rng = np.random.default_rng(22)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -1.5, -2, -3, -4, -6], np.float32)
    mk = lambda: grid[rng.integers(0, grid.size, (B, H, N, D))] * np.float32(0.25)  # noqa: E731
    q, k = mk(), mk()
    q[..., ::16] = 1.5  # 6 * 0.25: the block maximum of every 16 (and 32) elements
    k[..., ::16] = 1.5
    x = {"q": f32_to_bf16_bits(q), "k": f32_to_bf16_bits(k),
         "v": attention_inputs(B, H, H, N, D, seed=23)["v"]}
    nv = orc.nvfp4_anchored_forward(x["q"], x["k"], x["v"])
    mx = orc.directp_anchored_forward(x["q"], x["k"], x["v"])
    assert np.array_equal(nv["q_hat"], q.astype(np.float64))
    assert np.array_equal(nv["O"], mx["O"]) and np.array_equal(nv["lse"], mx["lse"])


def test_nvfp4_route_v_ones(orc):
    x = attention_inputs(1, 2, 1, 256, 128, seed=24)
    x["v"] = np.full_like(x["v"], 0x3F80)
    res = orc.nvfp4_anchored_forward(x["q"], x["k"], x["v"])
    assert np.array_equal(res["O"], np.ones_like(res["O"]))


def test_nvfp4_accuracy_against_fp64(orc):
    """Accuracy of O against fp64 softmax attention (textbook) on seeded inputs: with outlier
    channels (x10, two per head, as in the DiT workload) MXFP4's one scale per 32 elements flushes
    the ordinary channels of a block, NVFP4's E4M3 scale per 16 keeps them; on unit-variance inputs
    the finer scales help a little. Both routes on the integer-log2 anchor, so only Q/K differ."""
    from oracle import textbook

    def cos(a, b):
        a, b = a.reshape(-1), b.reshape(-1)
        return float(a @ b / np.sqrt((a @ a) * (b @ b)))

    out = {}
    for frac in (0.0, 0.01):
        x = attention_inputs(1, 2, 2, 2048, 128, seed=0, outlier_frac=frac)
        rows = np.sort(np.random.default_rng(1).choice(2 * 2048, 512, replace=False)).astype(np.int64)
        nv = orc.nvfp4_anchored_forward(x["q"], x["k"], x["v"], rows=rows)["O"]
        mx = orc.directp_anchored_forward(x["q"], x["k"], x["v"], rows=rows)["O"]
        ref = textbook.attention(*(orc.bf16_to_f64(x[n]) for n in ("q", "k", "v")), False)
        ref = (ref[0] if isinstance(ref, tuple) else ref).reshape(-1, 128)[rows]
        out[frac] = (cos(nv, ref), cos(mx, ref))
    print("O cosine vs fp64 (NVFP4, MXFP4): unit %s, outliers %s" % (out[0.0], out[0.01]))
    assert out[0.0][0] >= out[0.0][1] - 1e-3
    assert out[0.01][0] >= out[0.01][1] + 0.1
