"""Pins for the oracle's Direct-P on the integer-log2 anchor (ORC_P_DIRECT_ANCHOR).

Reading (gist.science summary, Methodology 1 "Direct Mapping" and "Range Guarding"): each 32-key
block's probabilities are the MX quantization, block exponent floor(log2 amax) - 2, of the
unnormalized exponentials 2^(S c) = e^(S/sqrt(D)); the oracle forms each code by the threshold
classifier from u = fmaf(S, c, 2 - floor(fp32(S_bmax c))). O = sum P V / sum P and LSE = ln sum P.

- Closed form: blocks of constant scores. Every key of a block gets 2^(2 + f) rounded to E2M1
  times 2^(t - 2), t and f the integer and fractional parts of S c: 4 * 2^(t-2) when 2^(2+f) < 5,
  else 6 * 2^(t-2); so l, O and LSE follow by hand.
- The written reading, materialized: S in binary64, exp2(S c), MX-quantized per 32 keys by an
  independently written quantizer, normalized. It must agree with the oracle except where u lies
  within rounding of a step point (a few rows at most), also at logits near 600 (the range the
  summary's range guard is for), where binary64 still holds 2^(S c).
- Block structure: permuting keys inside each aligned 32-key block leaves O and LSE unchanged,
  permuting across blocks changes them.
- Consistent normalization: V = 1 gives O = 1 exactly.
"""
import numpy as np
import pytest

from precision_attention_amd.inputs import attention_inputs, f32_to_bf16_bits
from tests.mxref import mx_e2m1_rows


def _dequant(orc, x):
    ops = orc.quantize_directp_operands(x["q"], x["k"], x["v"])
    return (orc.mx_dequantize(*ops["q"], orc.FMT_E2M1, "d"), orc.mx_dequantize(*ops["k"], orc.FMT_E2M1, "d"),
            orc.mx_dequantize(*ops["v"], orc.FMT_E2M1, "seq"))


def test_closed_form_constant_blocks(orc):
    """Three 32-key blocks of constant scores s0, s1, s2 (one query row). q = (1, 0, ...) and
    k_j = (s_b, 0, ...) with s_b exact MXFP4 values; V on the E2M1 grid with a 6 in every block
    (scale 2^0), so V is exact too."""
    D, N = 64, 96
    c = float(orc.log2e_scale(D))
    svals = [3.0, 10.0, -6.0]  # S c = 0.541, 1.803, -1.082: fractional parts 0.54, 0.80, 0.92
    q = np.zeros((1, 1, N, D), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, 1, N, D), np.float32)
    for b, sv in enumerate(svals):
        k[0, 0, 32 * b:32 * (b + 1), 0] = sv
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -1.5, -2, -3, -4, -6], np.float32)
    rng = np.random.default_rng(2)
    v = grid[rng.integers(0, grid.size, (1, 1, N, D))]
    v[0, 0, ::32, :] = 6.0
    x = {"q": f32_to_bf16_bits(q), "k": f32_to_bf16_bits(k), "v": f32_to_bf16_bits(v)}
    res = orc.directp_anchored_forward(x["q"], x["k"], x["v"])
    P = []
    for sv in svals:
        t = np.floor(sv * c)
        f = sv * c - t
        P.append((4.0 if 2.0 ** (2 + f) < 5.0 else 6.0) * 2.0 ** (t - 2))
    V = v[0, 0].astype(np.float64)
    l = sum(32 * p for p in P)
    O = sum(P[b] * V[32 * b:32 * (b + 1)].sum(0) for b in range(3)) / l
    for row in (0, N - 1):
        assert np.max(np.abs(res["O"][0, 0, row] - O)) < 1e-12
        assert res["lse"][0, 0, row] == pytest.approx(np.log(l), abs=1e-12)
        assert res["l"][0, 0, row] == pytest.approx(l, rel=1e-15)


@pytest.mark.parametrize("scale", [1.0, 12.0], ids=["unit", "logits_near_600"])
def test_materialized_reading(orc, scale):
    """O and LSE against S -> exp2(S c) -> independent MX quantization per 32 keys -> normalize,
    in binary64. scale 12 multiplies Q and K, so the largest logits S/sqrt(D) reach about 600."""
    B, H, N, D = 1, 2, 256, 64
    x = attention_inputs(B, H, H, N, D, seed=31)
    if scale != 1.0:
        for n in ("q", "k"):
            f = (x[n].astype(np.uint32) << 16).view(np.float32) * np.float32(scale)
            x[n] = f32_to_bf16_bits(f)
    Qd, Kd, Vd = _dequant(orc, x)
    res = orc.attn_fwd(Qd, Kd, Vd, 32, False, orc.P_DIRECT_ANCHOR)
    c = float(orc.log2e_scale(D))
    bad = 0
    for h in range(H):
        S = Qd[0, h] @ Kd[0, h].T
        if scale != 1.0:
            assert np.max(S / np.sqrt(D)) > 500
        Ph = mx_e2m1_rows(np.exp2(S * c))
        l = Ph.sum(axis=1)
        O = (Ph @ Vd[0, h]) / l[:, None]
        rel = np.abs(O - res["O"][0, h]).max(axis=1) / np.abs(O).max(axis=1)
        bad += int(np.sum((rel > 1e-12) | (np.abs(np.log(l) - res["lse"][0, h]) > 1e-12)))
    assert np.all(np.isfinite(res["O"])) and np.all(np.isfinite(res["lse"]))
    assert bad <= 2, bad


def test_block_structure(orc):
    B, H, N, D = 1, 1, 128, 64
    x = attention_inputs(B, H, H, N, D, seed=5)
    Qd, Kd, Vd = _dequant(orc, x)
    base = orc.attn_fwd(Qd, Kd, Vd, 32, False, orc.P_DIRECT_ANCHOR)
    rng = np.random.default_rng(6)
    within = np.concatenate([b0 + rng.permutation(32) for b0 in range(0, N, 32)])
    res = orc.attn_fwd(Qd, Kd[:, :, within], Vd[:, :, within], 32, False, orc.P_DIRECT_ANCHOR)
    assert np.max(np.abs(res["O"] - base["O"])) < 1e-14 and np.max(np.abs(res["lse"] - base["lse"])) < 1e-14
    across = rng.permutation(N)
    res = orc.attn_fwd(Qd, Kd[:, :, across], Vd[:, :, across], 32, False, orc.P_DIRECT_ANCHOR)
    assert np.max(np.abs(res["O"] - base["O"])) > 1e-4


def test_v_ones_and_key_block_independence(orc):
    x = attention_inputs(1, 2, 1, 256, 128, seed=8)
    ones = dict(x, v=np.full_like(x["v"], 0x3F80))
    res = orc.directp_anchored_forward(ones["q"], ones["k"], ones["v"])
    assert np.array_equal(res["O"], np.ones_like(res["O"]))
    Qd, Kd, Vd = _dequant(orc, x)
    r32 = orc.attn_fwd(Qd, Kd, Vd, 32, False, orc.P_DIRECT_ANCHOR)
    r128 = orc.attn_fwd(Qd, Kd, Vd, 128, False, orc.P_DIRECT_ANCHOR)
    assert np.array_equal(r32["O"], r128["O"]) and np.array_equal(r32["lse"], r128["lse"])
