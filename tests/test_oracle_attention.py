"""Pins for the oracle's forward and backward attention.

- Identity reduction: with every quantizer switched off the online (running-max)
  softmax must equal fp64 textbook attention (NumPy), for any key-block size, causal or
  not, with grouped-query heads.
- Consistent normalization (gist.science summary, Methodology 1): with V = 1 the output is
  exactly 1, because numerator and denominator accumulate the same represented values.
- Single anchor: with one key block covering the whole row, the Direct-P output equals an
  independently written "materialize S, MX-quantize exp2((S-m)c) per 32 keys, normalize".
- Causal boundary (summary, Methodology 2): row 0 sees only key 0, so O_0 = V_0 and
  LSE_0 = S_00 / sqrt(D).
- Backward (summary, Methodology 2): with identity quantizers the gradients equal central
  finite differences of the fp64 textbook loss sum(dO * O).
- Statistical sanity of the quantized routes against fp64 attention.
"""
import numpy as np
import pytest

from oracle import textbook
from precision_attention_amd.inputs import attention_inputs
from tests.mxref import mx_e2m1_rows


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("KB", [32, 64, 96])
def test_identity_reduces_to_textbook(orc, causal, KB):
    B, H, Hkv, N, D = 2, 4, 2, 160, 32
    Q, K, V = _rand((B, H, N, D), 1) * 2, _rand((B, Hkv, N, D), 2) * 2, _rand((B, Hkv, N, D), 3)
    res = orc.attn_fwd(Q, K, V, KB, causal, orc.P_EXACT)
    O, lse, _ = textbook.attention(Q, K, V, causal)
    assert np.max(np.abs(res["O"] - O)) < 1e-12
    assert np.max(np.abs(res["lse"] - lse)) < 1e-12


def test_row_subset_matches_full(orc):
    x = attention_inputs(1, 4, 2, 256, 64, seed=4)
    full = orc.directp_forward(x["q"], x["k"], x["v"], KB=64)
    rows = np.array([0, 5, 255, 256 + 17, 3 * 256 + 200], np.int64)
    sub = orc.directp_forward(x["q"], x["k"], x["v"], KB=64, rows=rows)
    assert np.array_equal(sub["O"], full["O"].reshape(-1, 64)[rows])
    assert np.array_equal(sub["lse"], full["lse"].reshape(-1)[rows])


@pytest.mark.parametrize("route", ["directp", "causal_fp8"])
def test_v_ones_gives_ones(orc, route):
    x = attention_inputs(1, 2, 1, 256, 64, seed=8)
    ones = np.full_like(x["v"], 0x3F80)  # bf16 1.0
    if route == "directp":
        res = orc.directp_forward(x["q"], x["k"], ones, KB=64)
    else:
        res = orc.causal_forward(x["q"], x["k"], ones, KB=64)
    assert np.array_equal(res["O"], np.ones_like(res["O"]))


def test_single_anchor_against_materialized_quantization(orc):
    B, H, N, D = 1, 2, 256, 64
    x = attention_inputs(B, H, H, N, D, seed=12)
    ops = orc.quantize_directp_operands(x["q"], x["k"], x["v"])
    Qd = orc.mx_dequantize(*ops["q"], orc.FMT_E2M1, "d")
    Kd = orc.mx_dequantize(*ops["k"], orc.FMT_E2M1, "d")
    Vd = orc.mx_dequantize(*ops["v"], orc.FMT_E2M1, "seq")
    res = orc.attn_fwd(Qd, Kd, Vd, N, False, orc.P_DIRECT)  # one key block: a single anchor
    c = float(orc.log2e_scale(D))
    mism = 0
    for h in range(H):
        S = Qd[0, h] @ Kd[0, h].T
        m = S.max(axis=1, keepdims=True)
        Ph = mx_e2m1_rows(np.exp2((S - m) * c))
        O = (Ph @ Vd[0, h]) / Ph.sum(axis=1, keepdims=True)
        err = np.abs(O - res["O"][0, h]).max(axis=1)
        mism += int(np.sum(err > 1e-12))
    # binary32 u versus binary64 exponent may flip a code at a step point: allow a few rows
    assert mism <= 2


@pytest.mark.parametrize("route", ["directp", "causal_fp8"])
def test_rescale_free_when_first_key_dominates(orc, route):
    """If key 0 holds every row's maximum, the running max never moves after the first
    block, so the result cannot depend on the key-block size."""
    rng = np.random.default_rng(21)
    N, D = 192, 32
    from precision_attention_amd.inputs import f32_to_bf16_bits

    q = np.abs(rng.standard_normal((1, 1, N, D))).astype(np.float32)
    k = rng.standard_normal((1, 1, N, D)).astype(np.float32)
    k[0, 0, 0, :] = 4.0
    v = rng.standard_normal((1, 1, N, D)).astype(np.float32)
    q16, k16, v16 = (f32_to_bf16_bits(a) for a in (q, k, v))
    fn = orc.directp_forward if route == "directp" else orc.causal_forward
    r32 = fn(q16, k16, v16, KB=32)
    r192 = fn(q16, k16, v16, KB=192)
    assert np.array_equal(r32["O"], r192["O"]) and np.array_equal(r32["lse"], r192["lse"])


def test_causal_row_zero(orc):
    x = attention_inputs(1, 2, 1, 128, 64, seed=5)
    res = orc.causal_forward(x["q"], x["k"], x["v"], KB=64)
    ops = res["ops"]
    Qd = orc.mx_dequantize(*ops["q"], orc.FMT_E2M1, "d")
    Kd = orc.mx_dequantize(*ops["k"], orc.FMT_E2M1, "d")
    Vd = orc.mx_dequantize(*ops["v8"], orc.FMT_E4M3, "seq")
    for h in range(2):
        assert np.array_equal(res["O"][0, h, 0], Vd[0, 0, 0])
        s00 = float(Qd[0, h, 0] @ Kd[0, 0, 0])
        assert res["lse"][0, h, 0] == pytest.approx(s00 / 8.0, abs=1e-12)
        assert res["l"][0, h, 0] == 1.0


def test_scores_exactness_is_checked(orc):
    # unquantized operands give scores that are not binary32 values: the oracle refuses
    Q = _rand((1, 1, 64, 32), 1)
    with pytest.raises(orc.OracleError):
        orc.attn_fwd(Q, Q, Q, 32, False, orc.P_DIRECT)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_identity_matches_finite_differences(orc, causal):
    B, H, Hkv, N, D = 1, 2, 1, 64, 32
    Q, K, V = _rand((B, H, N, D), 31), _rand((B, Hkv, N, D), 32), _rand((B, Hkv, N, D), 33)
    dO = _rand((B, H, N, D), 34)
    O, lse, _ = textbook.attention(Q, K, V, causal)
    g = orc.attn_bwd(Q, K, dO, V, dO, K, Q, O, dO, lse, causal=causal, quant=False)
    rng = np.random.default_rng(35)
    h = 1e-5
    for name, T, G in (("Q", Q, g["dQ"]), ("K", K, g["dK"]), ("V", V, g["dV"])):
        for _ in range(12):
            idx = tuple(rng.integers(0, s) for s in T.shape)
            Tp, Tm = T.copy(), T.copy()
            Tp[idx] += h
            Tm[idx] -= h
            args_p = {"Q": Q, "K": K, "V": V}
            args_m = {"Q": Q, "K": K, "V": V}
            args_p[name], args_m[name] = Tp, Tm
            fd = (textbook.loss(args_p["Q"], args_p["K"], args_p["V"], dO, causal)
                  - textbook.loss(args_m["Q"], args_m["K"], args_m["V"], dO, causal)) / (2 * h)
            assert abs(G[idx] - fd) <= 1e-6 * max(1.0, abs(fd)), (name, idx, G[idx], fd)


def _cos(a, b):
    a, b = np.ravel(a), np.ravel(b)
    return float(a @ b / np.linalg.norm(a) / np.linalg.norm(b))


def test_statistical_sanity_against_fp64(orc):
    B, H, Hkv, N, D = 1, 4, 2, 512, 128
    x = attention_inputs(B, H, Hkv, N, D, seed=0, with_do=True)
    Q, K, V = (orc.bf16_to_f64(x[n]) for n in ("q", "k", "v"))
    dO = orc.bf16_to_f64(x["do"])
    O, _, _ = textbook.attention(Q, K, V, False)
    dp = orc.directp_forward(x["q"], x["k"], x["v"], KB=128)
    assert _cos(dp["O"], O) >= 0.95
    # the FP8 P/V route is the more accurate one (the pages' Results, "Accuracy": ~0.990 against
    # ~0.944 for Direct-P, on their own workloads and formats)
    f8 = orc.fp8_forward(x["q"], x["k"], x["v"], KB=128, causal=False)
    print("cosine vs fp64: Direct-P %.4f, FP8 route %.4f" % (_cos(dp["O"], O), _cos(f8["O"], O)))
    assert _cos(f8["O"], O) > _cos(dp["O"], O) and _cos(f8["O"], O) >= 0.98
    Oc, lsec, _ = textbook.attention(Q, K, V, True)
    cf = orc.causal_forward(x["q"], x["k"], x["v"], KB=128)
    assert _cos(cf["O"], Oc) >= 0.98
    g_exact = orc.attn_bwd(Q, K, dO, V, dO, K, Q, Oc, dO, lsec, causal=True, quant=False)
    g = orc.causal_backward(x["q"], x["k"], x["v"], x["do"], cf["O_bf16"], cf["lse"].astype(np.float32))
    for n in ("dQ", "dK", "dV"):
        assert _cos(g[n], g_exact[n]) >= 0.97, n


def test_backward_row_and_column_subsets(orc):
    x = attention_inputs(1, 4, 2, 128, 64, seed=6, with_do=True)
    cf = orc.causal_forward(x["q"], x["k"], x["v"], KB=64)
    lse = cf["lse"].astype(np.float32)
    full = orc.causal_backward(x["q"], x["k"], x["v"], x["do"], cf["O_bf16"], lse)
    qrows = np.array([0, 31, 127, 128 + 64, 3 * 128 + 5], np.int64)
    kcols = np.array([0, 100, 128 + 127], np.int64)
    sub = orc.causal_backward(x["q"], x["k"], x["v"], x["do"], cf["O_bf16"], lse, qrows=qrows, kcols=kcols)
    assert np.array_equal(sub["dQ"], full["dQ"].reshape(-1, 64)[qrows])
    assert np.array_equal(sub["dK"], full["dK"].reshape(-1, 64)[kcols])
    assert np.array_equal(sub["dV"], full["dV"].reshape(-1, 64)[kcols])


@pytest.mark.parametrize("route", ["directp", "causal_fp8"])
def test_rescale_closed_form(orc, route):
    """Two 32-key blocks of constant scores s0 < s1 (exact MX values). Every key gets P = 1
    relative to its block's running max, so after the rescale
    O = (a * sum V_blk0 + sum V_blk1) / (32 a + 32), a = 2^((s0 - s1) c), and
    LSE = s1 / sqrt(D) + ln(32 a + 32)."""
    from precision_attention_amd.inputs import f32_to_bf16_bits

    N, D = 64, 32
    q = np.zeros((1, 1, N, D), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, 1, N, D), np.float32)
    k[0, 0, :32, 0] = 2.0
    k[0, 0, 32:, 0] = 6.0
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -1.5, -2, -3, -4, -6], np.float32)
    rng = np.random.default_rng(4)
    v = grid[rng.integers(0, grid.size, (1, 1, N, D))]
    v[0, 0, 0, :] = 6.0  # block max 6: scale 2^0, so every value is exact in MXFP4 and MXFP8
    v[0, 0, 32, :] = 6.0
    q16, k16, v16 = (f32_to_bf16_bits(a) for a in (q, k, v))
    if route == "directp":
        res = orc.directp_forward(q16, k16, v16, KB=32)
    else:
        # causal: only the last row sees both blocks
        res = orc.causal_forward(q16, k16, v16, KB=32)
    c = float(orc.log2e_scale(D))
    a = 2.0 ** ((2.0 - 6.0) * c)
    V = v[0, 0].astype(np.float64)
    want = (a * V[:32].sum(0) + V[32:].sum(0)) / (32 * a + 32)
    row = N - 1
    assert np.max(np.abs(res["O"][0, 0, row] - want)) < 1e-12
    assert res["lse"][0, 0, row] == pytest.approx(6.0 / np.sqrt(D) + np.log(32 * a + 32), abs=1e-12)
