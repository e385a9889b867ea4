"""Pins for the oracle's quantized backward and its softmax-scale constant.

The backward follows the gist.science technical summary, Methodology 2 "Quantized Causal
Backward" (*Reconstruction*: probabilities are rebuilt from the saved quantized Q/K and the
saved LSE; *Gradient Formats*: the gradient products take FP8 operands, read as MXFP8 blocked
along each product's contraction axis), and the arXiv abstract (FP8 gradient operands).

Each test below is built so that its expected values follow from the construction by hand, not
from the oracle's own formulas, and so that a plausible mistake in ``orc_attn_bwd`` fails it.
The mutations listed in each docstring were applied to ``oracle/fp4attn_oracle.c`` one at a
time, and each made the test fail:

- ``test_log2e_scale_literal_bits``: c computed as log2(e) * sqrt(D), or as 1/sqrt(D) without
  log2(e). (Forming it in binary32 as 1.44269504f / sqrtf(D) gives the same bits for D = 64 and
  128, so that is not a mistake.)
- ``test_bwd_prob_hand_values``: P = exp(S/sqrt(D) - LSE) in binary64 (the unquantized rule);
  LSE log2 e rounded once from binary64 instead of multiplied in binary32; P not rounded to
  binary32; u formed as fp32(S c) + nl (two roundings) instead of one fused multiply-add.
- ``test_quantized_backward_exact_case``: Delta added instead of subtracted (in the dQ or in the
  dK/dV part) or left out; the 1/sqrt(D) factor missing on dQ or dK, or applied to dV; dV fed
  dO's along-D view instead of its along-query view; dQ fed Q's FP8 view instead of K's; the
  causal mask j <= i taken as j < i; only the first query head of a KV group summed.
- ``test_quantized_backward_blocking_axes``: dS for dQ blocked along queries instead of keys;
  the MXFP8 rounding of dS for dQ, of dS for dK, or of P for dV skipped.
"""
from decimal import Decimal, getcontext

import numpy as np
import pytest

LOG2E_F32 = np.float32(1.44269504)


def _f32_bits(x) -> int:
    return int(np.float32(x).view(np.uint32))


def _round_to_f32(x: Decimal) -> np.float32:
    """Round a positive Decimal to the nearest binary32 (ties to even), exactly."""
    lo = np.float32(float(x))  # within an ulp of x; correct it by exact comparison
    for _ in range(4):
        d_lo = Decimal(float(lo))
        if d_lo > x:
            lo = np.nextafter(lo, np.float32(0))
            continue
        hi = np.nextafter(lo, np.float32(np.inf))
        d_hi = Decimal(float(hi))
        if d_hi <= x:
            lo = hi
            continue
        mid = (d_lo + d_hi) / 2
        if x < mid:
            return lo
        if x > mid:
            return hi
        return lo if (int(lo.view(np.uint32)) & 1) == 0 else hi
    raise AssertionError("rounding did not converge")


def test_log2e_scale_literal_bits(orc):
    """c = log2(e)/sqrt(D) rounded once to binary32: the literal bit patterns 0x3E38AA3B (D=64)
    and 0x3E0293EE (D=128), and the same values re-derived at 50 digits with Decimal."""
    assert _f32_bits(orc.log2e_scale(64)) == 0x3E38AA3B
    assert _f32_bits(orc.log2e_scale(128)) == 0x3E0293EE
    getcontext().prec = 50
    log2e = 1 / Decimal(2).ln()
    for D in (64, 128):
        exact = log2e / Decimal(D).sqrt()
        assert _f32_bits(_round_to_f32(exact)) == _f32_bits(orc.log2e_scale(D)), D


def _lse_with_integer_nl(k: int) -> np.float32:
    """A binary32 LSE whose binary32 product with binary32 log2(e) is exactly k (so the rebuilt
    probability of a zero score is exactly 2^-k); exp(-LSE) is then NOT exactly 2^-k."""
    lse = np.float32(k / float(np.float64(LOG2E_F32)))
    for _ in range(64):
        prod = np.float32(np.float64(lse) * np.float64(LOG2E_F32))  # one binary32 rounding
        if prod == k:
            return lse
        lse = np.nextafter(lse, np.float32(np.inf) if prod < k else np.float32(0))
    raise AssertionError("no LSE found for k=%d" % k)


def _score_with_integer_u(D: int, nl: int, targets=range(8, 16)):
    """A binary32 score S and an integer t with fmaf(S, c, nl) exactly equal to t (c = the
    pinned constant). The product of two binary32 values is exact in binary64 and so is adding
    the small integer nl, so rounding that sum once to binary32 is the fused multiply-add. One
    step of S moves S c by more than an ulp of t, so not every t is reachable: the first
    reachable t of ``targets`` is used."""
    c = np.float64(np.array([0x3E38AA3B if D == 64 else 0x3E0293EE], np.uint32).view(np.float32)[0])
    for t in targets:
        s0 = np.float32((t - nl) / c)
        for s in (np.nextafter(s0, np.float32(-np.inf)), s0, np.nextafter(s0, np.float32(np.inf))):
            if np.float32(np.float64(s) * c + np.float64(nl)) == t:
                return s, t
    raise AssertionError("no score found")


def test_bwd_prob_hand_values(orc):
    """P = fp32(2^(fmaf(S, c, -fp32(LSE log2 e)))), pinned on values known by construction and on
    a case where the binary32 steps matter:
    - S = 0 with fp32(LSE log2 e) = 5 exactly: P = 2^-5 exactly, although exp(-LSE) differs from
      2^-5 in the eighth digit;
    - S chosen so that the fused multiply-add gives exactly an integer t: P = 2^t;
    - a generic (S, LSE): 2^u evaluated at 50 digits from the exactly known binary32 u, rounded
      once to binary32."""
    lse5 = _lse_with_integer_nl(5)
    assert abs(np.exp(-np.float64(lse5)) / 2.0 ** -5 - 1.0) > 1e-9  # the two rules differ here
    for D in (64, 128):
        assert orc.bwd_prob(0.0, lse5, D) == 2.0 ** -5
        s, t = _score_with_integer_u(D, -5)
        assert orc.bwd_prob(s, lse5, D) == 2.0 ** t
    getcontext().prec = 50
    rng = np.random.default_rng(3)
    for D in (64, 128):
        c = Decimal(float(orc.log2e_scale(D)))
        for _ in range(20):
            s = np.float32(rng.normal() * 12.0)
            lse = np.float32(abs(rng.normal()) * 4.0 + 3.0)
            nl = -Decimal(float(_round_to_f32(Decimal(float(lse)) * Decimal(float(LOG2E_F32)))))
            u = Decimal(float(s)) * c + nl
            u32 = _round_to_f32(abs(u)) if u > 0 else -_round_to_f32(-u)
            want = _round_to_f32((Decimal(float(u32)) * Decimal(2).ln()).exp())
            assert orc.bwd_prob(s, lse, D) == float(want), (D, s, lse)


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
def test_quantized_backward_exact_case(orc, causal):
    """Every MXFP8 rounding of the quantized backward is exact here, so the quantized gradients
    must equal the hand-built closed form exactly.

    Construction (B=1, H=2 query heads on Hkv=1, N=D=64, scale 1/8): the MXFP4 scores are zero
    (Qs = Ks = 0) and every row's LSE is the binary32 value whose binary32 product with log2 e is
    exactly 5, so every visible probability is exactly 2^-5 (exact in MXFP8 along queries).
    V's FP8 view is the identity, so dP = dO's along-D view, which is set to M + Delta_i with M
    an integer matrix in [-7, 7] per head (every such block is exact in MXFP8 along either axis)
    and Delta_i = sum_d dO_id O_id an integer in [-3, 3] (O and dO only in column 0). Then
    dS = 2^-5 M on visible pairs, and, with the other FP8 views small integers:
      dQ_h = (1/8) 2^-5 (M_h * vis) Kk,   dK = (1/8) 2^-5 sum_h (M_h * vis)^T Qq_h,
      dV = 2^-5 sum_h vis^T dOq_h,
    all exact in binary64."""
    B, H, Hkv, N, D = 1, 2, 1, 64, 64
    rng = np.random.default_rng(11 + causal)
    vis = np.tril(np.ones((N, N))) if causal else np.ones((N, N))
    M = rng.integers(-7, 8, (H, N, N)).astype(np.float64)
    delta = rng.integers(-3, 4, (H, N)).astype(np.float64)
    Qs = np.zeros((B, H, N, D))
    Ks = np.zeros((B, Hkv, N, D))
    Vd = np.eye(N, D)[None, None].copy()  # [1, 1, N, D] with D == N: V_j = e_j
    dOd = (M + delta[:, :, None])[None]   # dP_ij = dOd_i . e_j = M_ij + Delta_i
    O = np.zeros((B, H, N, D))
    dO = np.zeros((B, H, N, D))
    O[0, :, :, 0] = delta
    dO[0, :, :, 0] = 1.0
    dOq = rng.integers(-4, 5, (B, H, N, D)).astype(np.float64)
    Kk = rng.integers(-4, 5, (B, Hkv, N, D)).astype(np.float64)
    Qq = rng.integers(-4, 5, (B, H, N, D)).astype(np.float64)
    lse = np.full((B, H, N), float(_lse_with_integer_nl(5)))
    g = orc.attn_bwd(Qs, Ks, dOd, Vd, dOq, Kk, Qq, O, dO, lse, causal=causal, quant=True)
    p = 2.0 ** -5
    dQ = np.stack([(1 / 8) * p * (M[h] * vis) @ Kk[0, 0] for h in range(H)])[None]
    dK = ((1 / 8) * p * sum((M[h] * vis).T @ Qq[0, h] for h in range(H)))[None, None]
    dV = (p * sum(vis.T @ dOq[0, h] for h in range(H)))[None, None]
    assert np.array_equal(g["dQ"], dQ)
    assert np.array_equal(g["dK"], dK)
    assert np.array_equal(g["dV"], dV)


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
def test_quantized_backward_blocking_axes(orc, causal):
    """Which axis each MXFP8 quantization blocks along, pinned by one dominant element per
    block: in a 32-block whose maximum is 2^20 times its other elements, those elements fall
    below half the smallest E4M3 subnormal and round to zero, while blocks without a dominant
    element stay exact.

    Construction (B=1, H=1, N=D=64, scale 1/8, zero scores except one): every visible P is 2^-5
    (as in the exact case) except P[i1, j1] = 2^t, made by one score S with fmaf(S, c, -5) = t
    exactly (t >= 14, so 2^t is at least 2^19 times 2^-5); dP = 1 on every pair except
    dP[i0, j0] = 2^20; Delta = 0. So dS equals P except dS[i0, j0] = 2^15 and dS[i1, j1] = 2^t,
    and:
    - dV uses P blocked along queries: in column j1 the other queries of i1's 32-block vanish;
    - dQ uses dS blocked along keys: in row i0 (row i1) the other keys of j0's (j1's) 32-block
      vanish;
    - dK uses dS blocked along queries: in column j0 (j1) the other queries of i0's (i1's)
      32-block vanish.
    The expected gradients are built from those rules by hand, in binary64, exactly."""
    B, H, Hkv, N, D = 1, 1, 1, 64, 64
    i0, j0, i1, j1 = 40, 7, 50, 33  # (i0, j0) and (i1, j1) visible under the mask too
    rng = np.random.default_rng(21 + causal)
    vis = np.tril(np.ones((N, N))) if causal else np.ones((N, N))
    s_big, t = _score_with_integer_u(D, -5, targets=range(14, 24))
    s_big = float(s_big)
    Qs = np.zeros((B, H, N, D))
    Ks = np.zeros((B, Hkv, N, D))
    Qs[0, 0, i1, 0] = s_big
    Ks[0, 0, j1, 0] = 1.0
    dOd = np.zeros((B, H, N, D))
    Vd = np.zeros((B, Hkv, N, D))
    dOd[0, 0, :, 0] = 1.0
    Vd[0, 0, :, 0] = 1.0
    dOd[0, 0, i0, 1] = 2.0 ** 20 - 1.0
    Vd[0, 0, j0, 1] = 1.0
    O = np.zeros((B, H, N, D))
    dO = np.zeros((B, H, N, D))
    dOq = rng.integers(-4, 5, (B, H, N, D)).astype(np.float64)
    Kk = rng.integers(-4, 5, (B, Hkv, N, D)).astype(np.float64)
    Qq = rng.integers(-4, 5, (B, H, N, D)).astype(np.float64)
    lse = np.full((B, H, N), float(_lse_with_integer_nl(5)))
    g = orc.attn_bwd(Qs, Ks, dOd, Vd, dOq, Kk, Qq, O, dO, lse, causal=causal, quant=True)

    small, big = 2.0 ** -5, {(i0, j0): 2.0 ** 15, (i1, j1): 2.0 ** t}
    blk = lambda t: slice(t // 32 * 32, t // 32 * 32 + 32)  # noqa: E731
    # P blocked along queries (columns): column j1 keeps only i1 inside i1's block
    Pq = small * vis
    Pq[blk(i1), j1] = 0.0
    Pq[i1, j1] = big[i1, j1]
    # dS blocked along keys (rows): rows i0 and i1 keep only their dominant inside its block
    dSk = small * vis
    for (i, j) in ((i0, j0), (i1, j1)):
        dSk[i, blk(j)] = 0.0
        dSk[i, j] = big[i, j]
    # dS blocked along queries (columns)
    dSq = small * vis
    for (i, j) in ((i0, j0), (i1, j1)):
        dSq[blk(i), j] = 0.0
        dSq[i, j] = big[i, j]
    dV = Pq.T @ dOq[0, 0]
    dQ = (1 / 8) * dSk @ Kk[0, 0]
    dK = (1 / 8) * dSq.T @ Qq[0, 0]
    assert np.array_equal(g["dV"][0, 0], dV)
    assert np.array_equal(g["dQ"][0, 0], dQ)
    assert np.array_equal(g["dK"][0, 0], dK)
