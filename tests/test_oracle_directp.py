"""Pins for the oracle's Direct-P probability construction.

Direct-P (gist.science summary, Methodology 1 "Direct Mapping"; arXiv abstract) classifies
each normalized log-score into one of the eight non-negative E2M1 magnitudes. The oracle's
reading: the class boundaries are where round-to-nearest-even E2M1 of the exact value 2^u
changes code. These tests derive those boundaries independently in 60-digit decimal
arithmetic and check the classifier against exp-then-round by brute force; they also check
that one block of Direct-P probabilities equals the MX quantization (the pinned quantizer) of
the exact probabilities exp2((S - m) c).
"""
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest

getcontext().prec = 60
LN2 = Decimal(2).ln()
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _pow2_dec(u):
    """2^u in 60-digit decimal for a binary32 u (exact for integer u)."""
    uf = float(u)
    if uf == int(uf) and abs(uf) < 200:
        return Decimal(2) ** int(uf)
    return (Decimal(uf) * LN2).exp()


def _rne_code_exact(u, grid):
    """Nearest code of exact 2^u on ``grid``, ties to even code, saturating."""
    p = _pow2_dec(u)
    top = Decimal(grid[-1])
    if p >= top:
        return len(grid) - 1
    lo = max(i for i, g in enumerate(grid) if Decimal(g) <= p)
    mid = (Decimal(grid[lo]) + Decimal(grid[lo + 1])) / 2
    if p < mid:
        return lo
    if p > mid:
        return lo + 1
    return lo if lo % 2 == 0 else lo + 1


def test_thresholds_are_exact_step_points(orc):
    T = orc.directp_thresholds()
    assert np.all(np.diff(T) > 0)
    for k, t in enumerate(T):
        t = np.float32(t)
        below = np.nextafter(t, np.float32(-np.inf))
        # code(t) = k + 1 and code(previous float) = k under exp-then-round
        assert _rne_code_exact(t, E2M1) == k + 1, k
        assert _rne_code_exact(below, E2M1) == k, k


def test_classifier_equals_exp_then_round(orc):
    T = orc.directp_thresholds()
    us = []
    for t in T:  # every binary32 within 40 ulps of each step point
        x = np.float32(t)
        for _ in range(40):
            x = np.nextafter(x, np.float32(-np.inf))
        for _ in range(81):
            us.append(x)
            x = np.nextafter(x, np.float32(np.inf))
    rng = np.random.default_rng(1)
    us += list(rng.uniform(-8.0, 4.0, 3000).astype(np.float32))
    us += [np.float32(v) for v in (-2.0, -1.0, 0.0, 1.0, 2.0, 3.0, -100.0, 100.0)]
    for u in us:
        assert orc.directp_code(u) == _rne_code_exact(u, E2M1), float(u)


def test_e4m3_of_exp2_brute_force(orc):
    grid = [orc.e4m3_decode(c) for c in range(127)]
    rng = np.random.default_rng(2)
    us = list(rng.uniform(-12.0, 9.5, 3000).astype(np.float32))
    # near the midpoints between adjacent codes, and the saturation point
    for a, b in zip(grid[1:60:7], grid[2:61:7]):
        m = np.float32(math.log2(0.5 * (a + b)))
        x = m
        for _ in range(3):
            x = np.nextafter(x, np.float32(-np.inf))
        for _ in range(7):
            us.append(x)
            x = np.nextafter(x, np.float32(np.inf))
    us += [np.float32(v) for v in (8.0, 8.8, 8.9, 9.0, -9.0, -10.0)]
    for u in us:
        assert orc.e4m3_code_of_exp2(u) == _rne_code_exact(u, grid), float(u)


def _mx_quantize_e2m1_block_exact(p, grid):
    """Reference for one block: OCP scale from the block max, nearest-even codes."""
    amax = max(p)
    e = math.floor(math.log2(amax)) - 2
    e = max(e, -127)
    return e, [grid[_nearest(x / 2.0 ** e, grid)] * 2.0 ** e for x in p]


def _nearest(a, grid):
    if a >= grid[-1]:
        return len(grid) - 1
    lo = max(i for i, g in enumerate(grid) if g <= a)
    mid = 0.5 * (grid[lo] + grid[lo + 1])
    return lo if a < mid or (a == mid and lo % 2 == 0) else lo + 1


@pytest.mark.parametrize("D", [64, 128])
def test_block_probs_are_mx_quantized_probabilities(orc, D):
    """P of a 32-key block = MX-E2M1 quantization of exp2((S - m) c), away from the rare
    scores where binary32 u and binary64 round differently."""
    rng = np.random.default_rng(D)
    c = float(orc.log2e_scale(D))
    agree = total = 0
    for trial in range(400):
        s = (rng.standard_normal(32) * 11.0).astype(np.float32)
        s = np.round(s * 4) / 4  # MX scores are multiples of small powers of two
        m = np.float32(s.max() + abs(rng.standard_normal()) * 20.0 * (trial % 3 != 0))
        eb, p = orc.block_probs(s, m, D, orc.P_DIRECT)
        exact = [2.0 ** ((float(x) - float(m)) * c) for x in s]
        e_ref, p_ref = _mx_quantize_e2m1_block_exact(exact, E2M1)
        assert eb == e_ref, trial
        agree += int(np.sum(np.asarray(p_ref) == p))
        total += 32
    assert agree >= total - 2, (agree, total)


def test_block_max_gets_probability_one(orc):
    # u of the running-max score is 2 (E2M1: 4 * 2^-2) or 8 (E4M3: 256 * 2^-8)
    rng = np.random.default_rng(9)
    for _ in range(200):
        s = (rng.standard_normal(32) * 30).astype(np.float32)
        m = s.max()
        for pmode in (orc.P_DIRECT, orc.P_E4M3):
            _, p = orc.block_probs(s, m, 128, pmode)
            assert p[np.argmax(s)] == 1.0
            assert np.all(p <= 1.5)


def test_far_block_underflows_to_zero(orc):
    s = np.full(32, -1000.0, np.float32)
    eb, p = orc.block_probs(s, np.float32(1000.0), 128, orc.P_DIRECT)
    assert eb == -127 and np.all(p == 0.0)
