"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the attention method: it only draws Gaussian tensors
with NumPy's PCG64 generator and rounds them to bfloat16 bits (round to nearest even).
Both the GPU path and the CPU oracle consume its output.

Recipe: ``rng = np.random.default_rng(seed)``; Q, then K, then V are drawn as
``rng.standard_normal(shape, dtype=float32)`` in [B, heads, N, D] order; dO (backward
only) is drawn next and multiplied by its standard deviation in float32; for the
outlier-channel workload, ``rng.choice(D, n_out, replace=False)`` per head follows, and
those channels of that head's Q, K and V are multiplied by 10 in float32. Every tensor is
then rounded to bfloat16.

Projection inputs (the QKV projection that feeds attention): X [B, N, Dm] is drawn first as
``standard_normal``, then the weight [(H + 2 Hkv) D, Dm] as ``standard_normal`` multiplied by
1/sqrt(Dm) in float32 (so that Q, K and V come out with unit variance), both rounded to bfloat16.
The "grid" variant draws integers instead (X in [-8, 8] / 4, W in [-8, 8] / 8), for which every
partial sum of X W^T is exact in float32.
"""
from __future__ import annotations

import math

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest even), returned as uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def attention_inputs(B, H, Hkv, N, D, seed=0, with_do=False, do_std=1e-2, outlier_frac=0.0):
    """Returns dict of bf16 bit tensors q [B,H,N,D], k/v [B,Hkv,N,D] (and do [B,H,N,D])."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N, D), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, N, D), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, N, D), dtype=np.float32)
    out = {}
    if with_do:
        do = rng.standard_normal((B, H, N, D), dtype=np.float32) * np.float32(do_std)
        out["do"] = f32_to_bf16_bits(do)
    if outlier_frac > 0.0:
        if H != Hkv:
            raise ValueError("outlier channels are defined for H == Hkv")
        n_out = int(math.ceil(outlier_frac * D))
        chans = np.zeros((H, n_out), np.int64)
        for h in range(H):
            ch = rng.choice(D, n_out, replace=False)
            chans[h] = ch
            q[:, h, :, ch] *= np.float32(10.0)
            k[:, h, :, ch] *= np.float32(10.0)
            v[:, h, :, ch] *= np.float32(10.0)
        out["outlier_channels"] = chans
    out["q"] = f32_to_bf16_bits(q)
    out["k"] = f32_to_bf16_bits(k)
    out["v"] = f32_to_bf16_bits(v)
    return out


def projection_inputs(B, N, Dm, H, Hkv, D, seed=0, grid=False):
    """Returns dict of bf16 bit tensors x [B, N, Dm] and w [(H + 2 Hkv) D, Dm]."""
    rng = np.random.default_rng(seed)
    F = (H + 2 * Hkv) * D
    if grid:
        x = rng.integers(-8, 9, (B, N, Dm)).astype(np.float32) * np.float32(0.25)
        w = rng.integers(-8, 9, (F, Dm)).astype(np.float32) * np.float32(0.125)
    else:
        x = rng.standard_normal((B, N, Dm), dtype=np.float32)
        w = rng.standard_normal((F, Dm), dtype=np.float32) * np.float32(1.0 / math.sqrt(Dm))
    return {"x": f32_to_bf16_bits(x), "w": f32_to_bf16_bits(w)}


# The workloads (shapes of the pages' benchmarks and training runs).
WORKLOADS = {
    "tiny_h1_n128_d64": dict(B=1, H=1, Hkv=1, N=128, D=64, causal=False),
    "directp_h16_n4096_d128": dict(B=1, H=16, Hkv=16, N=4096, D=128, causal=False),
    "dit_h24_n32768_d128_outliers": dict(B=1, H=24, Hkv=24, N=32768, D=128, causal=False, outlier_frac=0.01),
    "causal_llama8b_h32kv8_n8192_d128": dict(B=1, H=32, Hkv=8, N=8192, D=128, causal=True),
    "causal_bwd_llama8b_h32kv8_n8192_d128": dict(B=1, H=32, Hkv=8, N=8192, D=128, causal=True, with_do=True),
}
