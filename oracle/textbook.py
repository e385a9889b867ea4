"""fp64 textbook softmax attention -- TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The plain definition: S = Q K^T / sqrt(D), causal mask j <= i when asked, P = softmax(S)
row-wise, O = P V, LSE = log sum_j exp(S_ij). Query head h reads KV head h / (H/Hkv).
It is the reference for the BF16-MFMA variant and the target that the C oracle's online
softmax must reduce to when every quantizer is the identity.
"""
from __future__ import annotations

import numpy as np


def _expand_kv(K, H):
    Hkv = K.shape[1]
    return np.repeat(K, H // Hkv, axis=1)


def attention(Q, K, V, causal=False):
    Q = np.asarray(Q, np.float64)
    K = _expand_kv(np.asarray(K, np.float64), Q.shape[1])
    V = _expand_kv(np.asarray(V, np.float64), Q.shape[1])
    D = Q.shape[-1]
    N = Q.shape[2]
    S = np.matmul(Q, np.swapaxes(K, -1, -2)) / np.sqrt(D)
    if causal:
        mask = np.triu(np.ones((N, N), bool), k=1)
        S = np.where(mask, -np.inf, S)
    m = S.max(axis=-1, keepdims=True)
    E = np.exp(S - m)
    Z = E.sum(axis=-1, keepdims=True)
    P = E / Z
    O = np.matmul(P, V)
    lse = (m + np.log(Z))[..., 0]
    return O, lse, P


def loss(Q, K, V, dO, causal=False):
    """L = sum(dO * O): its gradient with respect to O is dO."""
    O, _, _ = attention(Q, K, V, causal)
    return float(np.sum(np.asarray(dO, np.float64) * O))
