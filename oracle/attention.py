"""Decode attention over a packed KV cache: the oracle (TEST INFRASTRUCTURE ONLY).

What a fused kernel must compute, written as its plain definition: the cached K and V are first
reconstructed exactly as the codec decodes them (oracle.unpack, or oracle.decode_residual for a
base plus one residual: vllm-rlt pull request #166, the reviews' hot-path options -- dequantize
to BF16 in registers and keep the BF16 matrix multiply; fuse dequantization and residual
reconstruction into attention), then one query token per query head attends over all T cached
tokens in float64:

    s[t] = scale * sum_d q[hq, d] * K[t, hk, d]
    p    = softmax(s)               (over t)
    o[hq, d] = sum_t p[t] * V[t, hk, d]

with grouped-query heads: query head hq reads KV head hk = hq // (Hq // H). The bf16 inputs are
widened exactly; every step after that is float64.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

import oracle


def reconstruct(base: "oracle.Packed", residual: Optional["oracle.Packed"] = None) -> np.ndarray:
    """bf16 bits [T, H, D] of the cache as the codec decodes it (base, or base + residual)."""
    x = oracle.unpack(base)
    if residual is not None:
        x = oracle.decode_residual(residual, x)
    return x


def decode_attention(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, scale: float) -> np.ndarray:
    """float64 [Hq, D] output of one decode step. q: bf16 bits [Hq, D]; k, v: bf16 bits [T, H, D]."""
    q = oracle.bf16_to_f32(q_bits).astype(np.float64)
    k = oracle.bf16_to_f32(k_bits).astype(np.float64)
    v = oracle.bf16_to_f32(v_bits).astype(np.float64)
    Hq, D = q.shape
    T, H, _ = k.shape
    if Hq % H:
        raise ValueError("query heads must be a multiple of KV heads")
    rep = Hq // H
    out = np.zeros((Hq, D), np.float64)
    for hq in range(Hq):
        hk = hq // rep
        s = scale * (k[:, hk, :] @ q[hq])
        p = np.exp(s - s.max())
        p /= p.sum()
        out[hq] = p @ v[:, hk, :]
    return out
