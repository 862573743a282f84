"""Numpy FP64 brute force for tiny shapes.

TEST INFRASTRUCTURE ONLY.  This is a second, independently written statement of
the attention definition ("WS2 Attention PR5 Drift Benchmark", section "Scope":
GQA with contiguous head groups, post-RoPE inputs; out and log-sum-exp as the
outputs).  It deliberately differs from the C oracle in form: it builds the
whole score matrix, exponentiates the raw scores with no max subtraction, and
normalises by the plain sum.  Use only where scores are small enough that
exp() cannot overflow (tiny D, unit-scale inputs).
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def attention(q, k, v, *, scale, causal=True, pos0=0, kv_len=None):
    """q uint16 [B, Sq, Hq, D]; k, v uint16 [B, Skv, Hkv, D] -> (out, lse) float64
    with out [B, Sq, Hq, D] and lse [B, Sq, Hq]."""
    return attention_f64(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v),
                         scale=scale, causal=causal, pos0=pos0, kv_len=kv_len)


def attention_f64(Q, K, V, *, scale, causal=True, pos0=0, kv_len=None):
    """The same definition on real-valued float64 inputs (any values, not only
    bf16 ones), so that it can be differentiated numerically."""
    B, Sq, Hq, D = Q.shape
    Skv, Hkv = K.shape[1], K.shape[2]
    kv_len = Skv if kv_len is None else kv_len
    g = Hq // Hkv
    # expand kv heads to q heads: q head h reads kv head h // g
    Ke = np.repeat(K, g, axis=2)
    Ve = np.repeat(V, g, axis=2)
    s = np.einsum("bqhd,bkhd->bhqk", Q, Ke) * scale
    pos = pos0 + np.arange(Sq)[:, None]
    key = np.arange(Skv)[None, :]
    allowed = key < kv_len
    if causal:
        allowed = allowed & (key <= pos)
    w = np.where(allowed[None, None], np.exp(s), 0.0)
    tot = w.sum(-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.log(tot)
        p = np.where(tot[..., None] > 0, w / tot[..., None], 0.0)
    out = np.einsum("bhqk,bkhd->bqhd", p, Ve)
    return out, np.transpose(lse, (0, 2, 1))
