"""fp64 reference of the attention sub-block of the packed Transformer layer.

TEST INFRASTRUCTURE ONLY (see the package docstring).

cti2026 README (git.firegun.top/Days-gone/cti2026), Transformer-layer listing:
    residual = x
    x = LayerNorm(x)
    qkv = Linear_qkv(x)                                  # [total_tokens, 1536]
    attn_out = FlashAttention_Varlen(qkv, user_offsets)
    x = residual + Linear_out(attn_out)
LayerNorm and Linear take their usual definitions (the page names the modules
only): LayerNorm(x) = (x - mean) / sqrt(var + eps) * gamma + beta over each row,
with the population variance; Linear(x) = x W^T + b with W stored [out, in].
"""
from __future__ import annotations

import numpy as np

from .attention import varlen_causal_attention


def layer_norm(x, gamma, beta, eps: float) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    mean = x.mean(axis=1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=1, keepdims=True)
    return (x - mean) / np.sqrt(var + eps) * np.asarray(gamma, np.float64) + np.asarray(beta, np.float64)


def linear(x, w, b) -> np.ndarray:
    """x [T, in] times w [out, in] transposed, plus b [out]."""
    return np.asarray(x, np.float64) @ np.asarray(w, np.float64).T + np.asarray(b, np.float64)


def attention_block(x, cu_seqlens, n_heads: int, head_dim: int, scale: float, gamma, beta, eps: float, w_qkv, b_qkv,
                    w_out, b_out) -> np.ndarray:
    """x + Linear_out(attention(Linear_qkv(LayerNorm(x)))) in fp64, no intermediate rounding."""
    x = np.asarray(x, np.float64)
    qkv = linear(layer_norm(x, gamma, beta, eps), w_qkv, b_qkv)
    attn = varlen_causal_attention(qkv, cu_seqlens, n_heads, head_dim, scale)
    return x + linear(attn, w_out, b_out)
