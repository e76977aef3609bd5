"""Seeded synthetic packed-batch generators.

This module only draws inputs: per-user lengths, the cumulative offsets
``cu_seqlens = [0, L0, L0+L1, ...]`` and the packed ``qkv`` rows rounded to
bf16.  It holds none of the attention arithmetic, so both the fp64 oracle
(``oracle/``) and the HIP path (``varlen_causal_attention_amd``) can be fed
from it without sharing any code with each other.

The packed layout follows the cti2026 README (git.firegun.top/Days-gone/cti2026),
input table (``user_offsets`` = ``[0, len1, len1+len2, ..., total_tokens]``) and
the Transformer layer listing there (``qkv = Linear_qkv(x)`` of width 1536 for
8 heads x 64).  The pages measure on a private competition dataset that is not
available; the five configurations below are synthetic stand-ins shaped like
the pages' batches (about 114 tokens per user at 6823 tokens / 60 users).

Recipe (every configuration): one ``numpy.random.default_rng(seed)``; lengths
are drawn first, then ``qkv = rng.standard_normal((T, 1536), float32)`` (times
``value_scale``), then rounded to bf16 with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

N_HEADS = 8
HEAD_DIM = 64
QKV_COLS = 3 * N_HEADS * HEAD_DIM  # 1536
OUT_COLS = N_HEADS * HEAD_DIM  # 512


@dataclasses.dataclass
class Workload:
    name: str
    lengths: np.ndarray  # int64 [U]
    cu_seqlens: np.ndarray  # int32 [U+1]
    max_seqlen: int  # value passed to the op (an upper bound, may exceed max(lengths))
    scale: float
    n_heads: int = N_HEADS
    head_dim: int = HEAD_DIM
    qkv_bf16: Optional["object"] = None  # torch.bfloat16 CPU tensor [T, 3*H*D]

    @property
    def num_users(self) -> int:
        return int(self.lengths.shape[0])

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    def causal_flops(self) -> float:
        """Algorithmic FLOPs: sum_u 4*H*D*L(L+1)/2 (QK^T and PV over the causal triangle)."""
        L = self.lengths.astype(np.float64)
        return float(np.sum(4.0 * self.n_heads * self.head_dim * L * (L + 1.0) / 2.0))

    def algorithmic_bytes(self) -> int:
        """qkv read once (3*H*D bf16) plus out written once (H*D bf16) per token."""
        return self.total_tokens * (3 + 1) * self.n_heads * self.head_dim * 2


def cu_from_lengths(lengths: Sequence[int]) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(lengths.shape[0] + 1, dtype=np.int64)
    np.cumsum(lengths, out=cu[1:])
    if cu[-1] >= 2**31:
        raise ValueError("total tokens must fit int32")
    return cu.astype(np.int32)


def rescale_to_sum(raw: np.ndarray, total: int, cap: int) -> np.ndarray:
    """Integer lengths in [1, cap] proportional to ``raw`` that sum exactly to ``total``.

    x = raw * total / sum(raw); L = clip(floor(x), 1, cap); then walk users in
    descending fractional part of x (stable, cyclic) adding 1 while sum < total
    (skipping users at cap) or subtracting 1 while sum > total (skipping users at 1).
    """
    raw = np.asarray(raw, dtype=np.float64)
    n = raw.shape[0]
    if not (n <= total <= n * cap):
        raise ValueError("total not reachable with lengths in [1, cap]")
    x = raw * (float(total) / float(raw.sum()))
    fl = np.floor(x)
    frac = x - fl
    L = np.clip(fl, 1, cap).astype(np.int64)
    order = np.argsort(-frac, kind="stable")
    s = int(L.sum())
    i = 0
    while s != total:
        u = order[i % n]
        if s < total and L[u] < cap:
            L[u] += 1
            s += 1
        elif s > total and L[u] > 1:
            L[u] -= 1
            s -= 1
        i += 1
    return L


def _lognormal_lengths(rng, n_users, total, cap):
    raw = np.clip(np.round(rng.lognormal(mean=4.3, sigma=0.9, size=n_users)), 1, cap)
    return rescale_to_sum(raw, total, cap)


def config_lengths(idx: int, rng: np.random.Generator):
    """(lengths, max_seqlen, value_scale) for configuration ``idx`` (1-based)."""
    if idx == 1:
        return np.array([1, 7, 16, 40], dtype=np.int64), 40, 1.0
    if idx == 2:
        L = _lognormal_lengths(rng, 60, 6823, 1024)
        return L, int(L.max()), 1.0
    if idx == 3:
        L = _lognormal_lengths(rng, 390, 44000, 2048)
        return L, int(L.max()), 1.0
    if idx == 4:
        L = np.concatenate([[8192], rng.integers(1, 65, 512)]).astype(np.int64)
        return L, 8192, 0.5
    if idx == 5:
        raw = np.clip(rng.zipf(1.3, 1000), 1, 4096).astype(np.float64)
        L = rescale_to_sum(raw, 131072, 4096)
        return L, 4096, 1.0
    raise ValueError(f"unknown configuration {idx}")


CONFIG_NAMES = {
    1: "tiny_4users_64tok",
    2: "pages_6823tok_60users",
    3: "long_44000tok_390users",
    4: "skewed_8192plus512users",
    5: "zipf_131072tok_1000users",
}


def draw_qkv(rng: np.random.Generator, total_tokens: int, cols: int = QKV_COLS, value_scale: float = 1.0):
    """N(0,1) float32 draws times ``value_scale``, rounded to bf16 (RNE) as a torch CPU tensor."""
    import torch

    x = rng.standard_normal((total_tokens, cols), dtype=np.float32)
    if value_scale != 1.0:
        x *= np.float32(value_scale)
    return torch.from_numpy(x).to(torch.bfloat16)


def draw_dout(total_tokens: int, n_heads: int = N_HEADS, seed: int = 1):
    """An upstream gradient dL/dout for the backward: N(0,1) float32 draws of
    ``[total_tokens, n_heads*64]`` rounded to bf16 (RNE), from its own seeded
    generator, as a torch CPU tensor."""
    rng = np.random.default_rng(seed)
    return draw_qkv(rng, total_tokens, cols=n_heads * HEAD_DIM)


@dataclasses.dataclass
class LayerParams:
    """Synthetic parameters of the layer's attention sub-block (bf16 torch CPU
    tensors, nn.Linear layout [out, in]): no trained weights exist here."""
    gamma: "object"
    beta: "object"
    w_qkv: "object"
    b_qkv: "object"
    w_out: "object"
    b_out: "object"
    eps: float = 1e-5


def make_layer_params(d_model: int = OUT_COLS, n_heads: int = N_HEADS, seed: int = 3) -> LayerParams:
    """gamma ~ 1 + 0.1 N(0,1), beta ~ 0.1 N(0,1), weights ~ N(0, 1/d_model) (unit
    variance through each product), biases ~ 0.1 N(0,1); rounded to bf16."""
    import torch

    rng = np.random.default_rng(seed)

    def bf16(a):
        return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)

    n_qkv = 3 * n_heads * HEAD_DIM
    return LayerParams(
        gamma=bf16(1.0 + 0.1 * rng.standard_normal(d_model)),
        beta=bf16(0.1 * rng.standard_normal(d_model)),
        w_qkv=bf16(rng.standard_normal((n_qkv, d_model)) / np.sqrt(d_model)),
        b_qkv=bf16(0.1 * rng.standard_normal(n_qkv)),
        w_out=bf16(rng.standard_normal((d_model, n_heads * HEAD_DIM)) / np.sqrt(n_heads * HEAD_DIM)),
        b_out=bf16(0.1 * rng.standard_normal(d_model)),
    )


def draw_layer_input(total_tokens: int, d_model: int = OUT_COLS, seed: int = 2):
    """The layer input x: N(0,1) float32 draws [total_tokens, d_model] rounded to bf16."""
    rng = np.random.default_rng(seed)
    return draw_qkv(rng, total_tokens, cols=d_model)


def make_config(idx: int, seed: int = 0, with_values: bool = True) -> Workload:
    rng = np.random.default_rng(seed)
    lengths, max_seqlen, vscale = config_lengths(idx, rng)
    cu = cu_from_lengths(lengths)
    w = Workload(CONFIG_NAMES[idx], lengths, cu, max_seqlen, 1.0 / 8.0)
    if with_values:
        w.qkv_bf16 = draw_qkv(rng, int(cu[-1]), value_scale=vscale)
    return w


def make_from_lengths(lengths: Sequence[int], seed: int = 0, n_heads: int = N_HEADS,
                      value_scale: float = 1.0, max_seqlen: Optional[int] = None,
                      name: str = "custom") -> Workload:
    """A packed batch with the given per-user lengths (zeros allowed) and N(0,1) bf16 values."""
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = cu_from_lengths(lengths)
    ms = int(lengths.max()) if max_seqlen is None and lengths.size else (max_seqlen or 0)
    w = Workload(name, lengths, cu, ms, 1.0 / np.sqrt(HEAD_DIM), n_heads=n_heads)
    w.qkv_bf16 = draw_qkv(rng, int(cu[-1]), cols=3 * n_heads * HEAD_DIM, value_scale=value_scale)
    return w


# Offsets [0, 10, 22, 37] (three users of 10, 12 and 15 tokens) are the shape of
# the block-diagonal equivalence test in the CTI-Inference-Opt plan
# 2026-06-14-cti-auc-recovery, Task 9, Step 1 (B=1, H=8, S=37, Dh=64).
PLAN_TEST_LENGTHS: List[int] = [10, 12, 15]
