"""fp64 reference for varlen block-diagonal causal self-attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

What is computed (the plain definition; no tiling, no online softmax):

* Packed stream.  Users' sequences are concatenated into ``T`` rows; user ``u``
  owns rows ``cu[u] .. cu[u+1]-1``.  cti2026 README (git.firegun.top/Days-gone/
  cti2026), input table: ``user_offsets = [0, len1, len1+len2, ..., total_tokens]``.
* Columns of ``qkv`` (width ``3*H*D``): q in ``[0, H*D)``, k in ``[H*D, 2*H*D)``,
  v in ``[2*H*D, 3*H*D)``, head ``h`` at ``h*D .. h*D+D-1`` inside each.  The
  pages only give the width (``qkv = Linear_qkv(x)  # [total_tokens, 1536]`` in
  the cti2026 Transformer-layer listing); this split is the plain reading.
* Attention.  softmax(Q K^T / sqrt(d)) V -- CTI-Inference-Opt
  推理优化方案 (inference optimisation plan), section 5.2 -- with the scale
  passed explicitly.  Query ``i`` of a user sees keys ``0..i`` of the same user
  only (diagonal included): cti2026 README, FlashAttention_Varlen section,
  "operator design" (causal pruning: row i looks at keys 0..i; isolation across
  users), and the plan 2026-06-14-cti-auc-recovery, Task 9, Step 3 (mask =
  same-user AND lower-triangular).  Masked scores are -inf before the softmax
  (推理优化方案 section 5.4: masked_fill(mask == 0, -inf)).
"""
from __future__ import annotations

import numpy as np


def split_qkv_head(qkv: np.ndarray, rows: slice, h: int, n_heads: int, head_dim: int):
    """Q, K, V blocks ``[rows, head_dim]`` of head ``h`` from the packed qkv matrix."""
    hd = n_heads * head_dim
    c = h * head_dim
    q = qkv[rows, c:c + head_dim]
    k = qkv[rows, hd + c:hd + c + head_dim]
    v = qkv[rows, 2 * hd + c:2 * hd + c + head_dim]
    return q, k, v


def _masked_softmax_rows(scores: np.ndarray, allowed: np.ndarray) -> np.ndarray:
    """Row softmax of ``scores`` with disallowed entries set to -inf first."""
    s = np.where(allowed, scores, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=1, keepdims=True)


def varlen_causal_attention(qkv: np.ndarray, cu_seqlens, n_heads: int, head_dim: int,
                            scale: float) -> np.ndarray:
    """fp64 ``[T, n_heads*head_dim]`` output, each user and head done as one dense L x L problem.

    ``qkv`` must already hold the exact bf16 input values as fp64 (upcasting bf16 to
    fp64 is exact).  Zero-length users produce no rows.
    """
    qkv = np.asarray(qkv, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T = int(cu[-1])
    if qkv.shape != (T, 3 * n_heads * head_dim):
        raise ValueError(f"qkv shape {qkv.shape} does not match T={T}, H={n_heads}, D={head_dim}")
    out = np.zeros((T, n_heads * head_dim), dtype=np.float64)
    for u in range(cu.shape[0] - 1):
        s, e = int(cu[u]), int(cu[u + 1])
        L = e - s
        if L <= 0:
            continue
        allowed = np.tril(np.ones((L, L), dtype=bool))  # key j <= query i
        for h in range(n_heads):
            q, k, v = split_qkv_head(qkv, slice(s, e), h, n_heads, head_dim)
            p = _masked_softmax_rows(scale * (q @ k.T), allowed)
            out[s:e, h * head_dim:(h + 1) * head_dim] = p @ v
    return out


def varlen_causal_attention_rows(qkv: np.ndarray, cu_seqlens, rows, n_heads: int, head_dim: int,
                                 scale: float) -> np.ndarray:
    """fp64 output of the selected packed rows only, ``[len(rows), n_heads*head_dim]``.

    Row ``r`` of user ``u`` (``cu[u] <= r < cu[u+1]``) attends to rows ``cu[u] .. r``:
    the same definition as ``varlen_causal_attention`` evaluated one query at a
    time, so full-size batches can be checked on a sample of rows.
    """
    qkv = np.asarray(qkv)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    hd = n_heads * head_dim
    out = np.zeros((len(rows), hd), dtype=np.float64)
    for n, r in enumerate(rows):
        u = int(np.searchsorted(cu, r, side="right")) - 1
        s = int(cu[u])
        keys = slice(s, int(r) + 1)
        for h in range(n_heads):
            c = h * head_dim
            q = np.asarray(qkv[r, c:c + head_dim], dtype=np.float64)
            k = np.asarray(qkv[keys, hd + c:hd + c + head_dim], dtype=np.float64)
            v = np.asarray(qkv[keys, 2 * hd + c:2 * hd + c + head_dim], dtype=np.float64)
            z = scale * (k @ q)
            e = np.exp(z - z.max())
            out[n, c:c + head_dim] = (e / e.sum()) @ v
    return out


def block_diagonal_causal_mask(cu_seqlens) -> np.ndarray:
    """Dense boolean ``[T, T]`` mask: entry (i, j) is True iff rows i and j belong to
    the same user and j <= i.

    Built the way the plan 2026-06-14-cti-auc-recovery, Task 9, Step 3 builds it:
    a per-row user id (each user index repeated by its length), equality of ids,
    and a lower-triangular matrix over the whole stream.
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    lengths = np.diff(cu)
    uid = np.repeat(np.arange(lengths.shape[0]), lengths)
    same = uid[None, :] == uid[:, None]
    T = uid.shape[0]
    lower = np.tril(np.ones((T, T), dtype=bool))
    return same & lower


def dense_masked_attention(qkv: np.ndarray, cu_seqlens, n_heads: int, head_dim: int,
                           scale: float) -> np.ndarray:
    """The whole packed stream as one ``T x T`` attention per head under the dense mask.

    This is the slow path the pages replace (scores over all T rows, then the
    block-diagonal causal mask); O(T^2) memory, for tiny inputs only.
    """
    qkv = np.asarray(qkv, dtype=np.float64)
    T = qkv.shape[0]
    allowed = block_diagonal_causal_mask(cu_seqlens)
    out = np.zeros((T, n_heads * head_dim), dtype=np.float64)
    if T == 0:
        return out
    for h in range(n_heads):
        q, k, v = split_qkv_head(qkv, slice(0, T), h, n_heads, head_dim)
        p = _masked_softmax_rows(scale * (q @ k.T), allowed)
        out[:, h * head_dim:(h + 1) * head_dim] = p @ v
    return out
