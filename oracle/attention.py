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


def varlen_causal_attention_backward(qkv: np.ndarray, cu_seqlens, dout: np.ndarray, n_heads: int, head_dim: int,
                                     scale: float) -> np.ndarray:
    """fp64 gradient ``dL/dqkv`` ``[T, 3*n_heads*head_dim]`` of the forward above, given ``dout = dL/dout``.

    The training step of the same op: the recsys README (github.com/cry-daniel/
    recsys), FusedHSTULayer section, runs an attention backward
    (``hstu_attn_varlen_bwd``) between the layer's other backward kernels; the
    pages give no formula for it, so this is the derivative of the definition
    written out.  Per user and head, with S = scale Q K^T (causal), P = rowwise
    softmax(S), O = P V:
      dV = P^T dO;   dP = dO V^T;   dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik);
      dQ = scale dS K;   dK = scale dS^T Q.
    (sum_k P_ik dP_ik = dO_i . O_i.)  Columns of ``dqkv`` follow the qkv layout.
    """
    qkv = np.asarray(qkv, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    hd = n_heads * head_dim
    T = int(cu[-1])
    if qkv.shape != (T, 3 * hd) or dout.shape != (T, hd):
        raise ValueError("shape mismatch")
    dqkv = np.zeros_like(qkv)
    for u in range(cu.shape[0] - 1):
        s, e = int(cu[u]), int(cu[u + 1])
        L = e - s
        if L <= 0:
            continue
        allowed = np.tril(np.ones((L, L), dtype=bool))
        for h in range(n_heads):
            q, k, v = split_qkv_head(qkv, slice(s, e), h, n_heads, head_dim)
            c = h * head_dim
            do = dout[s:e, c:c + head_dim]
            p = _masked_softmax_rows(scale * (q @ k.T), allowed)
            dp = do @ v.T
            ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
            dqkv[s:e, c:c + head_dim] = scale * (ds @ k)
            dqkv[s:e, hd + c:hd + c + head_dim] = scale * (ds.T @ q)
            dqkv[s:e, 2 * hd + c:2 * hd + c + head_dim] = p.T @ do
    return dqkv


def varlen_causal_attention_backward_magnitude(qkv: np.ndarray, cu_seqlens, dout: np.ndarray, n_heads: int,
                                               head_dim: int, scale: float) -> np.ndarray:
    """fp64 ``[T, 3*n_heads*head_dim]``: each gradient element of
    ``varlen_causal_attention_backward`` evaluated with every term of its expansion
    in the inputs and P replaced by its absolute value (sums of magnitudes, no
    cancellation):
      dS_mag_ij = P_ij (|dP|_ij + sum_d |dO_id| (P |V|)_id),  |dP| = |dO| |V|^T,
      dQ_mag = scale dS_mag |K|,  dK_mag = scale dS_mag^T |Q|,  dV_mag = P^T |dO|.
    Computing the gradient with each term perturbed by a relative error <= e
    changes it by at most e times this (to first order), so a test's tolerance
    for a rounded computation uses it; where terms cancel it far exceeds the
    gradient.
    """
    qkv = np.asarray(qkv, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    hd = n_heads * head_dim
    mag = np.zeros_like(qkv)
    for u in range(cu.shape[0] - 1):
        s, e = int(cu[u]), int(cu[u + 1])
        L = e - s
        if L <= 0:
            continue
        allowed = np.tril(np.ones((L, L), dtype=bool))
        for h in range(n_heads):
            q, k, v = split_qkv_head(qkv, slice(s, e), h, n_heads, head_dim)
            c = h * head_dim
            ado = np.abs(dout[s:e, c:c + head_dim])
            p = _masked_softmax_rows(scale * (q @ k.T), allowed)
            dmag = np.sum(ado * (p @ np.abs(v)), axis=1, keepdims=True)
            dsmag = p * (ado @ np.abs(v).T + dmag)
            mag[s:e, c:c + head_dim] = scale * (dsmag @ np.abs(k))
            mag[s:e, hd + c:hd + c + head_dim] = scale * (dsmag.T @ np.abs(q))
            mag[s:e, 2 * hd + c:2 * hd + c + head_dim] = p.T @ ado
    return mag


def varlen_causal_attention_lse(qkv: np.ndarray, cu_seqlens, n_heads: int, head_dim: int,
                                scale: float) -> np.ndarray:
    """fp64 ``[T, n_heads]``: ln sum_{j <= i} exp(scale q_i . k_j) over the row's user (the
    softmax's normaliser in log form, which the backward uses to recompute P)."""
    qkv = np.asarray(qkv, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T = int(cu[-1])
    lse = np.zeros((T, n_heads), dtype=np.float64)
    for u in range(cu.shape[0] - 1):
        s, e = int(cu[u]), int(cu[u + 1])
        L = e - s
        if L <= 0:
            continue
        allowed = np.tril(np.ones((L, L), dtype=bool))
        for h in range(n_heads):
            q, k, _ = split_qkv_head(qkv, slice(s, e), h, n_heads, head_dim)
            z = np.where(allowed, scale * (q @ k.T), -np.inf)
            m = z.max(axis=1)
            lse[s:e, h] = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
    return lse


def hstu_mask(L: int, c: int = 0, g: int = 0, group: int = 1, window=(-1, 0)) -> np.ndarray:
    """Boolean ``[L, L]`` mask of one user (entry (i, j): query row i sees key j).

    The recsys README (github.com/cry-daniel/recsys), HSTU section, gives the
    sequence as [contextual tokens][historical tokens][candidate tokens] --
    contextual tokens attended bidirectionally, history causally, candidates in
    groups of target_group_size -- and ``window_size=(-1, 0)`` as the causal
    default of its local mask.  Reading taken (the page gives only this layout):
    with nc = L - g,
      right == 0: every row sees the context keys j < c; a row i >= c sees the
        history keys max(c, i - left) <= j <= min(i, nc - 1) (left -1: no bound);
        a candidate row i >= nc also sees its own group's keys gs(i) <= j <= i,
        gs(i) = nc + floor((i - nc) / group) * group;
      otherwise (c = g = 0): i - left <= j <= i + right (-1: no bound that side).
    """
    left, right = window
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    lo = np.maximum(0, i - left) if left >= 0 else np.zeros_like(i)
    if right != 0:
        if c or g:
            raise ValueError("contexts and targets need a causal window")
        hi = np.minimum(L - 1, i + right) if right >= 0 else np.full_like(i, L - 1)
        return (j >= lo) & (j <= hi)
    nc = L - g
    ctx = j < c
    hist = (i >= c) & (j >= np.maximum(c, lo)) & (j <= np.minimum(i, nc - 1))
    gs = nc + ((i - nc) // group) * group
    grp = (i >= nc) & (j >= gs) & (j <= i)
    return ctx | hist | grp


def varlen_attention_masked(qkv: np.ndarray, cu_seqlens, n_heads: int, head_dim: int, scale: float,
                            num_contexts=None, num_targets=None, group: int = 1, window=(-1, 0)) -> np.ndarray:
    """fp64 ``[T, n_heads*head_dim]``: per user and head, softmax(scale Q K^T restricted to
    ``hstu_mask``) V, the user's context / candidate counts clamped to its length."""
    qkv = np.asarray(qkv, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T = int(cu[-1])
    out = np.zeros((T, n_heads * head_dim), dtype=np.float64)
    for u in range(cu.shape[0] - 1):
        s, e = int(cu[u]), int(cu[u + 1])
        L = e - s
        if L <= 0:
            continue
        c = min(max(int(num_contexts[u]), 0), L) if num_contexts is not None else 0
        g = min(max(int(num_targets[u]), 0), L - c) if num_targets is not None else 0
        allowed = hstu_mask(L, c, g, group, window)
        for h in range(n_heads):
            q, k, v = split_qkv_head(qkv, slice(s, e), h, n_heads, head_dim)
            out[s:e, h * head_dim:(h + 1) * head_dim] = _masked_softmax_rows(scale * (q @ k.T), allowed) @ v
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

    This is the mask that the plan 2026-06-14-cti-auc-recovery (Task 9, Step 3)
    applies to the whole packed stream.  Here it is formed from its definition:
    users own contiguous row ranges, so "same user and j <= i" holds exactly when
    the first row of row i's user is <= j <= i.
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T = int(cu[-1])
    rows = np.arange(T)
    # The user owning row r is the last u with cu[u] <= r (zero-length users own no row).
    first = cu[np.searchsorted(cu, rows, side="right") - 1]
    cols = rows[None, :]
    return (cols >= first[:, None]) & (cols <= rows[:, None])


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
