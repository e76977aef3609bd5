"""Pins of the mask-variant oracle (CPU).

Each variant is pinned outside its own dense-mask formulation: reductions to the
causal oracle and to full attention (torch SDPA, fp64), closed forms, and brute
force that rebuilds, for each query row, the sub-sequence of keys it sees (plus
the row) and evaluates it with the causal or full oracle.
"""
import numpy as np
import pytest
import torch

import oracle

H, D, SCALE = 2, 64, 0.125


def _qkv(L, seed):
    return np.random.default_rng(seed).standard_normal((L, 3 * H * D))


def _full(qkv):
    """Per-head attention over every key (no mask), torch SDPA in fp64."""
    L = qkv.shape[0]
    t = torch.tensor(qkv)
    q, k, v = (t[:, o * H * D:(o + 1) * H * D].reshape(L, H, D).transpose(0, 1) for o in range(3))
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=SCALE).transpose(0, 1).reshape(L, H * D).numpy()


def _row_on_subsequence(qkv, i, keys, causal):
    """Row i's output when it attends exactly to `keys` (ascending, containing i)."""
    sub = qkv[keys]
    pos = keys.index(i)
    if causal:  # i is the last key it sees
        assert pos == len(keys) - 1
        return oracle.varlen_causal_attention(sub, [0, len(keys)], H, D, SCALE)[pos]
    return _full(sub)[pos]


def test_defaults_are_the_causal_oracle():
    lengths = [1, 9, 0, 70]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    q = _qkv(80, 1)
    a = oracle.varlen_attention_masked(q, cu, H, D, SCALE)
    b = oracle.varlen_causal_attention(q, cu, H, D, SCALE)
    assert np.max(np.abs(a - b)) <= 1e-15


def test_no_mask_is_full_attention():
    q = _qkv(33, 2)
    a = oracle.varlen_attention_masked(q, [0, 33], H, D, SCALE, window=(-1, -1))
    assert np.max(np.abs(a - _full(q))) <= 1e-12


def test_closed_forms():
    q = _qkv(40, 3)
    # a window of 0 keys to the left: every row returns its own v
    a = oracle.varlen_attention_masked(q, [0, 40], H, D, SCALE, window=(0, 0))
    assert np.max(np.abs(a - q[:, 2 * H * D:])) <= 1e-15
    # a window covering the user is the causal mask; a context covering it, full attention
    causal = oracle.varlen_causal_attention(q, [0, 40], H, D, SCALE)
    assert np.max(np.abs(oracle.varlen_attention_masked(q, [0, 40], H, D, SCALE, window=(39, 0)) - causal)) <= 1e-15
    assert np.max(np.abs(oracle.varlen_attention_masked(q, [0, 40], H, D, SCALE, num_contexts=[40]) - _full(q))) \
        <= 1e-12
    # one context token changes nothing (row 0 sees key 0 either way)
    assert np.max(np.abs(oracle.varlen_attention_masked(q, [0, 40], H, D, SCALE, num_contexts=[1]) - causal)) <= 1e-15


@pytest.mark.parametrize("c,g,group,left", [(0, 6, 1, -1), (5, 9, 3, -1), (4, 0, 1, 7), (3, 8, 4, 5), (0, 10, 10, 2)])
def test_rows_equal_their_visible_subsequence(c, g, group, left):
    L = 37
    q = _qkv(L, 4 + c + g)
    out = oracle.varlen_attention_masked(q, [0, L], H, D, SCALE, num_contexts=[c], num_targets=[g], group=group,
                                         window=(left, 0))
    nc = L - g
    for i in range(L):
        if i < c:  # a context row sees the whole context, in both directions
            want = _row_on_subsequence(q, i, list(range(c)), causal=False)
        else:
            lo = max(c, i - left) if left >= 0 else c
            keys = list(range(c)) + list(range(lo, min(i, nc - 1) + 1))
            if i >= nc:
                gs = nc + ((i - nc) // group) * group
                keys += list(range(gs, i + 1))
            want = _row_on_subsequence(q, i, keys, causal=True)
        assert np.max(np.abs(out[i] - want)) <= 1e-12, i


@pytest.mark.parametrize("left,right", [(3, 2), (-1, 4), (6, -1)])
def test_non_causal_windows_by_subsequence(left, right):
    L = 25
    q = _qkv(L, 9)
    out = oracle.varlen_attention_masked(q, [0, L], H, D, SCALE, window=(left, right))
    for i in range(L):
        lo = max(0, i - left) if left >= 0 else 0
        hi = min(L - 1, i + right) if right >= 0 else L - 1
        assert np.max(np.abs(out[i] - _row_on_subsequence(q, i, list(range(lo, hi + 1)), causal=False))) <= 1e-12


def test_candidates_do_not_see_other_groups():
    L, g = 30, 12
    q = _qkv(L, 10)
    a = oracle.varlen_attention_masked(q, [0, L], H, D, SCALE, num_targets=[g], group=4)
    q2 = q.copy()
    q2[22:26] += 3.0  # the third group (rows 26..29 sit in the fourth)
    b = oracle.varlen_attention_masked(q2, [0, L], H, D, SCALE, num_targets=[g], group=4)
    assert np.array_equal(a[:22], b[:22]) and np.array_equal(a[26:], b[26:])
    assert not np.array_equal(a[22:26], b[22:26])
