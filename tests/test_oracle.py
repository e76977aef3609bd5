"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test names what fixes the expected value: a hand-derived fixture, a closed
form, an invariant of the definition, brute force over the dense mask, or a
library routine on a special case that reduces to textbook causal attention.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from conftest import read_golden

H, D = 8, 64


def _qkv64(w):
    return w.qkv_bf16.to(torch.float64).numpy()


def _rand_case(lengths, seed=0, n_heads=H, vs=1.0):
    return workloads.make_from_lengths(lengths, seed=seed, n_heads=n_heads, value_scale=vs)


# ---------------------------------------------------------------- fixtures ---

def test_worked_example_golden():
    g = read_golden("worked_example.txt")
    cu = np.array([int(x) for x in g["cu_seqlens"][0]])
    nh = int(g["n_heads"][0][0])
    hd = int(g["head_dim"][0][0])
    scale = float(g["scale"][0][0])
    qkv = np.array([[float(x) for x in r] for r in g["qkv_row"]])
    want = np.array([[float(x) for x in r] for r in g["out_row"]])
    got = oracle.varlen_causal_attention(qkv, cu, nh, hd, scale)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)
    got_dense = oracle.dense_masked_attention(qkv, cu, nh, hd, scale)
    np.testing.assert_allclose(got_dense, want, rtol=0, atol=1e-14)


def test_mask_golden():
    g = read_golden("mask_example.txt")
    cu = np.array([int(x) for x in g["cu_seqlens"][0]])
    want = np.array([[int(x) for x in r] for r in g["mask_row"]], dtype=bool)
    np.testing.assert_array_equal(oracle.block_diagonal_causal_mask(cu), want)


def test_worklist_golden():
    g = read_golden("worklist_example.txt")
    bm = int(g["tile_rows"][0][0])
    lengths = [int(x) for x in g["lengths"][0]]
    want = np.array([[int(a), int(b)] for a, b in g["item"]], dtype=np.int32)
    got = oracle.reference_worklist(workloads.cu_from_lengths(lengths), bm)
    np.testing.assert_array_equal(got, want)


# ------------------------------------------------------------ brute force ---

@pytest.mark.parametrize("lengths", [
    [1, 7, 16, 40],                      # the tiny configuration
    workloads.PLAN_TEST_LENGTHS,          # offsets [0, 10, 22, 37]
    [0, 5, 0, 0, 9, 1, 0],               # zero-length users anywhere
    [33],                                # one user
    [1, 1, 1, 1],                        # all length one
])
def test_per_user_matches_dense_mask_bruteforce(lengths):
    w = _rand_case(lengths, seed=len(lengths))
    qkv = _qkv64(w)
    a = oracle.varlen_causal_attention(qkv, w.cu_seqlens, H, D, w.scale)
    b = oracle.dense_masked_attention(qkv, w.cu_seqlens, H, D, w.scale)
    assert np.max(np.abs(a - b)) <= 1e-12


def test_tiny_config_matches_bruteforce():
    w = workloads.make_config(1)
    qkv = _qkv64(w)
    a = oracle.varlen_causal_attention(qkv, w.cu_seqlens, H, D, w.scale)
    b = oracle.dense_masked_attention(qkv, w.cu_seqlens, H, D, w.scale)
    assert np.max(np.abs(a - b)) <= 1e-12


# ---------------------------------------------------------- closed forms ---

def test_length_one_returns_own_v():
    w = _rand_case([1, 3, 1, 1, 2, 1], seed=3)
    qkv = _qkv64(w)
    out = oracle.varlen_causal_attention(qkv, w.cu_seqlens, H, D, w.scale)
    for u, L in enumerate(w.lengths):
        if L == 1:
            r = w.cu_seqlens[u]
            np.testing.assert_array_equal(out[r], qkv[r, 2 * H * D:3 * H * D])


def test_zero_query_gives_running_mean_of_v():
    w = _rand_case([5, 1, 12, 0, 7], seed=4)
    qkv = _qkv64(w).copy()
    qkv[:, :H * D] = 0.0
    out = oracle.varlen_causal_attention(qkv, w.cu_seqlens, H, D, w.scale)
    v = qkv[:, 2 * H * D:]
    for u in range(w.num_users):
        s, e = w.cu_seqlens[u], w.cu_seqlens[u + 1]
        for i in range(e - s):
            want = v[s:s + i + 1].sum(axis=0) / (i + 1)
            assert np.max(np.abs(out[s + i] - want)) <= 1e-12


def test_constant_v_returns_constant():
    w = _rand_case([4, 9, 1], seed=5)
    qkv = _qkv64(w).copy()
    c = np.linspace(-3.0, 3.0, H * D)
    qkv[:, 2 * H * D:] = c[None, :]
    out = oracle.varlen_causal_attention(qkv, w.cu_seqlens, H, D, w.scale)
    assert np.max(np.abs(out - c[None, :])) <= 1e-12


def test_two_key_row_closed_form():
    # Row 1 of a user: weights are sigmoid of the score difference.
    w = _rand_case([2], seed=6, n_heads=1)
    qkv = _qkv64(w)
    q1, k0, k1 = qkv[1, 0:64], qkv[0, 64:128], qkv[1, 64:128]
    v0, v1 = qkv[0, 128:192], qkv[1, 128:192]
    a = w.scale * (q1 @ k1 - q1 @ k0)
    s = 1.0 / (1.0 + np.exp(-a))
    want = v0 + s * (v1 - v0)
    out = oracle.varlen_causal_attention(qkv, w.cu_seqlens, 1, D, w.scale)
    assert np.max(np.abs(out[1] - want)) <= 1e-12


def test_huge_scores_stay_finite_and_pick_the_top_key():
    # Scores near +-2000: exp would overflow without the max shift; the softmax is
    # then one-hot on the largest score, so each row returns that key's v.
    qkv = np.zeros((3, 6))                          # one head, head_dim 2
    qkv[:, 0:2] = [[1, 0], [1, 0], [1, 0]]          # q
    qkv[:, 2:4] = [[-2000, 0], [2000, 0], [1000, 0]]  # k
    qkv[:, 4:6] = [[1, 2], [3, 4], [5, 6]]          # v
    out = oracle.varlen_causal_attention(qkv, [0, 3], 1, 2, 1.0)
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out, [[1, 2], [3, 4], [3, 4]], rtol=0, atol=1e-12)


# ---------------------------------------------------- library special case ---

@pytest.mark.parametrize("L", [1, 2, 17, 64, 130])
def test_single_user_matches_torch_causal_sdpa(L):
    w = _rand_case([L], seed=L)
    qkv = _qkv64(w)
    out = oracle.varlen_causal_attention(qkv, w.cu_seqlens, H, D, w.scale)
    t = torch.from_numpy(qkv)
    q = t[:, :H * D].reshape(L, H, D).transpose(0, 1).contiguous()
    k = t[:, H * D:2 * H * D].reshape(L, H, D).transpose(0, 1).contiguous()
    v = t[:, 2 * H * D:].reshape(L, H, D).transpose(0, 1).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=w.scale)
    ref = ref.transpose(0, 1).reshape(L, H * D).numpy()
    assert np.max(np.abs(out - ref)) <= 1e-12


# -------------------------------------------------------------- invariants ---

def test_isolation_perturbing_one_user_leaves_others_bit_identical():
    w = _rand_case([6, 20, 3, 11], seed=7)
    qkv = _qkv64(w)
    base = oracle.varlen_causal_attention(qkv, w.cu_seqlens, H, D, w.scale)
    s, e = w.cu_seqlens[1], w.cu_seqlens[2]
    qkv2 = qkv.copy()
    qkv2[s:e] = np.random.default_rng(1).standard_normal((e - s, qkv.shape[1]))
    pert = oracle.varlen_causal_attention(qkv2, w.cu_seqlens, H, D, w.scale)
    keep = np.ones(w.total_tokens, dtype=bool)
    keep[s:e] = False
    np.testing.assert_array_equal(base[keep], pert[keep])
    assert np.any(base[~keep] != pert[~keep])


def test_user_permutation_invariance():
    lengths = [6, 20, 3, 11]
    w = _rand_case(lengths, seed=8)
    qkv = _qkv64(w)
    out = oracle.varlen_causal_attention(qkv, w.cu_seqlens, H, D, w.scale)
    perm = [2, 0, 3, 1]
    rows = np.concatenate([np.arange(w.cu_seqlens[u], w.cu_seqlens[u + 1]) for u in perm])
    cu2 = workloads.cu_from_lengths([lengths[u] for u in perm])
    out2 = oracle.varlen_causal_attention(qkv[rows], cu2, H, D, w.scale)
    np.testing.assert_array_equal(out2, out[rows])


def test_future_keys_do_not_matter():
    # Changing rows after position i of a user leaves rows <= i unchanged.
    w = _rand_case([15], seed=9)
    qkv = _qkv64(w)
    base = oracle.varlen_causal_attention(qkv, w.cu_seqlens, H, D, w.scale)
    qkv2 = qkv.copy()
    qkv2[8:] += 1.0
    pert = oracle.varlen_causal_attention(qkv2, w.cu_seqlens, H, D, w.scale)
    np.testing.assert_array_equal(base[:8], pert[:8])
    assert np.any(base[8:] != pert[8:])


def test_scale_enters_as_multiplier_of_scores():
    # Doubling q and halving scale is the same problem.
    w = _rand_case([9, 4], seed=10)
    qkv = _qkv64(w)
    a = oracle.varlen_causal_attention(qkv, w.cu_seqlens, H, D, 0.125)
    qkv2 = qkv.copy()
    qkv2[:, :H * D] *= 2.0
    b = oracle.varlen_causal_attention(qkv2, w.cu_seqlens, H, D, 0.0625)
    assert np.max(np.abs(a - b)) <= 1e-12
    c = oracle.varlen_causal_attention(qkv, w.cu_seqlens, H, D, 0.0625)
    assert np.max(np.abs(a - c)) > 1e-3


def test_heads_are_independent_column_blocks():
    # Output head h depends only on q/k/v columns of head h.
    w = _rand_case([13, 5], seed=11)
    qkv = _qkv64(w)
    base = oracle.varlen_causal_attention(qkv, w.cu_seqlens, H, D, w.scale)
    qkv2 = qkv.copy()
    h = 3
    for part in range(3):
        c0 = part * H * D + h * D
        qkv2[:, c0:c0 + D] = -qkv2[:, c0:c0 + D] + 0.5
    pert = oracle.varlen_causal_attention(qkv2, w.cu_seqlens, H, D, w.scale)
    other = np.ones(H * D, dtype=bool)
    other[h * D:(h + 1) * D] = False
    np.testing.assert_array_equal(base[:, other], pert[:, other])
    assert np.any(base[:, ~other] != pert[:, ~other])


# ----------------------------------------------------------------- worklist ---

@pytest.mark.parametrize("seed", range(6))
def test_worklist_equals_sorted_pairs(seed):
    rng = np.random.default_rng(seed)
    lengths = rng.integers(0, 300, rng.integers(1, 40))
    cu = workloads.cu_from_lengths(lengths)
    got = oracle.reference_worklist(cu, 64)
    # Independent formulation: all (u, k) pairs, sorted by (-class, u, -k) with the
    # length class floor(log2(tiles)) taken from the bit length of the tile count.
    tiles = [-(-int(L) // 64) for L in lengths]
    pairs = [(u, k) for u, t in enumerate(tiles) for k in range(t)]
    pairs.sort(key=lambda p: (-(tiles[p[0]].bit_length() - 1), p[0], -p[1]))
    np.testing.assert_array_equal(got, np.array(pairs, dtype=np.int32).reshape(-1, 2))
    assert got.shape[0] == int(np.sum((lengths + 63) // 64))


def test_worklist_item_counts_of_configs():
    # Item counts at 64-row tiles for the five seed-0 configurations.
    want = {1: 4, 2: 136, 3: 886, 4: 640, 5: 2881}
    for i, n in want.items():
        w = workloads.make_config(i, with_values=False)
        assert oracle.reference_worklist(w.cu_seqlens, 64).shape[0] == n


def test_worklist_max_tiles_clamp():
    cu = workloads.cu_from_lengths([300, 10])
    got = oracle.reference_worklist(cu, 64, max_tiles=2)
    np.testing.assert_array_equal(got, [[0, 1], [0, 0], [1, 0]])


def test_worklist_length_classes():
    # Tiles 1, 2, 3, 4, 7, 8 -> classes 0, 1, 1, 2, 2, 3: user 5 first, then users
    # 3 and 4 (class 2, ascending), then 1 and 2, then 0; q-tiles descending.
    cu = workloads.cu_from_lengths([64, 128, 192, 256, 448, 512])
    got = oracle.reference_worklist(cu, 64)
    want = [(5, k) for k in range(7, -1, -1)] + [(3, k) for k in range(3, -1, -1)] + \
        [(4, k) for k in range(6, -1, -1)] + [(1, 1), (1, 0), (2, 2), (2, 1), (2, 0), (0, 0)]
    np.testing.assert_array_equal(got, np.array(want, dtype=np.int32))


def test_row_sampled_oracle_matches_full():
    w = _rand_case([3, 0, 70, 1, 129], seed=12)
    qkv = _qkv64(w)
    full = oracle.varlen_causal_attention(qkv, w.cu_seqlens, H, D, w.scale)
    rows = [0, 2, 3, 40, 72, 73, 74, 150, 201, 202]
    part = oracle.varlen_causal_attention_rows(qkv, w.cu_seqlens, rows, H, D, w.scale)
    assert np.max(np.abs(part - full[rows])) <= 1e-12
