"""The seeded generators: determinism and the recipe's stated properties (CPU only)."""
import numpy as np
import pytest
import torch

import workloads


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_lengths_deterministic_and_bounded(idx):
    a = workloads.make_config(idx, with_values=False)
    b = workloads.make_config(idx, with_values=False)
    np.testing.assert_array_equal(a.lengths, b.lengths)
    assert a.cu_seqlens[0] == 0 and np.all(np.diff(a.cu_seqlens) == a.lengths)
    assert a.lengths.min() >= 1
    assert a.lengths.max() <= a.max_seqlen


def test_config_sizes():
    tot = {1: 64, 2: 6823, 3: 44000, 5: 131072}
    users = {1: 4, 2: 60, 3: 390, 4: 513, 5: 1000}
    caps = {2: 1024, 3: 2048, 5: 4096}
    for i in range(1, 6):
        w = workloads.make_config(i, with_values=False)
        assert w.num_users == users[i]
        if i in tot:
            assert w.total_tokens == tot[i]
        if i in caps:
            assert w.lengths.max() <= caps[i]
    w1 = workloads.make_config(1, with_values=False)
    np.testing.assert_array_equal(w1.cu_seqlens, [0, 1, 8, 24, 64])
    w4 = workloads.make_config(4, with_values=False)
    assert w4.lengths[0] == 8192 and w4.lengths[1:].min() >= 1 and w4.lengths[1:].max() <= 64
    assert workloads.make_config(5, with_values=False).max_seqlen == 4096


def test_seed0_draw_statistics():
    # Regression pins of the recipe at seed 0 (min / median / max, ones).
    w2 = workloads.make_config(2, with_values=False)
    assert (w2.lengths.min(), w2.lengths.max()) == (9, 452)
    w3 = workloads.make_config(3, with_values=False)
    assert (w3.lengths.min(), w3.lengths.max()) == (2, 1233)
    w4 = workloads.make_config(4, with_values=False)
    assert w4.total_tokens == 25523
    w5 = workloads.make_config(5, with_values=False)
    assert w5.lengths.max() == 1315 and int((w5.lengths == 1).sum()) == 455


def test_rescale_exact_sum_and_caps():
    rng = np.random.default_rng(3)
    raw = rng.lognormal(4.3, 0.9, 50)
    L = workloads.rescale_to_sum(raw, 3000, 200)
    assert L.sum() == 3000 and L.min() >= 1 and L.max() <= 200
    L = workloads.rescale_to_sum(np.ones(10), 10, 5)
    np.testing.assert_array_equal(L, np.ones(10))


def test_values_are_bf16_rounded_normals():
    w = workloads.make_config(1)
    assert w.qkv_bf16.dtype == torch.bfloat16 and tuple(w.qkv_bf16.shape) == (64, 1536)
    again = workloads.make_config(1)
    assert torch.equal(w.qkv_bf16, again.qkv_bf16)
    x = w.qkv_bf16.float()
    assert abs(float(x.mean())) < 0.05 and 0.9 < float(x.std()) < 1.1
    w4 = workloads.make_config(4)
    assert 0.45 < float(w4.qkv_bf16.float().std()) < 0.55


def test_flop_and_byte_counts():
    w = workloads.make_config(1, with_values=False)
    # sum L(L+1)/2 = 1 + 28 + 136 + 820 = 985; times 4*8*64
    assert w.causal_flops() == 985 * 4 * 8 * 64
    assert w.algorithmic_bytes() == 64 * 4096
