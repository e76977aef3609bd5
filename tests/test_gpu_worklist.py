"""The GPU segment scheduler's worklist equals the reference order bit for bit (GPU)."""
import numpy as np
import pytest
import torch

import oracle
import varlen_causal_attention_amd as vlca
import workloads
from gpu_util import say

pytestmark = pytest.mark.gpu


def gpu_worklist(cu_np, max_seqlen):
    cu = torch.from_numpy(np.asarray(cu_np, dtype=np.int32)).cuda()
    items, count = vlca.build_worklist(cu, max_seqlen)
    torch.cuda.synchronize()
    return items.cpu().numpy(), int(count.cpu()[0])


def check(cu_np, max_seqlen, label):
    items, n = gpu_worklist(cu_np, max_seqlen)
    max_tiles = -(-max_seqlen // 64)
    ref = oracle.reference_worklist(cu_np, 64, max_tiles=max_tiles)
    say(f"[worklist] {label}: {n} items")
    assert n == ref.shape[0]
    np.testing.assert_array_equal(items[:n, :2], ref)
    cu = np.asarray(cu_np, dtype=np.int64)
    np.testing.assert_array_equal(items[:n, 2], cu[ref[:, 0]])
    np.testing.assert_array_equal(items[:n, 3], cu[ref[:, 0] + 1] - cu[ref[:, 0]])


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_configs(gpu, idx):
    w = workloads.make_config(idx, with_values=False)
    check(w.cu_seqlens, w.max_seqlen, w.name)


@pytest.mark.parametrize("seed", range(8))
def test_random_with_zero_length_users(gpu, seed):
    rng = np.random.default_rng(100 + seed)
    U = int(rng.integers(1, 3000))
    L = rng.integers(0, 700, U)
    L[rng.random(U) < 0.2] = 0
    check(workloads.cu_from_lengths(L), int(max(L.max(), 1)), f"random seed {seed} U={U}")


def test_many_users_beyond_lds_cache(gpu):
    rng = np.random.default_rng(7)
    L = rng.integers(0, 200, 20000)
    check(workloads.cu_from_lengths(L), 200, "U=20000")


def test_clamped_to_max_seqlen(gpu):
    # A user longer than max_seqlen (a precondition violation) is clamped, never overrun.
    check(workloads.cu_from_lengths([300, 10, 129]), 128, "clamp")


def test_empty_and_all_zero(gpu):
    items, n = gpu_worklist([0], 64)
    assert n == 0 and items.shape[0] == 0
    check(workloads.cu_from_lengths([0, 0, 0]), 64, "all zero")


def test_long_levels(gpu):
    check(workloads.cu_from_lengths([262144, 1, 70000]), 262144, "4096 levels")
