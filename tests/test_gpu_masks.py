"""HSTU-style mask variants (GPU, through varlen_causal_attn_fwd_masked) against
the fp64 oracle, every element, with the forward's bar (max |d| <= 2e-2, mean
|d| <= 2e-3): context prefixes, candidate groups, causal sliding windows,
non-causal windows and their combinations, ragged users (tile edges, users
shorter than their context or candidate counts), several head counts, and two
workload-sized batches."""
import numpy as np
import pytest
import torch

import oracle
import varlen_causal_attention_amd as vlca
import workloads
from gpu_util import assert_close, qkv64, say, to_gpu

pytestmark = pytest.mark.gpu

LENGTHS = [70, 3, 130, 64, 200, 1, 0, 129, 65]


def _counts(seed, hi):
    return list(np.random.default_rng(seed).integers(0, hi, len(LENGTHS)))


CASES = {
    "contexts": dict(c=[8, 5, 64, 0, 100, 1, 0, 129, 7]),
    "targets_group1": dict(g=[10, 1, 20, 0, 64, 1, 0, 3, 65]),
    "targets_group4_contexts": dict(c=[4, 0, 30, 10, 50, 0, 0, 0, 2], g=[12, 2, 40, 0, 100, 0, 0, 129, 8], group=4),
    "window_32": dict(window=(32, 0)),
    "window_100": dict(window=(100, 0)),
    "window_0": dict(window=(0, 0)),
    "window_1_contexts_targets": dict(c=[3, 1, 10, 5, 20, 0, 0, 64, 1], g=[5, 2, 7, 9, 70, 1, 0, 30, 64], group=3,
                                      window=(1, 0)),
    "hstu_window_64": dict(c=_counts(1, 20), g=_counts(2, 40), group=8, window=(64, 0)),
    "bidirectional": dict(window=(-1, -1)),
    "band_16_16": dict(window=(16, 16)),
    "lookahead_5": dict(window=(-1, 5)),
    "left_40_unbounded_right": dict(window=(40, -1)),
    "three_heads_contexts_window": dict(c=[8, 5, 64, 0, 100, 1, 0, 129, 7], window=(48, 0), n_heads=3),
    "sixteen_heads_targets": dict(g=[10, 1, 20, 0, 64, 1, 0, 3, 65], group=2, n_heads=16),
}


def _run(w, c=None, g=None, group=1, window=(-1, 0), max_seqlen=None):
    qkv, cu = to_gpu(w)
    ct = None if c is None else torch.tensor(c, dtype=torch.int32, device="cuda")
    tt = None if g is None else torch.tensor(g, dtype=torch.int32, device="cuda")
    out = vlca.fwd_masked(qkv, cu, w.max_seqlen if max_seqlen is None else max_seqlen, num_contexts=ct,
                          num_targets=tt, target_group_size=group, window=window, n_heads=w.n_heads, scale=w.scale)
    torch.cuda.synchronize()
    return out.cpu()


@pytest.mark.parametrize("name", sorted(CASES))
def test_mask_variants_all_elements(gpu, name):
    kw = dict(CASES[name])
    n_heads = kw.pop("n_heads", 8)
    w = workloads.make_from_lengths(LENGTHS, seed=31, n_heads=n_heads)
    say(f"[case] mask {name}: {kw}")
    out = _run(w, **kw)
    ref = oracle.varlen_attention_masked(qkv64(w), w.cu_seqlens, n_heads, 64, w.scale, num_contexts=kw.get("c"),
                                         num_targets=kw.get("g"), group=kw.get("group", 1),
                                         window=kw.get("window", (-1, 0)))
    assert_close(out, ref, name)


WORKLOAD_CASES = [
    # the pages' batch with HSTU-like users: up to 16 context tokens, up to 32 candidates
    # in groups of 8, a 256-token causal window
    (2, dict(c_hi=17, g_hi=33, group=8, window=(256, 0))),
    # the 44000-token batch with a 128-token sliding window
    (3, dict(window=(128, 0))),
]


@pytest.mark.parametrize("case", range(len(WORKLOAD_CASES)))
def test_mask_variants_workloads(gpu, case):
    idx, kw = WORKLOAD_CASES[case]
    w = workloads.make_config(idx)
    rng = np.random.default_rng(40 + idx)
    c = list(rng.integers(0, kw["c_hi"], w.num_users)) if "c_hi" in kw else None
    g = list(rng.integers(0, kw["g_hi"], w.num_users)) if "g_hi" in kw else None
    say(f"[case] mask on config {idx}: {kw}")
    out = _run(w, c=c, g=g, group=kw.get("group", 1), window=kw["window"])
    ref = oracle.varlen_attention_masked(qkv64(w), w.cu_seqlens, 8, 64, w.scale, num_contexts=c, num_targets=g,
                                         group=kw.get("group", 1), window=kw["window"])
    assert_close(out, ref, f"config {idx} {kw}")


def test_plain_causal_mask_is_the_forward(gpu):
    w = workloads.make_config(2)
    qkv, cu = to_gpu(w)
    ref = vlca.fwd(qkv, cu, w.max_seqlen, scale=w.scale)
    out = vlca.fwd_masked(qkv, cu, w.max_seqlen, window=(-1, 0), scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_masked_max_seqlen_and_zero_length_users(gpu):
    lengths = [70, 3, 130, 64, 200]
    c, g = [8, 1, 20, 0, 30], [4, 1, 9, 64, 50]
    w = workloads.make_from_lengths(lengths, seed=5)
    a = _run(w, c=c, g=g, group=2, window=(40, 0))
    b = _run(w, c=c, g=g, group=2, window=(40, 0), max_seqlen=65536)
    assert torch.equal(a, b)
    L2 = [0, 70, 3, 0, 130, 64, 0, 200]
    w2 = workloads.Workload("padded", np.asarray(L2), workloads.cu_from_lengths(L2), w.max_seqlen, w.scale)
    w2.qkv_bf16 = w.qkv_bf16
    d = _run(w2, c=[5, 8, 1, 3, 20, 0, 7, 30], g=[5, 4, 1, 3, 9, 64, 7, 50], group=2, window=(40, 0))
    assert torch.equal(a, d)


def test_bad_masks_raise(gpu):
    w = workloads.make_config(1)
    qkv, cu = to_gpu(w)
    ct = torch.zeros(w.num_users, dtype=torch.int32, device="cuda")
    for kw in (dict(target_group_size=0), dict(window=(-2, 0)), dict(num_contexts=ct, window=(4, 3))):
        with pytest.raises(vlca.VlcaError) as e:
            vlca.fwd_masked(qkv, cu, w.max_seqlen, **kw)
        assert e.value.code == -13


def test_masked_single_kernel_shared_ordering(gpu):
    """200 users (more than 64: the single-kernel plan orders them one user per
    thread and shares the descriptors), zero-length users among them, with
    contexts, candidate groups and a window, against the oracle; the scheduler
    plan (forced by a large max_seqlen) gives the same bits."""
    rng = np.random.default_rng(77)
    lengths = [int(x) for x in rng.integers(0, 150, 200)]
    w = workloads.make_from_lengths(lengths, seed=77)
    c = [int(x) for x in rng.integers(0, 20, 200)]
    g = [int(x) for x in rng.integers(0, 30, 200)]
    assert vlca.single_kernel(w.num_users, w.max_seqlen, w.n_heads)
    assert not vlca.single_kernel(w.num_users, 65536, w.n_heads)
    say(f"[case] masked, 200 users T={w.total_tokens}")
    out = _run(w, c=c, g=g, group=4, window=(48, 0))
    ref = oracle.varlen_attention_masked(qkv64(w), w.cu_seqlens, 8, 64, w.scale, num_contexts=c, num_targets=g,
                                         group=4, window=(48, 0))
    assert_close(out, ref, "masked, 200 users")
    out2 = _run(w, c=c, g=g, group=4, window=(48, 0), max_seqlen=65536)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
