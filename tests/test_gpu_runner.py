"""Bucketed graph runner (GPU): every bucket's graph replay equals the eager
forward bit for bit, with batches that fill their bucket partly and have fewer
users than the padded offsets hold; above the top bucket (or with too many
users) the runner falls back to the eager forward.  Buckets are the pages' ten
(2560 .. 7168 tokens in steps of 512) with 20 users per batch (cti2026 README,
CUDA Graph section)."""
import numpy as np
import pytest
import torch

import varlen_causal_attention_amd as vlca
import workloads
from gpu_util import say, to_gpu

pytestmark = pytest.mark.gpu


def batch(total, users, seed):
    """A packed batch of `users` lognormal lengths summing to `total` (the pages' length law)."""
    rng = np.random.default_rng(seed)
    cap = max(1024, total)  # one user may hold the whole batch
    raw = np.clip(np.round(rng.lognormal(mean=4.3, sigma=0.9, size=users)), 1, cap)
    lengths = workloads.rescale_to_sum(raw, total, cap)
    return workloads.make_from_lengths(list(lengths), seed=seed)


def eager(w, qkv, cu):
    out = vlca.fwd(qkv, cu, w.max_seqlen, scale=w.scale)
    torch.cuda.synchronize()
    return out


@pytest.fixture(scope="module")
def runner(gpu):
    r = vlca.GraphRunner(vlca.PAGES_BUCKETS, max_users=20, scale=0.125, precapture=True)
    assert r.captured() == len(vlca.PAGES_BUCKETS)
    yield r
    r.close()


def test_every_bucket_replay_matches_eager(runner):
    buckets = vlca.PAGES_BUCKETS
    for b, top in enumerate(buckets):
        lo = buckets[b - 1] if b else 1221  # the pages' smallest batch
        for k, (total, users) in enumerate([(top, 20), (lo + 1, 20), ((lo + top) // 2, 7), (lo + 3, 1)]):
            w = batch(total, users, seed=100 * b + k)
            qkv, cu = to_gpu(w)
            ref = eager(w, qkv, cu)
            out, used = runner.run(qkv, cu, w.total_tokens, w.max_seqlen)
            torch.cuda.synchronize()
            say(f"[case] bucket {top}: {w.total_tokens} tokens, {users} users -> bucket {used}")
            assert used == b
            assert torch.equal(out, ref), (top, total, users)


def test_replays_interleaved_across_buckets(runner):
    ws = [batch(t, 20, seed=7 + t) for t in (6900, 2600, 5000, 2600, 7168, 3100)]
    data = [to_gpu(w) for w in ws]
    refs = [eager(w, *d) for w, d in zip(ws, data)]
    say("[case] runner: six batches in a row on one stream, three buckets twice")
    outs = [runner.run(d[0], d[1], w.total_tokens, w.max_seqlen)[0] for w, d in zip(ws, data)]
    torch.cuda.synchronize()
    for o, r in zip(outs, refs):
        assert torch.equal(o, r)


def test_eager_fallback(runner):
    w = batch(9000, 20, seed=3)  # above the top bucket
    qkv, cu = to_gpu(w)
    ref = eager(w, qkv, cu)
    out, used = runner.run(qkv, cu, w.total_tokens, w.max_seqlen)
    torch.cuda.synchronize()
    assert used == -1 and torch.equal(out, ref)
    w = batch(3000, 25, seed=4)  # more users than the padded offsets hold
    qkv, cu = to_gpu(w)
    ref = eager(w, qkv, cu)
    out, used = runner.run(qkv, cu, w.total_tokens, w.max_seqlen)
    torch.cuda.synchronize()
    assert used == -1 and torch.equal(out, ref)


def test_static_buffers_no_copy(runner):
    """The producer writes straight into the runner's static qkv buffer and reads the
    result from its static out buffer."""
    w = batch(4321, 18, seed=5)
    qkv, cu = to_gpu(w)
    ref = eager(w, qkv, cu)
    T = w.total_tokens
    runner.qkv_static[:T].copy_(qkv)
    runner.out_static.fill_(0)
    out, used = runner.run(runner.qkv_static, cu, T, w.max_seqlen, out=runner.out_static)
    torch.cuda.synchronize()
    assert used == 4 and out.data_ptr() == runner.out_static.data_ptr()
    assert torch.equal(runner.out_static[:T], ref)
    assert bool((runner.out_static[T:] == 0).all())  # rows past the batch untouched


def test_lazy_capture(gpu):
    r = vlca.GraphRunner((1024, 2048, 4096), max_users=8, scale=0.125, precapture=False)
    try:
        assert r.captured() == 0
        w = batch(1500, 8, seed=6)
        qkv, cu = to_gpu(w)
        ref = eager(w, qkv, cu)
        for _ in range(2):
            out, used = r.run(qkv, cu, w.total_tokens, w.max_seqlen)
            torch.cuda.synchronize()
            assert used == 1 and torch.equal(out, ref)
        assert r.captured() == 1
    finally:
        r.close()
