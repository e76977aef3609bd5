"""fwd captured in a HIP graph (torch.cuda.CUDAGraph) and replayed, and fwd on
several streams at once.  Every replay, with eager work and synchronisations in
between, must reproduce the eager output bit for bit; so must every call on a
stream that runs at the same time as another.  Covers the single-kernel path
and the scheduler + worklist path, with the capture stream's library state
created before the capture (an eager call first) or during it (a fresh stream),
and a graph replayed after a larger eager call has replaced its stream's
worklist."""
import numpy as np
import pytest
import torch

import varlen_causal_attention_amd as vlca
import workloads
from gpu_util import say, to_gpu

pytestmark = pytest.mark.gpu


SPLIT_LENGTHS = [1000, 700, 3, 450, 0, 320]

GRAPH_CASES = [
    ("config 1", lambda: workloads.make_config(1)),
    ("config 2", lambda: workloads.make_config(2)),
    ("config 3", lambda: workloads.make_config(3)),
    # Long items split into key-range parts (the pool exists after the eager call),
    # on the single-kernel plan and, with a larger max_seqlen, on the scheduler plan.
    ("split items, single kernel", lambda: workloads.make_from_lengths(SPLIT_LENGTHS, seed=13)),
    ("split items, scheduler plan", lambda: workloads.make_from_lengths(SPLIT_LENGTHS, seed=13, max_seqlen=65536)),
]


@pytest.mark.parametrize("case", range(len(GRAPH_CASES)))
def test_graph_replay_matches_eager(gpu, case):
    name, make = GRAPH_CASES[case]
    w = make()
    single = vlca.single_kernel(w.num_users, w.max_seqlen, w.n_heads)
    say(f"[case] graph capture of fwd, {name} ({w.name}), single kernel: {single}")
    qkv, cu = to_gpu(w)
    s = torch.cuda.Stream()
    out = torch.zeros((w.total_tokens, 512), dtype=torch.bfloat16, device="cuda")
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # eager call on the capture stream (creates its workspace if any)
        vlca.fwd(qkv, cu, w.max_seqlen, scale=w.scale, out=out)
    s.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        vlca.fwd(qkv, cu, w.max_seqlen, scale=w.scale, out=out)
    torch.cuda.synchronize()
    for rep in range(4):
        out.zero_()                     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep} differs from the eager result"
    del g


@pytest.mark.parametrize("case", range(len(GRAPH_CASES)))
def test_graph_captured_on_fresh_stream_matches_eager(gpu, case):
    """No call on the capture stream before the capture: its worklist and split
    pool are created during the capture (outside the graph), and the split
    decision does not depend on that."""
    name, make = GRAPH_CASES[case]
    w = make()
    say(f"[case] graph capture on a fresh stream, {name} ({w.name})")
    qkv, cu = to_gpu(w)
    ref = vlca.fwd(qkv, cu, w.max_seqlen, scale=w.scale)  # eager, on the default stream
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    out = torch.zeros((w.total_tokens, 512), dtype=torch.bfloat16, device="cuda")
    g = torch.cuda.CUDAGraph()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        vlca.fwd(qkv, cu, w.max_seqlen, scale=w.scale, out=out)
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep} differs from the eager result"
        with torch.cuda.stream(s):  # eager call on the capture stream between replays
            again = vlca.fwd(qkv, cu, w.max_seqlen, scale=w.scale)
        torch.cuda.synchronize()
        assert torch.equal(again, ref)
    del g


def test_graph_replay_after_worklist_growth(gpu):
    """Capture a small scheduler-plan call, then run a much larger eager call on
    the same stream (its worklist is replaced by a larger one), then replay: the
    graph still uses the worklist it was captured with, which is kept."""
    small = workloads.make_from_lengths(list(np.random.default_rng(41).integers(1, 200, 300)), seed=41)
    big = workloads.make_config(5)
    assert not vlca.single_kernel(small.num_users, small.max_seqlen, 8)
    say("[case] graph replay after the capture stream's worklist grew")
    qs, cs = to_gpu(small)
    qb, cb = to_gpu(big)
    ref_small = vlca.fwd(qs, cs, small.max_seqlen, scale=small.scale)
    ref_big = vlca.fwd(qb, cb, big.max_seqlen, scale=big.scale)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    out = torch.zeros((small.total_tokens, 512), dtype=torch.bfloat16, device="cuda")
    g = torch.cuda.CUDAGraph()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        vlca.fwd(qs, cs, small.max_seqlen, scale=small.scale, out=out)
    torch.cuda.synchronize()
    for rep in range(3):
        with torch.cuda.stream(s):
            # 1000 users x 64 q-tiles: far more items than the captured worklist holds
            o_big = vlca.fwd(qb, cb, 262144 if rep == 2 else big.max_seqlen, scale=big.scale)
        torch.cuda.synchronize()
        assert torch.equal(o_big, ref_big)
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_small), f"replay {rep} after growth differs"
    del g


def test_single_kernel_plan(gpu):
    w2 = workloads.make_config(2, with_values=False)
    w3 = workloads.make_config(3, with_values=False)
    assert vlca.single_kernel(w2.num_users, w2.max_seqlen, 8)
    assert not vlca.single_kernel(w3.num_users, w3.max_seqlen, 8)
    assert not vlca.single_kernel(0, 64, 8)


def test_concurrent_streams_match_sequential(gpu):
    """Two streams run the scheduler plan at the same time, each many times over:
    each stream has its own worklist buffer and work counters, so every output
    equals the one computed alone."""
    wa = workloads.make_config(3)
    wb = workloads.make_from_lengths(list(range(1, 400)), seed=12)
    say(f"[case] concurrent fwd on two streams: {wa.name} and {wb.total_tokens} tokens over {wb.num_users} users")
    ga, gb = to_gpu(wa), to_gpu(wb)
    ref_a = vlca.fwd(ga[0], ga[1], wa.max_seqlen, scale=wa.scale)
    ref_b = vlca.fwd(gb[0], gb[1], wb.max_seqlen, scale=wb.scale)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    outs_a, outs_b = [], []
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    for _ in range(8):
        with torch.cuda.stream(sa):
            outs_a.append(vlca.fwd(ga[0], ga[1], wa.max_seqlen, scale=wa.scale))
        with torch.cuda.stream(sb):
            outs_b.append(vlca.fwd(gb[0], gb[1], wb.max_seqlen, scale=wb.scale))
    torch.cuda.synchronize()
    for o in outs_a:
        assert torch.equal(o, ref_a)
    for o in outs_b:
        assert torch.equal(o, ref_b)


def test_concurrent_streams_single_kernel_split(gpu):
    """The same on the single-kernel plan with long items split into key-range
    parts: each stream has its own pool of part states and arrival counters, and
    every call leaves the counters ready for the next."""
    wa = workloads.make_config(2)
    wb = workloads.make_from_lengths(SPLIT_LENGTHS, seed=13)
    for w in (wa, wb):
        assert vlca.single_kernel(w.num_users, w.max_seqlen, w.n_heads)
    say(f"[case] concurrent split single-kernel fwd on two streams: {wa.name} and lengths {list(wb.lengths)}")
    ga, gb = to_gpu(wa), to_gpu(wb)
    ref_a = vlca.fwd(ga[0], ga[1], wa.max_seqlen, scale=wa.scale)
    ref_b = vlca.fwd(gb[0], gb[1], wb.max_seqlen, scale=wb.scale)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    outs_a, outs_b = [], []
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    for _ in range(8):
        with torch.cuda.stream(sa):
            outs_a.append(vlca.fwd(ga[0], ga[1], wa.max_seqlen, scale=wa.scale))
        with torch.cuda.stream(sb):
            outs_b.append(vlca.fwd(gb[0], gb[1], wb.max_seqlen, scale=wb.scale))
    torch.cuda.synchronize()
    for o in outs_a:
        assert torch.equal(o, ref_a)
    for o in outs_b:
        assert torch.equal(o, ref_b)
