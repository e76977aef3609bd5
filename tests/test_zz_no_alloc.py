"""varlen_causal_attn_fwd_noalloc against varlen_causal_attn_fwd (GPU), through the C ABI.

The no-allocation entry point runs the same launch plan and split decision as
fwd over a fixed per-device scratch array instead of the stream's state, so its
output must equal fwd's bit for bit.  Each case makes two calls in a row, the
second on a smaller batch, so the second runs over what the first left in the
scratch array.
"""
import numpy as np
import pytest
import torch

import varlen_causal_attention_amd as vlca
import workloads
from gpu_util import say, to_gpu

pytestmark = pytest.mark.gpu


def _batch(kind):
    if kind == "config 3":
        return workloads.make_config(3)
    if kind == "config 2":
        return workloads.make_config(2)
    if kind == "config 1":
        return workloads.make_config(1)
    if kind == "split batch":
        return workloads.make_from_lengths([1000, 700, 3, 450, 0, 320], seed=13)
    if kind == "small split batch":
        return workloads.make_from_lengths([640, 5, 330], seed=14)
    if kind == "split batch, scheduler plan":
        return workloads.make_from_lengths([1000, 700, 3, 450, 0, 320], seed=13, max_seqlen=65536)
    if kind == "300 short users":
        return workloads.make_from_lengths(list(np.random.default_rng(41).integers(1, 9, 300)), seed=41)
    raise ValueError(kind)


# (first call, second call on a smaller batch)
PAIRS = [
    ("config 3", "config 1"),                       # scheduler plan, then single kernel
    ("split batch, scheduler plan", "300 short users"),  # split units in the scratch worklist, then whole items
    ("split batch", "small split batch"),           # split pool reused by the second call
    ("config 2", "config 1"),
]


def _noalloc(w, qkv, cu):
    out = torch.full((w.total_tokens, w.n_heads * w.head_dim), 3.0, dtype=torch.bfloat16, device="cuda")
    vlca.fwd_noalloc(qkv, cu, w.max_seqlen, out, n_heads=w.n_heads, head_dim=w.head_dim, scale=w.scale)
    return out


@pytest.mark.parametrize("case", range(len(PAIRS)))
def test_noalloc_matches_fwd_two_calls(gpu, case):
    first, second = PAIRS[case]
    wa, wb = _batch(first), _batch(second)
    assert wb.total_tokens < wa.total_tokens
    say(f"[case] fwd_noalloc vs fwd: {first} ({wa.total_tokens} rows), then {second} ({wb.total_tokens} rows)")
    ga, gb = to_gpu(wa), to_gpu(wb)
    ref_a = vlca.fwd(ga[0], ga[1], wa.max_seqlen, scale=wa.scale)
    ref_b = vlca.fwd(gb[0], gb[1], wb.max_seqlen, scale=wb.scale)
    torch.cuda.synchronize()
    out_a = _noalloc(wa, *ga)
    out_b = _noalloc(wb, *gb)
    torch.cuda.synchronize()
    assert torch.equal(out_a, ref_a), f"{first}: fwd_noalloc differs from fwd"
    assert torch.equal(out_b, ref_b), f"{second}: fwd_noalloc differs from fwd"


def test_noalloc_refuses_too_large_worklist(gpu):
    # 8193 users x 64 q-tiles > 524288 scratch items: refused on the host, nothing launched.
    lengths = [1] * 8193
    w = workloads.make_from_lengths(lengths, seed=1)
    qkv, cu = to_gpu(w)
    out = torch.zeros((w.total_tokens, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(vlca.VlcaError) as e:
        vlca.fwd_noalloc(qkv, cu, 4096, out, scale=w.scale)
    assert e.value.code == -11
    torch.cuda.synchronize()
    assert bool((out == 0).all())
    # the same batch with a bound that fits runs, and equals fwd
    ref = vlca.fwd(qkv, cu, 64, scale=w.scale)
    vlca.fwd_noalloc(qkv, cu, 64, out, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_noalloc_in_graph_replays(gpu):
    """Captured into a graph (the no-allocation entry point's main caller), replayed
    with eager calls of the same entry point on a smaller batch in between."""
    w, ws = _batch("split batch"), _batch("config 1")
    say("[case] fwd_noalloc captured in a graph, replays interleaved with eager calls")
    qkv, cu = to_gpu(w)
    qs, cs = to_gpu(ws)
    ref = vlca.fwd(qkv, cu, w.max_seqlen, scale=w.scale)
    ref_s = vlca.fwd(qs, cs, ws.max_seqlen, scale=ws.scale)
    out = torch.zeros((w.total_tokens, 512), dtype=torch.bfloat16, device="cuda")
    out_s = torch.zeros((ws.total_tokens, 512), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        vlca.fwd_noalloc(qkv, cu, w.max_seqlen, out, scale=w.scale)
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep}"
        vlca.fwd_noalloc(qs, cs, ws.max_seqlen, out_s, scale=ws.scale)
        torch.cuda.synchronize()
        assert torch.equal(out_s, ref_s)
    del g
