"""fwd captured in a HIP graph (torch.cuda.CUDAGraph) and replayed: every replay,
with eager work and synchronisations in between, must reproduce the eager
output bit for bit.  Covers the single-kernel path (no worklist buffer) and the
scheduler + worklist path (its buffer exists before capture)."""
import pytest
import torch

import varlen_causal_attention_amd as vlca
import workloads
from gpu_util import say, to_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("idx", [1, 2, 3])
def test_graph_replay_matches_eager(gpu, idx):
    w = workloads.make_config(idx)
    single = vlca.single_kernel(w.num_users, w.max_seqlen, w.n_heads)
    say(f"[case] graph capture of fwd, config {idx} ({w.name}), single kernel: {single}")
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


def test_single_kernel_plan(gpu):
    w2 = workloads.make_config(2, with_values=False)
    w3 = workloads.make_config(3, with_values=False)
    assert vlca.single_kernel(w2.num_users, w2.max_seqlen, 8)
    assert not vlca.single_kernel(w3.num_users, w3.max_seqlen, 8)
    assert not vlca.single_kernel(0, 64, 8)
