"""Helpers shared by the GPU test modules (not collected by pytest)."""
import sys

import numpy as np
import torch

import varlen_causal_attention_amd as vlca

# Acceptance bound against the fp64 oracle for the bf16 output (max and mean
# absolute difference over every compared element).
TOL_MAX = 2e-2
TOL_MEAN = 2e-3


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def to_gpu(w):
    return w.qkv_bf16.cuda(), torch.from_numpy(np.asarray(w.cu_seqlens, dtype=np.int32)).cuda()


def run_fwd(w, max_seqlen=None, qkv=None, cu=None):
    if qkv is None:
        qkv, cu = to_gpu(w)
    out = vlca.fwd(qkv, cu, w.max_seqlen if max_seqlen is None else max_seqlen, n_heads=w.n_heads,
                   head_dim=w.head_dim, scale=w.scale)
    torch.cuda.synchronize()
    return out.cpu()


def qkv64(w):
    return w.qkv_bf16.to(torch.float64).numpy()


def deltas(out_bf16, ref):
    d = np.abs(out_bf16.to(torch.float64).numpy() - ref)
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0


def assert_close(out_bf16, ref, label=""):
    mx, mn = deltas(out_bf16, ref)
    say(f"[parity] {label}: max|d|={mx:.3e} mean|d|={mn:.3e}")
    assert np.all(np.isfinite(out_bf16.float().numpy())), label
    assert mx <= TOL_MAX and mn <= TOL_MEAN, (label, mx, mn)
    return mx, mn
