"""Training path (GPU, through the C ABI): varlen_causal_attn_fwd_lse and
varlen_causal_attn_bwd against the fp64 oracle, element by element.

Tolerance.  bf16 has 8 significant bits: its unit roundoff is u = 2^-8.  The
backward's inputs are bf16 and exact; its intermediate quantities carry
relative errors of a few u -- P from the log-sum-exp (<= u, below) and rounded to
bf16 for the dV MFMA (u), D from the bf16-rounded forward output (u), dS rounded
to bf16 (u) -- accumulated in fp32, and the gradients are rounded to bf16 (u of
the result).  Perturbing every term of a gradient's expansion by a relative
error <= e changes it by at most e times the expansion taken in absolute values
(oracle.varlen_causal_attention_backward_magnitude); inside dS = P (dP - D) the
two terms cancel, so that magnitude can far exceed the gradient.  The bar is the
forward's (max |d| <= 2e-2 for outputs of order one, in units of the element's
magnitude once it passes 1) plus that bound with e = 4u:
    |d| <= 2e-2 max(1, |ref|) + 4u * magnitude      for every element,
and, for N(0,1) inputs (the workloads' values, for which the forward's mean bar
is stated), mean |d| <= 2e-3 s per block (dq, dk, dv), s = max(1, rms(reference
block)), which any systematic error (a missed mask, a wrong scale) exceeds.
Inputs scaled by c scale the cancelling terms by up to c^2: there only the
per-element bound, which scales with them, is checked.  The
log-sum-exp sums bf16-rounded weights (relative error <= u, so <= u in the log)
in fp32 over at most 8192 keys: |d lse| <= 2^-8 + 8192 * 2^-24.
"""
import numpy as np
import pytest
import torch

import oracle
import varlen_causal_attention_amd as vlca
import workloads
from gpu_util import qkv64, say, to_gpu

pytestmark = pytest.mark.gpu

LSE_TOL = 2.0 ** -8 + 8192 * 2.0 ** -24


def run_train(w, dout, max_seqlen=None):
    qkv, cu = to_gpu(w)
    ms = w.max_seqlen if max_seqlen is None else max_seqlen
    out, lse = vlca.fwd_lse(qkv, cu, ms, n_heads=w.n_heads, scale=w.scale)
    dqkv = vlca.bwd(qkv, out, dout.cuda(), lse, cu, ms, n_heads=w.n_heads, scale=w.scale)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), dqkv.cpu()


U_BF16 = 2.0 ** -8


def assert_grads_close(dqkv, ref, mag, n_heads, label, check_mean=True):
    hd = n_heads * 64
    g = dqkv.to(torch.float64).numpy()
    assert np.all(np.isfinite(g)), label
    for blk, name in enumerate(("dq", "dk", "dv")):
        a, r, m = (x[:, blk * hd:(blk + 1) * hd] for x in (g, ref, mag))
        if not r.size:
            continue
        sc = max(1.0, float(np.sqrt(np.mean(r * r))))
        d = np.abs(a - r)
        bar = 2e-2 * np.maximum(1.0, np.abs(r)) + 4 * U_BF16 * m
        i = int(np.argmax(d / bar))
        mn = float(d.mean())
        say(f"[parity] {label} {name}: max|d|/bar={float(d.flat[i] / bar.flat[i]):.3f} (|d| {d.flat[i]:.3e}, "
            f"|ref| {abs(r.flat[i]):.3f}, magnitude {m.flat[i]:.2f}) max|d|={float(d.max()):.3e} "
            f"mean|d|={mn:.3e} (rms scale {sc:.3f})")
        assert d.flat[i] <= bar.flat[i], (label, name, float(d.flat[i]), float(bar.flat[i]))
        assert mn <= 2e-3 * sc or not check_mean, (label, name, mn, sc)


def oracle_grads(w, q, dout):
    d = dout.double().numpy()
    return (oracle.varlen_causal_attention_backward(q, w.cu_seqlens, d, w.n_heads, 64, w.scale),
            oracle.varlen_causal_attention_backward_magnitude(q, w.cu_seqlens, d, w.n_heads, 64, w.scale))


CASES = {
    "tiny_1_7_16_40": dict(lengths=[1, 7, 16, 40]),
    "tile_edges": dict(lengths=[63, 64, 65, 127, 128, 129, 1, 2]),
    "zero_length_users": dict(lengths=[0, 5, 0, 0, 9, 1, 0, 200, 0]),
    "single_user_1000": dict(lengths=[1000]),
    "one_head": dict(lengths=[70, 3, 130], n_heads=1),
    "three_heads": dict(lengths=[70, 3, 130, 64], n_heads=3),
    "sixteen_heads": dict(lengths=[33, 190], n_heads=16),
    "scaled_values_x2": dict(lengths=[300, 17], value_scale=2.0),
    "300_users": dict(lengths=list(np.random.default_rng(5).integers(0, 150, 300))),
    # Users whose rows end at each of the 64 positions of their diagonal tile, in
    # one-tile and two-tile users (every wave's diagonal step, dQ and dK/dV).
    "diag_every_residue": dict(lengths=list(range(1, 129)), n_heads=1),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_backward_small_cases(gpu, name):
    kw = CASES[name]
    w = workloads.make_from_lengths(kw["lengths"], seed=23, n_heads=kw.get("n_heads", 8),
                                    value_scale=kw.get("value_scale", 1.0))
    dout = workloads.draw_dout(w.total_tokens, w.n_heads, seed=24)
    say(f"[case] backward {name}")
    out, lse, dqkv = run_train(w, dout)
    q = qkv64(w)
    assert torch.equal(out, vlca.fwd(*to_gpu(w), w.max_seqlen, n_heads=w.n_heads, scale=w.scale).cpu())
    ref_lse = oracle.varlen_causal_attention_lse(q, w.cu_seqlens, w.n_heads, 64, w.scale)
    assert float(np.max(np.abs(lse.double().numpy() - ref_lse))) <= LSE_TOL
    ref, mag = oracle_grads(w, q, dout)
    assert_grads_close(dqkv, ref, mag, w.n_heads, name, check_mean=kw.get("value_scale", 1.0) == 1.0)


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_backward_configs_all_elements(gpu, idx):
    w = workloads.make_config(idx)
    dout = workloads.draw_dout(w.total_tokens, seed=idx)
    say(f"[case] backward config {idx} {w.name} T={w.total_tokens}")
    out, lse, dqkv = run_train(w, dout)
    q = qkv64(w)
    ref_lse = oracle.varlen_causal_attention_lse(q, w.cu_seqlens, 8, 64, w.scale)
    assert float(np.max(np.abs(lse.double().numpy() - ref_lse))) <= LSE_TOL
    ref, mag = oracle_grads(w, q, dout)
    assert_grads_close(dqkv, ref, mag, 8, w.name)
    # length-one users: dV is dO exactly (P = 1), dQ and dK vanish up to rounding
    ones = w.cu_seqlens[:-1][w.lengths == 1]
    if ones.size:
        assert torch.equal(dqkv[ones, 1024:], dout[ones])
        assert float(dqkv[ones, :1024].abs().max()) <= 1e-3


def test_backward_deterministic_and_invariant(gpu):
    w = workloads.make_from_lengths([1000, 700, 3, 450, 0, 320], seed=13)
    dout = workloads.draw_dout(w.total_tokens, seed=13)
    say("[case] backward: run twice, max_seqlen and zero-length users")
    _, _, a = run_train(w, dout)
    _, _, b = run_train(w, dout)
    assert torch.equal(a, b)
    _, _, c = run_train(w, dout, max_seqlen=65536)
    assert torch.equal(a, c)
    L2 = [0, 0, 1000, 0, 700, 3, 450, 0, 320, 0]
    w2 = workloads.Workload("padded", np.asarray(L2), workloads.cu_from_lengths(L2), w.max_seqlen, w.scale)
    w2.qkv_bf16 = w.qkv_bf16
    _, _, d = run_train(w2, dout)
    assert torch.equal(a, d)


def test_backward_rows_past_the_last_user_untouched(gpu):
    w = workloads.make_from_lengths([37, 3, 130], seed=17)
    pad = 50
    qkv = torch.cat([w.qkv_bf16, torch.ones((pad, 1536), dtype=torch.bfloat16)]).cuda()
    cu = torch.from_numpy(np.asarray(w.cu_seqlens, dtype=np.int32)).cuda()
    out, lse = vlca.fwd_lse(qkv, cu, w.max_seqlen, scale=w.scale)
    dout = torch.cat([workloads.draw_dout(w.total_tokens, seed=3), torch.ones((pad, 512), dtype=torch.bfloat16)]).cuda()
    dqkv = torch.full_like(qkv, 5.0)
    vlca.bwd(qkv, out, dout, lse, cu, w.max_seqlen, scale=w.scale, dqkv=dqkv)
    torch.cuda.synchronize()
    assert bool((dqkv[w.total_tokens:] == 5.0).all())


def test_autograd_wrapper(gpu):
    w = workloads.make_from_lengths([90, 1, 200, 33], seed=29)
    dout = workloads.draw_dout(w.total_tokens, seed=30).cuda()
    qkv, cu = to_gpu(w)
    x = qkv.clone().requires_grad_(True)
    y = vlca.attention(x, cu, w.max_seqlen, scale=w.scale)
    y.backward(dout)
    torch.cuda.synchronize()
    out, lse = vlca.fwd_lse(qkv, cu, w.max_seqlen, scale=w.scale)
    ref = vlca.bwd(qkv, out, dout, lse, cu, w.max_seqlen, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(y.detach(), out) and torch.equal(x.grad, ref)
