"""The attention's neighbours (GPU, through the C ABI) against the fp64 layer
oracle: qkv = LayerNorm(x) W_qkv^T + b (LayerNorm fused into the product) and
y = residual + attn W_out^T + b (bias and residual fused into its epilogue),
every element, and the whole attention sub-block.

Tolerance.  u = 2^-8 (bf16).  Each output is one dot product over 512 terms in
fp32 whose inputs carry at most one bf16 rounding (LayerNorm's output is rounded
to bf16 before the product; attn and the weights are exact bf16), then rounded
to bf16.  A dot product whose terms carry relative errors <= e is off by <= e
times the sum of their absolute values, M = |A| |W|^T (+ |b| + |residual|).  Bar
per element: |d| <= 2e-2 max(1, |ref|) + 4u M; per tensor: mean |d| <= 2e-3 s,
s = max(1, rms(ref)).  For the whole sub-block the attention output itself
carries the forward's error, which the output product sums over 512 columns:
there the bar adds sum_k |W_out[n, k]| times the forward's mean bar (2e-3).
"""
import numpy as np
import pytest
import torch

import oracle
import varlen_causal_attention_amd as vlca
import workloads
from gpu_util import say

pytestmark = pytest.mark.gpu

U = 2.0 ** -8


def _close(out, ref, mag, label, extra=0.0):
    d = np.abs(out.to(torch.float64).numpy() - ref)
    bar = 2e-2 * np.maximum(1.0, np.abs(ref)) + 4 * U * mag + extra
    i = int(np.argmax(d / bar))
    sc = max(1.0, float(np.sqrt(np.mean(ref * ref))))
    say(f"[parity] {label}: max|d|/bar={float(d.flat[i] / bar.flat[i]):.3f} max|d|={float(d.max()):.3e} "
        f"mean|d|={float(d.mean()):.3e} (rms scale {sc:.3f})")
    assert d.flat[i] <= bar.flat[i], (label, float(d.flat[i]), float(bar.flat[i]))
    assert float(d.mean()) <= 2e-3 * sc, (label, float(d.mean()), sc)


def _gpu(p):
    return {k: getattr(p, k).cuda() for k in ("gamma", "beta", "w_qkv", "b_qkv", "w_out", "b_out")}


@pytest.mark.parametrize("T", [1, 63, 64, 65, 200, 6823, 44000])
def test_ln_qkv(gpu, T):
    p = workloads.make_layer_params()
    x = workloads.draw_layer_input(T, seed=T)
    g = _gpu(p)
    say(f"[case] ln_qkv T={T}")
    out = vlca.ln_qkv(x.cuda(), g["gamma"], g["beta"], g["w_qkv"], g["b_qkv"], eps=p.eps)
    torch.cuda.synchronize()
    f = lambda t: t.to(torch.float64).numpy()  # noqa: E731
    ln = oracle.layer_norm(f(x), f(p.gamma), f(p.beta), p.eps)
    ref = oracle.linear(ln, f(p.w_qkv), f(p.b_qkv))
    mag = np.abs(ln) @ np.abs(f(p.w_qkv)).T + np.abs(f(p.b_qkv))
    _close(out.cpu(), ref, mag, f"ln_qkv T={T}")


@pytest.mark.parametrize("T,heads,offset", [(300, 2, 0.0), (1000, 10, 0.0), (129, 8, 40.0), (6823, 8, -300.0)])
def test_ln_qkv_shapes_and_offsets(gpu, T, heads, offset):
    """Output widths of 3 and 15 column chunks (grids whose groups hold different
    chunk counts), and rows whose mean dominates their spread (every third row
    shifted by `offset`: the variance is then taken as the mean square
    deviation)."""
    p = workloads.make_layer_params(n_heads=heads)
    x = workloads.draw_layer_input(T, seed=T + heads)
    if offset:
        xf = x.float()
        xf[::3] += offset
        x = xf.to(torch.bfloat16)
    g = _gpu(p)
    say(f"[case] ln_qkv T={T} n_out={3 * heads * 64} offset={offset}")
    out = vlca.ln_qkv(x.cuda(), g["gamma"], g["beta"], g["w_qkv"], g["b_qkv"], eps=p.eps)
    torch.cuda.synchronize()
    assert out.shape == (T, 3 * heads * 64)
    f = lambda t: t.to(torch.float64).numpy()  # noqa: E731
    ln = oracle.layer_norm(f(x), f(p.gamma), f(p.beta), p.eps)
    ref = oracle.linear(ln, f(p.w_qkv), f(p.b_qkv))
    mag = np.abs(ln) @ np.abs(f(p.w_qkv)).T + np.abs(f(p.b_qkv))
    _close(out.cpu(), ref, mag, f"ln_qkv T={T} n_out={3 * heads * 64} offset={offset}")


def test_ln_qkv_wide_sampled(gpu):
    """A 4096-column output over 44000 rows: the grid-fill model then gives each
    workgroup its longest run (16 chunks, the bound of its bias slice).  Every
    element of 1500 sampled rows, the first and the last rows is checked."""
    T, n_out = 44000, 4096
    p = workloads.make_layer_params()
    rng = np.random.default_rng(11)
    w = torch.from_numpy((rng.standard_normal((n_out, 512)) / np.sqrt(512)).astype(np.float32)).to(torch.bfloat16)
    b = torch.from_numpy((0.1 * rng.standard_normal(n_out)).astype(np.float32)).to(torch.bfloat16)
    x = workloads.draw_layer_input(T, seed=12)
    say(f"[case] ln_qkv T={T} n_out={n_out} (sampled rows)")
    out = vlca.ln_qkv(x.cuda(), p.gamma.cuda(), p.beta.cuda(), w.cuda(), b.cuda(), eps=p.eps)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([rng.choice(T, 1500, replace=False), [0, 1, T - 2, T - 1]]))
    f = lambda t: t.to(torch.float64).numpy()  # noqa: E731
    xs = f(x)[rows]
    ln = oracle.layer_norm(xs, f(p.gamma), f(p.beta), p.eps)
    ref = oracle.linear(ln, f(w), f(b))
    mag = np.abs(ln) @ np.abs(f(w)).T + np.abs(f(b))
    _close(out.cpu()[torch.from_numpy(rows)], ref, mag, f"ln_qkv T={T} n_out={n_out} sampled")


@pytest.mark.parametrize("T", [1, 65, 6823, 44000])
def test_out_residual(gpu, T):
    p = workloads.make_layer_params()
    attn = workloads.draw_layer_input(T, seed=100 + T)
    res = workloads.draw_layer_input(T, seed=200 + T)
    g = _gpu(p)
    say(f"[case] out_residual T={T}")
    y = vlca.out_residual(attn.cuda(), g["w_out"], g["b_out"], res.cuda())
    torch.cuda.synchronize()
    f = lambda t: t.to(torch.float64).numpy()  # noqa: E731
    ref = f(res) + oracle.linear(f(attn), f(p.w_out), f(p.b_out))
    mag = np.abs(f(attn)) @ np.abs(f(p.w_out)).T + np.abs(f(p.b_out)) + np.abs(f(res))
    _close(y.cpu(), ref, mag, f"out_residual T={T}")
    # in place on the residual
    r2 = res.cuda()
    vlca.out_residual(attn.cuda(), g["w_out"], g["b_out"], r2, out=r2)
    torch.cuda.synchronize()
    assert torch.equal(r2.cpu(), y.cpu())


@pytest.mark.parametrize("idx", [1, 2, 3])
def test_attention_block(gpu, idx):
    w = workloads.make_config(idx, with_values=False)
    p = workloads.make_layer_params()
    x = workloads.draw_layer_input(w.total_tokens, seed=idx)
    g = _gpu(p)
    cu = torch.from_numpy(np.asarray(w.cu_seqlens, dtype=np.int32)).cuda()
    say(f"[case] attention sub-block on config {idx}")
    y = vlca.attention_block(x.cuda(), cu, w.max_seqlen, g["gamma"], g["beta"], g["w_qkv"], g["b_qkv"], g["w_out"],
                             g["b_out"], eps=p.eps, scale=w.scale)
    torch.cuda.synchronize()
    f = lambda t: t.to(torch.float64).numpy()  # noqa: E731
    ref = oracle.attention_block(f(x), w.cu_seqlens, 8, 64, w.scale, f(p.gamma), f(p.beta), p.eps, f(p.w_qkv),
                                 f(p.b_qkv), f(p.w_out), f(p.b_out))
    qkv = oracle.linear(oracle.layer_norm(f(x), f(p.gamma), f(p.beta), p.eps), f(p.w_qkv), f(p.b_qkv))
    attn = oracle.varlen_causal_attention(qkv, w.cu_seqlens, 8, 64, w.scale)
    mag = np.abs(attn) @ np.abs(f(p.w_out)).T + np.abs(f(p.b_out)) + np.abs(f(x))
    extra = 2e-3 * np.abs(f(p.w_out)).sum(axis=1)[None, :]
    _close(y.cpu(), ref, mag, f"attention block config {idx}", extra=extra)


def test_bad_shapes(gpu):
    p = workloads.make_layer_params()
    g = _gpu(p)
    x = workloads.draw_layer_input(10).cuda()
    with pytest.raises(vlca.VlcaError) as e:
        vlca.ln_qkv(x, g["gamma"], g["beta"], g["w_qkv"][:100], g["b_qkv"][:100])
    assert e.value.code == -14
    with pytest.raises(ValueError):
        vlca.out_residual(x, g["w_out"], g["b_out"], x[:5])
