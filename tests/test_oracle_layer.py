"""Pins of the layer oracle (CPU): LayerNorm against torch's layer_norm (fp64,
a library routine) and its invariants, Linear against a brute-force sum, and the
attention sub-block's closed forms (zero output projection passes the residual
through; a constant value block gives the running mean of prefix V, as the
attention pins fix)."""
import numpy as np
import torch

import oracle


def test_layer_norm_matches_torch_and_normalises():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 512)) * 3 + 2
    g, b = rng.standard_normal(512), rng.standard_normal(512)
    ref = torch.nn.functional.layer_norm(torch.tensor(x), (512,), torch.tensor(g), torch.tensor(b), 1e-5).numpy()
    assert np.max(np.abs(oracle.layer_norm(x, g, b, 1e-5) - ref)) <= 1e-12
    y = oracle.layer_norm(x, np.ones(512), np.zeros(512), 0.0)
    assert np.max(np.abs(y.mean(axis=1))) <= 1e-12 and np.max(np.abs(y.var(axis=1) - 1)) <= 1e-12


def test_linear_brute_force():
    rng = np.random.default_rng(2)
    x, w, b = rng.standard_normal((3, 5)), rng.standard_normal((4, 5)), rng.standard_normal(4)
    want = np.array([[sum(x[i, k] * w[o, k] for k in range(5)) + b[o] for o in range(4)] for i in range(3)])
    assert np.max(np.abs(oracle.linear(x, w, b) - want)) <= 1e-12


def test_block_closed_forms():
    rng = np.random.default_rng(3)
    T, H, D = 40, 8, 64
    cu = [0, 10, 40]
    x = rng.standard_normal((T, 512))
    g, b = 1 + 0.1 * rng.standard_normal(512), 0.1 * rng.standard_normal(512)
    wq, bq = rng.standard_normal((1536, 512)) / 22.6, rng.standard_normal(1536) * 0.1
    # zero output projection: the block is the identity on x
    y = oracle.attention_block(x, cu, H, D, 0.125, g, b, 1e-5, wq, bq, np.zeros((512, 512)), np.zeros(512))
    assert np.array_equal(y, x)
    # q block of the projection zero, v block the identity on LN(x): uniform causal
    # weights, so each row's attention output is the running mean of LN(x) rows
    wq2 = np.zeros((1536, 512))
    wq2[1024:] = np.eye(512)
    y = oracle.attention_block(x, cu, H, D, 0.125, g, b, 1e-5, wq2, np.zeros(1536), np.eye(512), np.zeros(512))
    ln = oracle.layer_norm(x, g, b, 1e-5)
    for s, e in ((0, 10), (10, 40)):
        want = x[s:e] + np.cumsum(ln[s:e], axis=0) / np.arange(1, e - s + 1)[:, None]
        assert np.max(np.abs(y[s:e] - want)) <= 1e-12
