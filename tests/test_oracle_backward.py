"""Pins of the fp64 backward oracle and log-sum-exp (CPU).

The pages give no formula for the attention backward, so the oracle's gradient is
pinned to the derivative itself, independently of its formulas:
  * central finite differences of L = sum(dout * fwd(qkv)) over every input entry
    of a small ragged batch (catches a dropped term, a sign, a missing scale or a
    transposed operand in any of dQ, dK, dV);
  * torch.autograd through scaled_dot_product_attention(is_causal=True) in fp64
    on one user (a library routine on the single-segment special case);
  * closed forms: a length-1 user has dV = dO and dQ = dK = 0; equal keys give
    dQ = 0; gradients of one user do not depend on another's values;
  * the log-sum-exp against scipy's logsumexp.
"""
import numpy as np
import pytest
import torch

import oracle

H, D = 2, 64
SCALE = 0.125


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _loss(qkv, cu, dout):
    return float(np.sum(dout * oracle.varlen_causal_attention(qkv, cu, H, D, SCALE)))


def test_finite_differences_every_entry():
    lengths = [1, 3, 0, 4, 2]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T = int(cu[-1])
    qkv = _rand((T, 3 * H * D), 1, 0.7)
    dout = _rand((T, H * D), 2)
    g = oracle.varlen_causal_attention_backward(qkv, cu, dout, H, D, SCALE)
    eps = 1e-6
    fd = np.zeros_like(qkv)
    for idx in np.ndindex(*qkv.shape):
        x = qkv.copy()
        x[idx] += eps
        lp = _loss(x, cu, dout)
        x[idx] -= 2 * eps
        lm = _loss(x, cu, dout)
        fd[idx] = (lp - lm) / (2 * eps)
    assert np.max(np.abs(fd - g)) <= 1e-7 * max(1.0, np.max(np.abs(g)))
    # every block has gradient signal (the test cannot pass on zeros)
    for blk in range(3):
        assert np.max(np.abs(g[:, blk * H * D:(blk + 1) * H * D])) > 0.05


def test_single_user_matches_torch_autograd_sdpa():
    L = 37
    qkv = _rand((L, 3 * H * D), 3)
    dout = _rand((L, H * D), 4)
    g = oracle.varlen_causal_attention_backward(qkv, [0, L], dout, H, D, SCALE)
    t = torch.tensor(qkv, dtype=torch.float64, requires_grad=True)
    q = t[:, :H * D].reshape(L, H, D).transpose(0, 1)
    k = t[:, H * D:2 * H * D].reshape(L, H, D).transpose(0, 1)
    v = t[:, 2 * H * D:].reshape(L, H, D).transpose(0, 1)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=SCALE)
    o = o.transpose(0, 1).reshape(L, H * D)
    o.backward(torch.tensor(dout, dtype=torch.float64))
    assert np.max(np.abs(t.grad.numpy() - g)) <= 1e-12


def test_length_one_user_closed_form():
    lengths = [1, 5, 1]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    qkv = _rand((7, 3 * H * D), 5)
    dout = _rand((7, H * D), 6)
    g = oracle.varlen_causal_attention_backward(qkv, cu, dout, H, D, SCALE)
    for r in (0, 6):
        assert np.array_equal(g[r, 2 * H * D:], dout[r])  # P = 1: dV = dO
        assert np.max(np.abs(g[r, :2 * H * D])) <= 1e-15  # dS = dO.v - dO.v = 0


def test_equal_keys_give_zero_dq():
    L = 9
    qkv = _rand((L, 3 * H * D), 7)
    qkv[:, H * D:2 * H * D] = qkv[0, H * D:2 * H * D]  # every key the same
    dout = _rand((L, H * D), 8)
    g = oracle.varlen_causal_attention_backward(qkv, [0, L], dout, H, D, SCALE)
    assert np.max(np.abs(g[:, :H * D])) <= 1e-12  # rows of dS sum to 0
    assert np.max(np.abs(g[:, 2 * H * D:])) > 0.1


def test_isolation_across_users():
    lengths = [6, 4, 8]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    qkv = _rand((18, 3 * H * D), 9)
    dout = _rand((18, H * D), 10)
    a = oracle.varlen_causal_attention_backward(qkv, cu, dout, H, D, SCALE)
    qkv2 = qkv.copy()
    qkv2[6:10] = _rand((4, 3 * H * D), 11)
    dout2 = dout.copy()
    dout2[6:10] = -dout[6:10]
    b = oracle.varlen_causal_attention_backward(qkv2, cu, dout2, H, D, SCALE)
    keep = np.r_[0:6, 10:18]
    assert np.array_equal(a[keep], b[keep])
    assert not np.array_equal(a[6:10], b[6:10])


def test_lse_matches_logsumexp():
    from scipy.special import logsumexp

    lengths = [1, 7, 0, 20]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    qkv = _rand((28, 3 * H * D), 12, 2.0)
    lse = oracle.varlen_causal_attention_lse(qkv, cu, H, D, SCALE)
    for u in range(len(lengths)):
        s = int(cu[u])
        for i in range(lengths[u]):
            for h in range(H):
                q = qkv[s + i, h * D:(h + 1) * D]
                k = qkv[s:s + i + 1, H * D + h * D:H * D + (h + 1) * D]
                assert abs(lse[s + i, h] - logsumexp(SCALE * (k @ q))) <= 1e-12


def test_magnitude_bounds_the_gradient_and_is_tight_without_cancellation():
    lengths = [5, 1, 30]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    qkv = _rand((36, 3 * H * D), 13)
    dout = _rand((36, H * D), 14)
    g = oracle.varlen_causal_attention_backward(qkv, cu, dout, H, D, SCALE)
    m = oracle.varlen_causal_attention_backward_magnitude(qkv, cu, dout, H, D, SCALE)
    assert np.all(m >= np.abs(g) - 1e-12)  # triangle inequality
    assert np.max(m[:, :2 * H * D] - np.abs(g[:, :2 * H * D])) > 0.1  # dq, dk terms do cancel
    # brute force on one dQ element: the expansion dQ_id = scale sum_j P_ij (dP_ij -
    # sum_k P_ik dP_ik) k_jd with dP_ij = sum_e dO_ie v_je, every product in absolute value
    s0, i, d = 6, 20, 3  # user 2 (rows 6..35), its row 20, dim 3, head 0
    qq, kk, vv = (qkv[s0:s0 + 30, o:o + D] for o in (0, H * D, 2 * H * D))
    z = SCALE * (kk[:i + 1] @ qq[i])
    pr = np.exp(z - z.max()) / np.exp(z - z.max()).sum()
    do = dout[s0 + i, :D]
    brute = 0.0
    for j in range(i + 1):
        a = sum(abs(do[e] * vv[j, e]) for e in range(D))
        b = sum(pr[k2] * abs(do[e] * vv[k2, e]) for k2 in range(i + 1) for e in range(D))
        brute += pr[j] * (a + b) * abs(kk[j, d])
    assert abs(SCALE * brute - m[s0 + i, d]) <= 1e-10 * m[s0 + i, d]
    # with dO >= 0 every dV term is >= 0: the bound is attained
    pos = np.abs(dout)
    g2 = oracle.varlen_causal_attention_backward(qkv, cu, pos, H, D, SCALE)
    m2 = oracle.varlen_causal_attention_backward_magnitude(qkv, cu, pos, H, D, SCALE)
    assert np.max(np.abs(m2[:, 2 * H * D:] - g2[:, 2 * H * D:])) <= 1e-12
    # dV's bound is linear in |dO|
    assert np.allclose(oracle.varlen_causal_attention_backward_magnitude(qkv, cu, 3 * dout, H, D, SCALE)[:, 2 * H * D:],
                       3 * m[:, 2 * H * D:])
