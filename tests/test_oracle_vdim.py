"""Pins for the oracle with a value width dv different from the query/key width
d (the "Paired Head Attention" article, section "Source 1: model
configuration", gives every attention module its own qk_dim and v_dim).

What fixes the values, independently of oracle.c:
  * the dense numpy brute force (tests/brute.py) and torch's fp64
    scaled_dot_product_attention, which accepts a value width of its own;
  * the column split: attention is linear in V, so the output for V = [V1 | V2]
    is [O(V1) | O(V2)], and each half is an equal-width problem the other
    tests pin; in the backward, dV splits the same way and dQ, dK add up;
  * fp64 central finite differences of L = sum(O * dO) and torch autograd.
"""
import numpy as np
import pytest
import torch

import oracle
import brute


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


CASES = [  # N, H, d, dv, cu, paired, causal, window
    (14, 2, 8, 16, [0, 6, 14], 0, 1, 0),
    (12, 4, 8, 4, [0, 12], 1, 1, 5),
    (10, 4, 4, 12, [0, 3, 10], 2, 1, 0),
    (9, 2, 8, 4, [0, 4, 9], 0, 0, 0),
]


@pytest.mark.parametrize("case", CASES)
def test_forward_against_brute_force(case):
    N, H, d, dv, cu, paired, causal, window = case
    cu = np.array(cu, np.int32)
    q, k, v = rnd((N, H, d), 1), rnd((N, H, d), 2), rnd((N, H, dv), 3)
    o, lse = oracle.attn_fwd(q, k, v, cu, paired, causal, window, 0.3)
    ob, lseb, _ = brute.attention(q, k, v, cu, paired, causal, window, 0.3)
    assert o.shape == (N, H, dv)
    np.testing.assert_allclose(o, ob, atol=1e-12)
    np.testing.assert_allclose(lse, lseb, atol=1e-12)


@pytest.mark.parametrize("d,dv", [(16, 32), (16, 8)])
def test_forward_against_torch_sdpa(d, dv):
    N, H = 20, 3
    q, k, v = rnd((N, H, d), 4), rnd((N, H, d), 5), rnd((N, H, dv), 6)
    o, _ = oracle.attn_fwd(q, k, v, np.array([0, N], np.int32), 0, 1, 0)
    t = lambda x: torch.from_numpy(x).transpose(0, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True)
    np.testing.assert_allclose(o, ref.transpose(0, 1).numpy(), atol=1e-12)


@pytest.mark.parametrize("paired", [0, 1, 2])
def test_column_split_forward_and_backward(paired):
    N, H, d = 16, 4, 8
    cu = np.array([0, 7, 16], np.int32)
    q, k = rnd((N, H, d), 7), rnd((N, H, d), 8)
    v1, v2, g1, g2 = (rnd((N, H, d), 9 + i) for i in range(4))
    o, lse = oracle.attn_fwd(q, k, np.concatenate([v1, v2], 2), cu, paired, 1, 6)
    o1, lse1 = oracle.attn_fwd(q, k, v1, cu, paired, 1, 6)
    o2, _ = oracle.attn_fwd(q, k, v2, cu, paired, 1, 6)
    np.testing.assert_allclose(o, np.concatenate([o1, o2], 2), atol=1e-13)
    np.testing.assert_allclose(lse, lse1, atol=1e-13)
    dq, dk, dv = oracle.attn_bwd(q, k, np.concatenate([v1, v2], 2), np.concatenate([g1, g2], 2),
                                 cu, paired, 1, 6)
    a = oracle.attn_bwd(q, k, v1, g1, cu, paired, 1, 6)
    b = oracle.attn_bwd(q, k, v2, g2, cu, paired, 1, 6)
    np.testing.assert_allclose(dq, a[0] + b[0], atol=1e-12)
    np.testing.assert_allclose(dk, a[1] + b[1], atol=1e-12)
    np.testing.assert_allclose(dv, np.concatenate([a[2], b[2]], 2), atol=1e-12)


@pytest.mark.parametrize("case", CASES[:3])
def test_backward_against_finite_differences(case):
    N, H, d, dv, cu, paired, causal, window = case
    N = min(N, 8)
    cu = np.array([0, 3, N], np.int32)
    q, k = rnd((N, H, d), 20), rnd((N, H, d), 21)
    v, g = rnd((N, H, dv), 22), rnd((N, H, dv), 23)
    grads = oracle.attn_bwd(q, k, v, g, cu, paired, causal, window, 0.5)

    def loss(qq, kk, vv):
        o, _ = oracle.attn_fwd(qq, kk, vv, cu, paired, causal, window, 0.5)
        return float((o * g).sum())

    eps = 1e-6
    for i, (name, x) in enumerate((("q", q), ("k", k), ("v", v))):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            args = [q, k, v]
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args[i] = xp
            lp = loss(*args)
            args[i] = xm
            num[idx] = (lp - loss(*args)) / (2 * eps)
        assert grads[i].shape == x.shape
        np.testing.assert_allclose(grads[i], num, atol=1e-8, err_msg=name)


def test_backward_against_torch_autograd():
    N, H, d, dv = 18, 2, 8, 24
    cu = np.array([0, N], np.int32)
    q, k = rnd((N, H, d), 30), rnd((N, H, d), 31)
    v, g = rnd((N, H, dv), 32), rnd((N, H, dv), 33)
    dq, dk, dv_ = oracle.attn_bwd(q, k, v, g, cu, 0, 1, 0)
    tq, tk, tv = (torch.from_numpy(x).transpose(0, 1).clone().requires_grad_(True)
                  for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    (out * torch.from_numpy(g).transpose(0, 1)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.transpose(0, 1).numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.transpose(0, 1).numpy(), atol=1e-12)
    np.testing.assert_allclose(dv_, tv.grad.transpose(0, 1).numpy(), atol=1e-12)


def test_rows_and_sampled_match_full():
    N, H, d, dv = 20, 4, 8, 16
    cu = np.array([0, 9, 20], np.int32)
    q, k = rnd((N, H, d), 40), rnd((N, H, d), 41)
    v, g = rnd((N, H, dv), 42), rnd((N, H, dv), 43)
    o, lse = oracle.attn_fwd(q, k, v, cu, 1, 1, 7)
    rows = [(0, 0), (1, 39), (1, 18), (0, 25)]
    orow, lrow = oracle.attn_fwd_rows(q, k, v, cu, rows, 1, 1, 7)
    dq, dk, dvf = oracle.attn_bwd(q, k, v, g, cu, 1, 1, 7)
    sq, sk, sv = oracle.attn_bwd_sampled(q, k, v, g, cu, rows, rows, 1, 1, 7)
    for r, (j, s) in enumerate(rows):
        t, h = s // 2, j + (s % 2) * (H // 2)
        np.testing.assert_array_equal(orow[r], o[t, h])
        assert lrow[r] == lse[j, s]
        np.testing.assert_allclose(sq[r], dq[t, h], atol=1e-13)
        np.testing.assert_allclose(sk[r], dk[t, h], atol=1e-13)
        np.testing.assert_allclose(sv[r], dvf[t, h], atol=1e-13)


def test_grouped_kv_with_separate_value_width():
    N, H, Hkv, d, dv = 12, 4, 2, 8, 16
    cu = np.array([0, 5, 12], np.int32)
    q, k, v = rnd((N, H, d), 50), rnd((N, Hkv, d), 51), rnd((N, Hkv, dv), 52)
    g = rnd((N, H, dv), 53)
    o, _ = oracle.attn_fwd_gqa(q, k, v, cu, 1, 0)
    ob, _, _ = brute.attention(q, np.repeat(k, 2, 1), np.repeat(v, 2, 1), cu, 0, 1, 0)
    np.testing.assert_allclose(o, ob, atol=1e-12)
    dq, dk, dv_ = oracle.attn_bwd_gqa(q, k, v, g, cu, 1, 0)
    assert dk.shape == (N, Hkv, d) and dv_.shape == (N, Hkv, dv)


def test_value_shape_is_checked():
    q = rnd((4, 2, 8), 60)
    with pytest.raises(ValueError):
        oracle.attn_fwd(q, q, rnd((4, 3, 8), 61), np.array([0, 4], np.int32))
    with pytest.raises(ValueError):
        oracle.attn_bwd(q, q, rnd((4, 2, 16), 62), rnd((4, 2, 8), 63), np.array([0, 4], np.int32))
