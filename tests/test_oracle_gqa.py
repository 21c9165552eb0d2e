"""Pins of the oracle's grouped-query attention (query heads in groups that
share one K/V head; "Upgrading a textbook decoder", section 4 "GQA &
FlashAttention") against torch's own grouped scaled-dot-product attention and
its autograd, in fp64 on the CPU, and against brute force for one K/V head."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def sdpa_gqa(q, k, v, cu, window, requires_grad=False):
    """torch SDPA with enable_gqa per sequence (fp64), returns O [N, H, d]."""
    outs, leaves = [], []
    qt, kt, vt = (torch.from_numpy(x).requires_grad_(requires_grad) for x in (q, k, v))
    for b, e in zip(cu[:-1], cu[1:]):
        if e == b:
            continue
        L = e - b
        qs, ks, vs = (x[b:e].transpose(0, 1).unsqueeze(0) for x in (qt, kt, vt))
        i = torch.arange(L)
        mask = (i[None, :] <= i[:, None])
        if window > 0:
            mask &= (i[:, None] - i[None, :]) < window
        o = F.scaled_dot_product_attention(qs, ks, vs, attn_mask=mask, enable_gqa=True)
        outs.append(o[0].transpose(0, 1))
    return torch.cat(outs, 0), (qt, kt, vt)


@pytest.mark.parametrize("H,Hkv,cu,window", [
    (4, 2, [0, 37], 0),
    (6, 3, [0, 20, 51], 0),
    (8, 1, [0, 16, 16, 45], 7),       # MQA, an empty sequence, a window
    (6, 2, [0, 64], 17),
])
def test_gqa_forward_matches_torch_grouped_sdpa(H, Hkv, cu, window):
    N, d = cu[-1], 16
    q, k, v = rnd((N, H, d), 1), rnd((N, Hkv, d), 2), rnd((N, Hkv, d), 3)
    o, lse = oracle.attn_fwd_gqa(q, k, v, np.array(cu, np.int32), 1, window)
    ref, _ = sdpa_gqa(q, k, v, cu, window)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12)
    assert lse.shape == (H, N)


@pytest.mark.parametrize("H,Hkv,cu,window", [(4, 2, [0, 23, 41], 0), (6, 1, [0, 30], 9)])
def test_gqa_backward_matches_torch_autograd(H, Hkv, cu, window):
    N, d = cu[-1], 8
    q, k, v, g = rnd((N, H, d), 4), rnd((N, Hkv, d), 5), rnd((N, Hkv, d), 6), rnd((N, H, d), 7)
    dq, dk, dv = oracle.attn_bwd_gqa(q, k, v, g, np.array(cu, np.int32), 1, window)
    o, (qt, kt, vt) = sdpa_gqa(q, k, v, cu, window, requires_grad=True)
    (o * torch.from_numpy(g)).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(dk, kt.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(dv, vt.grad.numpy(), atol=1e-10)


def test_single_kv_head_brute_force():
    """MQA on a tiny causal problem, every row written out by hand."""
    N, H, d = 5, 3, 4
    q, k, v = rnd((N, H, d), 8), rnd((N, 1, d), 9), rnd((N, 1, d), 10)
    o, lse = oracle.attn_fwd_gqa(q, k, v, np.array([0, N], np.int32))
    s = 1 / np.sqrt(d)
    for h in range(H):
        for i in range(N):
            z = np.array([s * q[i, h] @ k[j, 0] for j in range(i + 1)])
            p = np.exp(z - z.max())
            np.testing.assert_allclose(o[i, h], (p / p.sum()) @ v[:i + 1, 0], atol=1e-13)
            np.testing.assert_allclose(lse[h, i], z.max() + np.log(p.sum()), atol=1e-13)


def test_expand_rejects_uneven_groups():
    with pytest.raises(ValueError):
        oracle.expand_kv(np.zeros((2, 3, 4)), 4)
