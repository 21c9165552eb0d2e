"""Pins of the oracle's QK RMS-norm and of the transpose of its rotation (the
rope backward): against torch's own rms_norm and its autograd, the adjoint
identity <rope(x), y> = <x, rope_bwd(y)>, the inverse rope_bwd(rope(x)) = x,
closed forms and finite differences."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def rnd(shape, seed, scale=1.0):
    return scale * np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("d,eps", [(64, 1e-6), (128, 1e-6), (8, 0.3)])
def test_rms_norm_matches_torch(d, eps):
    x = rnd((7, 3, d), 1, 3.0)
    ref = F.rms_norm(torch.from_numpy(x), (d,), eps=eps).numpy()
    np.testing.assert_allclose(oracle.rms_norm(x, eps), ref, atol=1e-14)


def test_rms_norm_closed_forms():
    d, eps = 16, 1e-6
    c = 2.5
    x = np.full((1, 1, d), c)
    np.testing.assert_allclose(oracle.rms_norm(x, eps), c / np.sqrt(c * c + eps), atol=1e-15)
    # scale invariance up to eps: norm(a x) -> norm(x) as eps -> 0
    x = rnd((4, 2, d), 2)
    np.testing.assert_allclose(oracle.rms_norm(1000 * x, 0.0), oracle.rms_norm(x, 0.0),
                               atol=1e-13)
    np.testing.assert_allclose(np.zeros((1, 1, d)), oracle.rms_norm(np.zeros((1, 1, d)), eps))


@pytest.mark.parametrize("d,eps", [(64, 1e-6), (16, 0.5)])
def test_rms_norm_backward_matches_torch_autograd(d, eps):
    x, g = rnd((5, 3, d), 3), rnd((5, 3, d), 4)
    xt = torch.from_numpy(x).requires_grad_(True)
    (F.rms_norm(xt, (d,), eps=eps) * torch.from_numpy(g)).sum().backward()
    np.testing.assert_allclose(oracle.rms_norm_bwd(x, g, eps), xt.grad.numpy(), atol=1e-12)


def test_rms_norm_backward_is_orthogonal_to_x_without_eps():
    # with eps = 0 the norm is scale invariant, so its gradient is orthogonal to x
    x, g = rnd((6, 2, 32), 5), rnd((6, 2, 32), 6)
    dx = oracle.rms_norm_bwd(x, g, 0.0)
    np.testing.assert_allclose((dx * x).sum(-1), 0.0, atol=1e-12)


@pytest.mark.parametrize("convention,paired", [(1, 0), (2, 0), (2, 1), (1, 2)])
def test_rope_bwd_is_the_adjoint_and_the_inverse(convention, paired):
    cu = np.array([0, 9, 9, 40], np.int32)
    x, y = rnd((40, 4, 16), 7), rnd((40, 4, 16), 8)
    rx = oracle.rope(x, cu, convention, 10000.0, paired)
    ry = oracle.rope_bwd(y, cu, convention, 10000.0, paired)
    assert abs((rx * y).sum() - (x * ry).sum()) < 1e-11
    np.testing.assert_allclose(oracle.rope_bwd(rx, cu, convention, 10000.0, paired), x,
                               atol=1e-13)


@pytest.mark.parametrize("norm", [False, True])
def test_qk_prep_backward_against_finite_differences(norm):
    cu = np.array([0, 3, 7], np.int32)
    x, g = rnd((7, 2, 8), 9), rnd((7, 2, 8), 10)
    dx = oracle.qk_prep_bwd(x, g, cu, 2, 100.0, 1, norm, 1e-3)
    f = lambda z: (oracle.qk_prep(z, cu, 2, 100.0, 1, norm, 1e-3) * g).sum()
    h = 1e-6
    for idx in [(0, 0, 0), (3, 1, 5), (6, 0, 7), (4, 1, 2)]:
        e = np.zeros_like(x)
        e[idx] = h
        assert abs((f(x + e) - f(x - e)) / (2 * h) - dx[idx]) < 1e-7
