"""Pins for the oracle's rotary embedding (CPU only).

Each check is fixed by the pages or by the mathematics of a rotation, not by
re-typing the oracle's own expressions:
  * position 0 is the identity; every pair keeps its norm;
  * rotations compose additively, R(a) R(b) = R(a + b);
  * for head_dim 2 the rotation is multiplication of a + ib by exp(i p), the
    textbook complex form;
  * the score q'_m . k'_n depends only on m - n ("Upgrading a textbook decoder",
    juejin.cn, section 2 "RoPE": the relative-position property);
  * frequencies: theta_0 = 1, theta_{d/4} = base^(-1/2), a geometric sequence;
  * half-split on x equals adjacent-pair on the pair-interleaved x;
  * paired stagger: head h of token t rotates as unpaired position 2t + h mod 2
    ("Paired Head Attention" article, hncyxsy.com, "Staggered rotary");
  * a complex-multiplication brute force on random tiny inputs.
"""
import numpy as np
import pytest

import oracle
import brute


def rng(seed=0):
    return np.random.default_rng(seed)


@pytest.mark.parametrize("conv", [1, 2])
def test_position_zero_is_identity(conv):
    x = rng(1).standard_normal((7, 3, 16))
    cu = np.array([0, 3, 7], dtype=np.int32)
    y = oracle.rope(x, cu, conv)
    np.testing.assert_array_equal(y[0], x[0])
    np.testing.assert_array_equal(y[3], x[3])
    assert not np.allclose(y[1], x[1])


@pytest.mark.parametrize("conv", [1, 2])
def test_pair_norms_preserved(conv):
    x = rng(2).standard_normal((40, 2, 32))
    y = oracle.rope(x, np.array([0, 40], np.int32), conv)
    if conv == 1:
        nx = x[..., :16] ** 2 + x[..., 16:] ** 2
        ny = y[..., :16] ** 2 + y[..., 16:] ** 2
    else:
        nx = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
        ny = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    np.testing.assert_allclose(ny, nx, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("conv", [1, 2])
def test_composition(conv):
    """R(b) R(a) x == R(a + b) x, using token offsets as positions."""
    d, a, b = 16, 5, 9
    x = rng(3).standard_normal((d,))
    L = a + b + 1
    buf = np.zeros((L, 1, d))
    buf[a, 0] = x
    ra = oracle.rope(buf, np.array([0, L], np.int32), conv)[a, 0]
    buf2 = np.zeros((L, 1, d))
    buf2[b, 0] = ra
    rba = oracle.rope(buf2, np.array([0, L], np.int32), conv)[b, 0]
    buf3 = np.zeros((L, 1, d))
    buf3[a + b, 0] = x
    rab = oracle.rope(buf3, np.array([0, L], np.int32), conv)[a + b, 0]
    np.testing.assert_allclose(rba, rab, rtol=0, atol=1e-12)


@pytest.mark.parametrize("conv", [1, 2])
def test_head_dim_two_is_complex_multiplication(conv):
    x = rng(4).standard_normal((11, 1, 2))
    y = oracle.rope(x, np.array([0, 11], np.int32), conv)
    z = (x[:, 0, 0] + 1j * x[:, 0, 1]) * np.exp(1j * np.arange(11))   # theta_0 = 1
    np.testing.assert_allclose(y[:, 0, 0], z.real, atol=1e-13)
    np.testing.assert_allclose(y[:, 0, 1], z.imag, atol=1e-13)


@pytest.mark.parametrize("conv", [1, 2])
@pytest.mark.parametrize("d", [8, 64, 128])
def test_frequency_spot_values(conv, d):
    """Angle of a unit vector at position p is p * theta_i with theta_0 = 1,
    theta_{d/4} = base^-1/2 and a constant ratio between neighbours."""
    half = d // 2
    base = 10000.0
    p = 1
    x = np.zeros((2, half, d))   # token 1, head i carries a unit vector in pair i
    for i in range(half):
        ia, ib = (i, i + half) if conv == 1 else (2 * i, 2 * i + 1)
        x[1, i, ia] = 1.0
    y = oracle.rope(x, np.array([0, 2], np.int32), conv, base)
    ang = []
    for i in range(half):
        ia, ib = (i, i + half) if conv == 1 else (2 * i, 2 * i + 1)
        ang.append(np.arctan2(y[1, i, ib], y[1, i, ia]) / p)
    ang = np.array(ang)
    assert abs(ang[0] - 1.0) < 1e-13
    assert abs(ang[half // 2] - 0.01) < 1e-15     # base^(-1/2) for base 1e4
    ratio = ang[1:] / ang[:-1]
    np.testing.assert_allclose(ratio, ratio[0], rtol=1e-12)
    # extrapolating the sequence one step past the end reaches 1/base
    assert abs(ang[-1] * ratio[0] - 1.0 / base) < 1e-15


@pytest.mark.parametrize("conv", [1, 2])
def test_relative_position_property(conv):
    d = 32
    r = rng(5)
    q, k = r.standard_normal(d), r.standard_normal(d)
    L = 200
    def rot(vec, pos):
        buf = np.zeros((L, 1, d))
        buf[pos, 0] = vec
        return oracle.rope(buf, np.array([0, L], np.int32), conv)[pos, 0]
    for m, n in [(3, 17), (40, 2), (100, 100)]:
        ref = rot(q, m) @ rot(k, n)
        for delta in (1, 7, 50):
            assert abs(rot(q, m + delta) @ rot(k, n + delta) - ref) < 1e-12
    # and it does depend on the offset
    assert abs(rot(q, 3) @ rot(k, 17) - rot(q, 3) @ rot(k, 18)) > 1e-6


def test_half_split_equals_adjacent_on_interleaved_pairs():
    d = 16
    x = rng(6).standard_normal((9, 2, d))
    cu = np.array([0, 4, 9], np.int32)
    perm = np.empty(d, dtype=np.int64)          # adjacent slot -> half-split index
    perm[0::2] = np.arange(d // 2)
    perm[1::2] = np.arange(d // 2) + d // 2
    y_half = oracle.rope(x, cu, 1)
    y_adj = oracle.rope(x[..., perm], cu, 2)
    np.testing.assert_allclose(y_adj, y_half[..., perm], atol=1e-13)


@pytest.mark.parametrize("conv", [1, 2])
def test_paired_stagger_matches_unpaired_positions(conv):
    """Paired head h at token t == unpaired RoPE at position 2t + (h mod 2)."""
    d, T, H = 16, 6, 4
    x = rng(7).standard_normal((T, H, d))
    y = oracle.rope(x, np.array([0, T], np.int32), conv, paired=1)
    L = 2 * T + 2
    for t in range(T):
        for h in range(H):
            buf = np.zeros((L, 1, d))
            pos = 2 * t + (h % 2)
            buf[pos, 0] = x[t, h]
            ref = oracle.rope(buf, np.array([0, L], np.int32), conv)[pos, 0]
            np.testing.assert_allclose(y[t, h], ref, atol=1e-13)


@pytest.mark.parametrize("conv", [1, 2])
@pytest.mark.parametrize("paired", [0, 1])
def test_rope_against_complex_brute_force(conv, paired):
    x = rng(8 + conv + paired).standard_normal((13, 4, 8))
    cu = np.array([0, 5, 5, 13], np.int32)   # includes an empty sequence
    np.testing.assert_allclose(oracle.rope(x, cu, conv, 500.0, paired),
                               brute.rope(x, cu, conv, 500.0, paired), atol=1e-12)


def test_rope_rejects_bad_arguments():
    x = np.zeros((4, 3, 8))
    with pytest.raises(ValueError):
        oracle.rope(x, np.array([0, 3], np.int32), 1)          # cu does not end at N
    with pytest.raises(ValueError):
        oracle.rope(x, np.array([0, 4], np.int32), 1, paired=1)  # odd head count
    with pytest.raises(ValueError):
        oracle.rope(x, np.array([0, 4], np.int32), 3)          # unknown convention
