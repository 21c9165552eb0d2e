"""Pins for the oracle's attention forward and backward (CPU only).

What fixes each value, independently of oracle.c:
  * golden fixtures under tests/golden/ holding the pages' worked examples
    (interleave order, the position-4 visibility example, the paired window,
    the 4x4 lower-triangular mask);
  * closed forms: with q = 0 every visible key gets the same weight, so
    LSE = ln(#visible) and O = mean of the visible values; the first slot of a
    sequence returns its own value; rows of P sum to one;
  * a library route: torch's fp64 scaled_dot_product_attention(is_causal=True)
    per sequence, the fallback the "Upgrading a textbook decoder" article
    (juejin.cn, section 4) uses, and batched for equal-length sequences;
  * a dense numpy brute force (tests/brute.py) on tiny random inputs;
  * backward: fp64 central finite differences of L = sum(O * dO), torch
    autograd through SDPA, and the invariants sum_keys dK = 0 and
    sum_keys dV = sum_queries dO per sequence and head.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- pairing --

def test_interleave_order_matches_page_example():
    g = golden("interleave_order.json")
    H, T = 2, 3
    labels = {}
    for t in range(T):
        for h in range(H):
            s, j = oracle.slot_map(t, h, H, 1)
            assert j == 0
            labels[s] = g["before"][h][t]
    assert [labels[s] for s in range(2 * T)] == g["after"]
    # H = 2: the prose reading (partner h ^ 1) gives the same order
    for t in range(T):
        for h in range(H):
            assert oracle.slot_map(t, h, H, 2) == oracle.slot_map(t, h, H, 1)


@pytest.mark.parametrize("H", [2, 4, 6])
def test_slot_map_is_the_memory_view(H):
    """paired=1 equals viewing [N, H, d] memory as [2N, H/2, d]."""
    N, d = 5, 3
    x = np.arange(N * H * d).reshape(N, H, d)
    view = x.reshape(2 * N, H // 2, d)
    for n in range(N):
        for h in range(H):
            s, j = oracle.slot_map(n, h, H, 1)
            np.testing.assert_array_equal(view[s, j], x[n, h])


@pytest.mark.parametrize("paired", [1, 2])
def test_slot_map_matches_literal_list(paired):
    H, N = 6, 4
    x = np.arange(N * H, dtype=np.float64).reshape(N, H, 1)
    seqs, origin = brute.interleave(x, H, paired)
    for j, org in enumerate(origin):
        for slot, (t, h) in enumerate(org):
            assert oracle.slot_map(int(t), int(h), H, paired) == (slot, j)


# ------------------------------------------------------- closed-form pins --

def visible_count(cu, mult, causal, window, i):
    for b, e in zip(cu[:-1], cu[1:]):
        b, e = b * mult, e * mult
        if b <= i < e:
            c = 0
            for j in range(b, e):
                if causal and j > i:
                    continue
                if window > 0 and i - j >= window:
                    continue
                c += 1
            return c
    raise AssertionError


@pytest.mark.parametrize("paired,causal,window", [(0, 1, 0), (0, 0, 0), (0, 1, 3), (1, 1, 0),
                                                  (1, 1, 5), (2, 1, 4), (1, 0, 0)])
def test_zero_query_gives_log_count_and_mean(paired, causal, window):
    N, H, d = 11, 4, 6
    cu = np.array([0, 4, 4, 11], np.int32)
    q = np.zeros((N, H, d))
    k = rnd((N, H, d), 1)
    v = rnd((N, H, d), 2)
    o, lse = oracle.attn_fwd(q, k, v, cu, paired, causal, window)
    mult = 2 if paired else 1
    Hs = H // 2 if paired else H
    for j in range(Hs):
        for i in range(N * mult):
            assert lse[j, i] == pytest.approx(np.log(visible_count(cu, mult, causal, window, i)),
                                              abs=1e-14)
    # O = mean of visible values, via the brute-force slot lists
    vs, origin = brute.interleave(v, H, paired)
    mask = brute.dense_mask(list(cu), mult, causal, window)
    for j in range(Hs):
        for slot, (t, h) in enumerate(origin[j]):
            np.testing.assert_allclose(o[t, h], vs[j][mask[slot]].mean(axis=0), atol=1e-13)


@pytest.mark.parametrize("paired", [0, 1])
def test_rows_sum_to_one(paired):
    N, H, d = 9, 2, 5
    cu = np.array([0, 9], np.int32)
    o, _ = oracle.attn_fwd(rnd((N, H, d), 3) * 3, rnd((N, H, d), 4) * 3, np.ones((N, H, d)), cu,
                           paired, 1, 0)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-15)


def test_first_slot_returns_its_value():
    N, H, d = 12, 4, 8
    cu = np.array([0, 5, 12], np.int32)
    q, k, v = rnd((N, H, d), 5), rnd((N, H, d), 6), rnd((N, H, d), 7)
    for paired in (0, 1):
        o, lse = oracle.attn_fwd(q, k, v, cu, paired, 1, 0, 0.3)
        for start in cu[:-1]:
            if paired:   # slot 2*start holds the first pair member of each head
                for h in range(H // 2):
                    np.testing.assert_array_equal(o[start, h], v[start, h])
                    assert lse[h, 2 * start] == pytest.approx(0.3 * q[start, h] @ k[start, h],
                                                              abs=1e-14)
            else:
                np.testing.assert_array_equal(o[start], v[start])
                for h in range(H):
                    assert lse[h, start] == pytest.approx(0.3 * q[start, h] @ k[start, h],
                                                          abs=1e-14)


def visible_by_one_hot(T, window=0):
    """Paired H = 2 with q = 0 and one-hot values: returns, for every query
    slot, the set of visible key slots as read off the output."""
    N, H = T, 2
    d = 2 * T
    v = np.zeros((N, H, d))
    for t in range(T):
        for h in range(H):
            s, _ = oracle.slot_map(t, h, H, 1)
            v[t, h, s] = 1.0
    o, _ = oracle.attn_fwd(np.zeros((N, H, d)), rnd((N, H, d), 8), v,
                           np.array([0, T], np.int32), 1, 1, window)
    seen = {}
    for t in range(T):
        for h in range(H):
            s, _ = oracle.slot_map(t, h, H, 1)
            row = o[t, h]
            keys = set(np.nonzero(row > 1e-12)[0].tolist())
            np.testing.assert_allclose(row[sorted(keys)], 1.0 / len(keys), atol=1e-14)
            seen[(t, h)] = keys
    return seen


def test_paired_visibility_page_example():
    g = golden("paired_visibility.json")
    p = g["position"] - 1           # 0-based token index
    seen = visible_by_one_hot(8)
    slot = lambda t, h: oracle.slot_map(t, h, 2, 1)[0]
    head2_keys_of_head1_query = sorted(t + 1 for t in range(8) if slot(t, 1) in seen[(p, 0)])
    head1_keys_of_head2_query = sorted(t + 1 for t in range(8) if slot(t, 0) in seen[(p, 1)])
    assert head2_keys_of_head1_query == g["head1_query_sees_head2_keys"]
    assert head1_keys_of_head2_query == g["head2_query_sees_head1_keys"]


def test_paired_window_page_statement():
    g = golden("paired_window.json")
    W = g["window_slots"]
    T = 200
    seen = visible_by_one_hot(T, W)
    slot = lambda t, h: oracle.slot_map(t, h, 2, 1)[0]
    for t in (150, 199):
        for h in (0, 1):
            keys = seen[(t, h)]
            assert len(keys) == g["total_key_slots"]
            for hh in (0, 1):
                positions = [tt for tt in range(T) if slot(tt, hh) in keys]
                assert len(positions) == g["positions_per_head"]


def test_tril_mask_page_example():
    g = golden("tril_mask.json")
    for T, key in ((4, "block_size_4"), (2, "seq_len_2"), (3, "seq_len_3")):
        d = T
        v = np.eye(T).reshape(T, 1, d)
        o, _ = oracle.attn_fwd(np.zeros((T, 1, d)), rnd((T, 1, d), 9), v,
                               np.array([0, T], np.int32), 0, 1, 0)
        vis = (o[:, 0, :] > 1e-12).astype(int)
        assert vis.tolist() == g[key]


# ------------------------------------------------ brute force / libraries --

CASES = [
    # N, H, d, cu, paired, causal, window
    (16, 1, 4, [0, 16], 0, 1, 0),
    (20, 3, 8, [0, 7, 7, 20], 0, 1, 0),
    (20, 2, 8, [0, 9, 20], 0, 0, 0),
    (24, 4, 8, [0, 5, 17, 24], 0, 1, 4),
    (12, 2, 16, [0, 12], 1, 1, 0),
    (15, 6, 8, [0, 6, 15], 1, 1, 0),
    (15, 6, 8, [0, 6, 15], 1, 1, 7),
    (15, 4, 8, [0, 10, 15], 2, 1, 5),
    (10, 4, 4, [0, 3, 10], 1, 0, 0),
]


@pytest.mark.parametrize("case", CASES)
def test_forward_against_dense_brute_force(case):
    N, H, d, cu, paired, causal, window = case
    cu = np.array(cu, np.int32)
    q, k, v = rnd((N, H, d), 10), rnd((N, H, d), 11), rnd((N, H, d), 12)
    o, lse = oracle.attn_fwd(q, k, v, cu, paired, causal, window, 0.4)
    ob, lseb, probs = brute.attention(q, k, v, cu, paired, causal, window, 0.4)
    np.testing.assert_allclose(o, ob, atol=1e-12)
    np.testing.assert_allclose(lse, lseb, atol=1e-12)
    for p in probs:
        np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-15)


def test_forward_against_torch_sdpa_per_sequence():
    N, H, d = 40, 3, 16
    cu = np.array([0, 13, 13, 31, 40], np.int32)
    q, k, v = rnd((N, H, d), 13), rnd((N, H, d), 14), rnd((N, H, d), 15)
    o, _ = oracle.attn_fwd(q, k, v, cu, 0, 1, 0)
    for b, e in zip(cu[:-1], cu[1:]):
        if e == b:
            continue
        t = lambda x: torch.from_numpy(x[b:e]).transpose(0, 1)   # [H, L, d]
        ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True)
        np.testing.assert_allclose(o[b:e], ref.transpose(0, 1).numpy(), atol=1e-12)


def test_forward_window_against_torch_sdpa_with_boolean_mask():
    N, H, d, W = 30, 2, 8, 6
    q, k, v = rnd((N, H, d), 16), rnd((N, H, d), 17), rnd((N, H, d), 18)
    o, _ = oracle.attn_fwd(q, k, v, np.array([0, N], np.int32), 0, 1, W)
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    mask = (j <= i) & (i - j < W)
    t = lambda x: torch.from_numpy(x).transpose(0, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=mask)
    np.testing.assert_allclose(o, ref.transpose(0, 1).numpy(), atol=1e-12)


def test_equal_sequences_equal_batched_sdpa():
    """cu = [0, T, 2T, ...] is the B x T batch of the GPT-2-style problem."""
    B, T, H, d = 3, 16, 2, 8
    N = B * T
    q, k, v = rnd((N, H, d), 19), rnd((N, H, d), 20), rnd((N, H, d), 21)
    o, _ = oracle.attn_fwd(q, k, v, np.arange(0, N + 1, T, dtype=np.int32), 0, 1, 0)
    t = lambda x: torch.from_numpy(x).reshape(B, T, H, d).transpose(1, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True)
    np.testing.assert_allclose(o, ref.transpose(1, 2).reshape(N, H, d).numpy(), atol=1e-12)


def test_rows_api_matches_full():
    N, H, d = 30, 6, 8
    cu = np.array([0, 11, 30], np.int32)
    q, k, v = rnd((N, H, d), 22), rnd((N, H, d), 23), rnd((N, H, d), 24)
    o, lse = oracle.attn_fwd(q, k, v, cu, 1, 1, 9)
    rows = [(0, 0), (2, 59), (1, 22), (0, 21), (2, 5)]
    orow, lrow = oracle.attn_fwd_rows(q, k, v, cu, rows, 1, 1, 9)
    for r, (j, s) in enumerate(rows):
        # slot s of attention head j is token s // 2, head j + (s % 2) * H/2
        t, h = s // 2, j + (s % 2) * (H // 2)
        np.testing.assert_array_equal(orow[r], o[t, h])
        assert lrow[r] == lse[j, s]


# -------------------------------------------------------------- backward --

BWD_CASES = [
    (10, 2, 4, [0, 10], 0, 1, 0),
    (12, 2, 4, [0, 5, 12], 0, 1, 3),
    (8, 4, 4, [0, 3, 8], 1, 1, 0),
    (8, 4, 4, [0, 8], 1, 1, 5),
    (9, 2, 4, [0, 4, 9], 0, 0, 0),
]


@pytest.mark.parametrize("case", BWD_CASES)
def test_backward_against_finite_differences(case):
    N, H, d, cu, paired, causal, window = case
    cu = np.array(cu, np.int32)
    q, k, v, g = (rnd((N, H, d), 30 + i) for i in range(4))
    dq, dk, dv = oracle.attn_bwd(q, k, v, g, cu, paired, causal, window, 0.5)

    def loss(qq, kk, vv):
        o, _ = oracle.attn_fwd(qq, kk, vv, cu, paired, causal, window, 0.5)
        return float((o * g).sum())

    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = loss(args["q"], args["k"], args["v"])
            args[name] = xm
            lm = loss(args["q"], args["k"], args["v"])
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(grad, num, atol=1e-8, err_msg=name)


def test_backward_against_torch_autograd():
    N, H, d = 24, 2, 8
    cu = np.array([0, 24], np.int32)
    q, k, v, g = (rnd((N, H, d), 40 + i) for i in range(4))
    dq, dk, dv = oracle.attn_bwd(q, k, v, g, cu, 0, 1, 0)
    tq, tk, tv = (torch.from_numpy(x).transpose(0, 1).clone().requires_grad_(True)
                  for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    (out * torch.from_numpy(g).transpose(0, 1)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.transpose(0, 1).numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.transpose(0, 1).numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.transpose(0, 1).numpy(), atol=1e-12)


@pytest.mark.parametrize("paired", [0, 1])
def test_backward_sum_invariants(paired):
    N, H, d = 26, 4, 8
    cu = np.array([0, 9, 26], np.int32)
    q, k, v, g = (rnd((N, H, d), 50 + i) for i in range(4))
    dq, dk, dv = oracle.attn_bwd(q, k, v, g, cu, paired, 1, 6)
    for b, e in zip(cu[:-1], cu[1:]):
        if paired:   # sums run over both members of each attention head
            for j in range(H // 2):
                hs = [j, j + H // 2]
                np.testing.assert_allclose(dk[b:e][:, hs].sum(axis=(0, 1)), 0.0, atol=1e-12)
                np.testing.assert_allclose(dv[b:e][:, hs].sum(axis=(0, 1)),
                                           g[b:e][:, hs].sum(axis=(0, 1)), atol=1e-12)
        else:
            np.testing.assert_allclose(dk[b:e].sum(axis=0), 0.0, atol=1e-12)
            np.testing.assert_allclose(dv[b:e].sum(axis=0), g[b:e].sum(axis=0), atol=1e-12)


def test_backward_sampled_matches_full():
    N, H, d = 20, 4, 8
    cu = np.array([0, 7, 20], np.int32)
    q, k, v, g = (rnd((N, H, d), 60 + i) for i in range(4))
    dq, dk, dv = oracle.attn_bwd(q, k, v, g, cu, 1, 1, 7)
    qr = [(0, 3), (1, 39), (1, 14)]
    kc = [(0, 0), (1, 13), (0, 38), (1, 14)]
    sq, sk, sv = oracle.attn_bwd_sampled(q, k, v, g, cu, qr, kc, 1, 1, 7)
    tok = lambda j, s: (s // 2, j + (s % 2) * (H // 2))
    for r, (j, s) in enumerate(qr):
        np.testing.assert_allclose(sq[r], dq[tok(j, s)], atol=1e-14)
    for r, (j, s) in enumerate(kc):
        np.testing.assert_allclose(sk[r], dk[tok(j, s)], atol=1e-14)
        np.testing.assert_allclose(sv[r], dv[tok(j, s)], atol=1e-14)


def test_forward_rejects_bad_arguments():
    x = np.zeros((4, 2, 8))
    with pytest.raises(ValueError):
        oracle.attn_fwd(x, x, x, np.array([0, 4], np.int32), 0, 0, 3)   # window without causal
    with pytest.raises(ValueError):
        oracle.attn_fwd(x, x, x, np.array([0, 5], np.int32))             # cu past N
    with pytest.raises(ValueError):
        oracle.attn_fwd(x, x, x, np.array([0, 3, 2, 4], np.int32))       # decreasing cu
