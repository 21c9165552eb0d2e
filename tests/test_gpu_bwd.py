"""GPU parity of attn_bwd (dQ, dK, dV of the rotated inputs) against the fp64
oracle's chain-rule backward, through the C ABI.

The GPU forward and backward both run on the oracle's rotated, bf16-rounded
Q', K' (so the oracle receives nothing from the GPU).  Gradients are stored
in fp32 but computed on bf16 MFMA, so the bf16 bound (2e-2) applies.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import transformer_causal_self_amd as tca
from transformer_causal_self_amd import workloads as wl
from parity import (LSE_TOL, assert_close, f64, make_plan, oracle_rotated, sample_rows, say,
                    slot_to_token, tol)

pytestmark = pytest.mark.gpu

W = wl.WORKLOADS


def gpu_fwd_bwd(w, inp, qt, kt):
    plan = make_plan(w, inp["cu"])
    q, k, v, do = qt.cuda(), kt.cuda(), inp["v"].cuda(), inp["do"].cuda()
    o, lse = tca.attn_fwd(plan, q, k, v)
    dq, dk, dv = tca.attn_bwd(plan, q, k, v, o, lse, do)
    torch.cuda.synchronize()
    return [x.cpu().double().numpy() for x in (dq, dk, dv)]


def oracle_bwd(w, inp, qt, kt):
    return oracle.attn_bwd(f64(qt), f64(kt), f64(inp["v"]), f64(inp["do"]), inp["cu"], w.paired,
                           w.causal, w.window, w.scale)


CASES = [
    # name, workload
    ("long-context T=1000", W[5].scaled(1000)),
    ("long-context T=1500 two sequences", dataclasses.replace(W[5], n_tokens=1500, batch=2)),
    ("varlen window 2048 d128", W[4].scaled(3000, doc_range=(300, 1400))),
    ("paired varlen window 128 d128", W[3].scaled(1200, doc_range=(100, 700))),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bwd_reduced(case):
    name, w = case
    w = dataclasses.replace(w, backward=True)
    inp = wl.generate(w, with_grad=True)
    say(f"bwd {name}")
    _, _, qt, kt = oracle_rotated(w, inp)
    got = gpu_fwd_bwd(w, inp, qt, kt)
    ref = oracle_bwd(w, inp, qt, kt)
    for g, r, n in zip(got, ref, ("dQ", "dK", "dV")):
        assert_close(g, r, tol(w), n)


EDGE = [
    # name, H, d, cu, paired, window, rope
    ("tile-edge lengths", 2, 64, [0, 1, 64, 127, 191, 319, 448, 577], 0, 0, 1),
    ("empty sequences d128", 2, 128, [0, 0, 65, 65, 194, 194], 0, 0, 2),
    ("window 1", 2, 64, [0, 300], 0, 1, 1),
    ("window 129", 2, 64, [0, 40, 500], 0, 129, 1),
    ("paired H6 window 129", 6, 64, [0, 97, 301], 1, 129, 2),
    # 128-row items at d = 128 (its own schedule): lengths 127, 128, 129, 257
    ("item-edge lengths d128", 2, 128, [0, 127, 255, 384, 641], 0, 0, 1),
    ("window 200 d128", 2, 128, [0, 700], 0, 200, 2),
    # a window of INT32_MAX slots (a common "no window" value) is no window
    ("window INT32_MAX", 2, 64, [0, 90, 400], 0, 2147483647, 1),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_bwd_edge_cases(case):
    name, H, d, cu, paired, window, rope = case
    w = dataclasses.replace(W[5], n_tokens=cu[-1], heads=H, head_dim=d, paired=paired,
                            window=window, rope=rope, doc_range=None, batch=1)
    inp = wl.tensors(w, seed=21, with_grad=True)
    inp["cu"] = np.array(cu, np.int32)
    say(f"bwd edge case {name}")
    _, _, qt, kt = oracle_rotated(w, inp)
    got = gpu_fwd_bwd(w, inp, qt, kt)
    ref = oracle_bwd(w, inp, qt, kt)
    for g, r, n in zip(got, ref, ("dQ", "dK", "dV")):
        assert_close(g, r, tol(w), n)


def sampled_slots(T, H, rng, n=512):
    """(head, slot) pairs for a sampled full-size check: in every head the
    first and last slots, the edges of the 64- and 128-row tiles and of the
    2048-slot runs that share an XCD, then random slots, half of them among the
    last 2048 (where a row sees the most keys and its values are smallest)."""
    fixed = [0, 1, 63, 64, 127, 128, 2047, 2048, T // 2 - 1, T // 2, T - 129, T - 128, T - 2,
             T - 1]
    out = {(h, s) for h in range(H) for s in fixed if 0 <= s < T}
    while len(out) < n:
        s = int(rng.integers(0, T)) if len(out) % 2 else int(rng.integers(max(0, T - 2048), T))
        out.add((int(rng.integers(H)), s))
    return sorted(out)


def test_bwd_full_size_sampled():
    """The full long-context problem (T=16384, H=12, d=64); the oracle computes
    512 sampled dQ rows and 512 dK/dV columns (every head's tile edges and
    ends, random slots weighted toward the late ones)."""
    w = W[5]
    inp = wl.generate(w)
    say("bwd full long-context problem")
    _, _, qt, kt = oracle_rotated(w, inp)
    dq, dk, dv = gpu_fwd_bwd(w, inp, qt, kt)
    for x in (dq, dk, dv):
        assert np.isfinite(x).all()
    q_rows = sampled_slots(w.n_tokens, w.heads, np.random.default_rng(5))
    k_cols = sampled_slots(w.n_tokens, w.heads, np.random.default_rng(6))
    assert len(q_rows) >= 512 and len(k_cols) >= 512
    sq, sk, sv = oracle.attn_bwd_sampled(f64(qt), f64(kt), f64(inp["v"]), f64(inp["do"]),
                                         inp["cu"], q_rows, k_cols, 0, 1, 0, 0.0)
    assert_close(np.stack([dq[s, j] for j, s in q_rows]), sq, tol(w), "dQ rows")
    assert_close(np.stack([dk[s, j] for j, s in k_cols]), sk, tol(w), "dK cols")
    assert_close(np.stack([dv[s, j] for j, s in k_cols]), sv, tol(w), "dV cols")


@pytest.mark.parametrize("num", [3, 4])
def test_bwd_full_size_sampled_windowed(num):
    """Problems 3 (paired, window 128) and 4 (varlen, window 2048) at full
    size, d = 128 (the backward's own d = 128 schedule): sampled dQ rows and
    dK/dV columns from the oracle, sequence edges and tile edges included."""
    w = dataclasses.replace(W[num], backward=True)
    inp = wl.generate(w, with_grad=True)
    say(f"bwd full problem {num}: N={w.n_tokens}")
    _, _, qt, kt = oracle_rotated(w, inp)
    dq, dk, dv = gpu_fwd_bwd(w, inp, qt, kt)
    for x in (dq, dk, dv):
        assert np.isfinite(x).all()
    q_rows = sample_rows(w, inp["cu"], np.random.default_rng(10 + num), n_random=24)
    k_cols = sample_rows(w, inp["cu"], np.random.default_rng(20 + num), n_random=16)
    sq, sk, sv = oracle.attn_bwd_sampled(f64(qt), f64(kt), f64(inp["v"]), f64(inp["do"]),
                                         inp["cu"], q_rows, k_cols, w.paired, w.causal,
                                         w.window, w.scale)
    at = lambda x, rows: np.stack([x[slot_to_token(s, j, w.heads, w.paired)] for j, s in rows])
    assert_close(at(dq, q_rows), sq, tol(w), "dQ rows")
    assert_close(at(dk, k_cols), sk, tol(w), "dK cols")
    assert_close(at(dv, k_cols), sv, tol(w), "dV cols")


def test_max_heads_fwd_bwd():
    """num_heads x head_dim at the plan's limit (2^20: 8192 heads of width
    128), the longest rows the 32-bit tile offsets cover: sampled O, LSE and
    dQ rows and dK, dV columns for heads at both ends of the row."""
    w = dataclasses.replace(W[4], n_tokens=200, heads=8192, window=0, doc_range=None, batch=1,
                            backward=True)
    inp = wl.tensors(w, seed=31, with_grad=True)
    inp["cu"] = np.array([0, 200], np.int32)
    say("fwd+bwd at 8192 heads x 128")
    _, _, qt, kt = oracle_rotated(w, inp)
    plan = make_plan(w, inp["cu"])
    q, k, v, do = qt.cuda(), kt.cuda(), inp["v"].cuda(), inp["do"].cuda()
    o, lse = tca.attn_fwd(plan, q, k, v)
    dq, dk, dv = tca.attn_bwd(plan, q, k, v, o, lse, do)
    torch.cuda.synchronize()
    rows = [(j, s) for j in (0, 1, 4095, 8191) for s in (0, 1, 63, 64, 127, 128, 199)]
    o_ref, lse_ref = oracle.attn_fwd_rows(f64(qt), f64(kt), f64(inp["v"]), inp["cu"], rows, 0, 1, 0,
                                          w.scale)
    sq, sk, sv = oracle.attn_bwd_sampled(f64(qt), f64(kt), f64(inp["v"]), f64(inp["do"]),
                                         inp["cu"], rows, rows, 0, 1, 0, w.scale)
    pick = lambda x: np.stack([x[s, j].cpu().double().numpy() for j, s in rows])
    assert_close(pick(o), o_ref, tol(w), "O rows")
    assert_close(np.array([lse[j, s].item() for j, s in rows]), lse_ref, LSE_TOL, "LSE rows")
    assert_close(pick(dq), sq, tol(w), "dQ rows")
    assert_close(pick(dk), sk, tol(w), "dK cols")
    assert_close(pick(dv), sv, tol(w), "dV cols")


def test_bwd_deterministic():
    w = dataclasses.replace(W[4].scaled(3000, doc_range=(300, 1400)), backward=True)
    inp = wl.generate(w, with_grad=True)
    _, _, qt, kt = oracle_rotated(w, inp)
    a = gpu_fwd_bwd(w, inp, qt, kt)
    b = gpu_fwd_bwd(w, inp, qt, kt)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_bwd_fp32_is_unsupported():
    w = W[1]
    inp = wl.generate(w, with_grad=True)
    plan = make_plan(w, inp["cu"])
    q = inp["q"].cuda()
    lse = torch.empty((w.heads, w.n_tokens), device="cuda")
    with pytest.raises(tca.AttnError) as e:
        tca.attn_bwd(plan, q, q, q, q, lse, q,
                     *(torch.empty(q.shape, device="cuda") for _ in range(3)))
    assert e.value.status == -2


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_non_causal_varlen(d):
    """causal = 0: every key of a query's sequence is visible (ragged lengths,
    an empty and a one-token sequence), forward and backward against the
    oracle."""
    cu = [0, 90, 90, 91, 300, 557]
    w = dataclasses.replace(W[5], n_tokens=cu[-1], heads=2, head_dim=d, causal=0, window=0,
                            rope=1, doc_range=None, batch=1)
    inp = wl.tensors(w, seed=41, with_grad=True)
    inp["cu"] = np.array(cu, np.int32)
    say(f"non-causal varlen fwd+bwd d{d}")
    _, _, qt, kt = oracle_rotated(w, inp)
    plan = make_plan(w, inp["cu"])
    q, k, v, do = qt.cuda(), kt.cuda(), inp["v"].cuda(), inp["do"].cuda()
    o, lse = tca.attn_fwd(plan, q, k, v)
    dq, dk, dv = tca.attn_bwd(plan, q, k, v, o, lse, do)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(f64(qt), f64(kt), f64(inp["v"]), inp["cu"], 0, 0, 0,
                                     w.scale)
    assert_close(o.cpu().double().numpy(), o_ref, tol(w), "O")
    assert_close(lse.cpu().double().numpy(), lse_ref, LSE_TOL, "LSE")
    ref = oracle_bwd(w, inp, qt, kt)
    for g, r, n in zip((dq, dk, dv), ref, ("dQ", "dK", "dV")):
        assert_close(g.cpu().double().numpy(), r, tol(w), n)
