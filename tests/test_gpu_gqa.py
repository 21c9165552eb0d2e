"""GPU parity of grouped-query attention (query heads in groups sharing one
K/V head; "Upgrading a textbook decoder", section 4 "GQA & FlashAttention")
against the fp64 oracle, which repeats the K/V heads as the page does and runs
its plain attention.  The GPU kernels index the shared K/V head instead of
copying it; dK and dV of a K/V head gather the whole group.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import transformer_causal_self_amd as tca
from transformer_causal_self_amd import workloads as wl
from parity import LSE_TOL, assert_close, f64, make_plan, say, tol

pytestmark = pytest.mark.gpu

W = wl.WORKLOADS

CASES = [
    ("H6 Hkv2 d64 causal two docs", dataclasses.replace(W[5], n_tokens=900, heads=6, kv_heads=2,
                                                         batch=2)),
    ("H8 Hkv1 d128 window 100 varlen", dataclasses.replace(
        W[4].scaled(2000, doc_range=(300, 900)), heads=8, kv_heads=1, window=100)),
    ("H12 Hkv4 d64 long causal", dataclasses.replace(W[5], n_tokens=1500, kv_heads=4)),
    ("H4 Hkv2 d128 window 700", dataclasses.replace(W[4].scaled(1600, doc_range=(500, 1200)),
                                                     heads=4, kv_heads=2, window=700)),
]
IDS = [c[0] for c in CASES]
FP32 = ("fp32 H6 Hkv3 d64", dataclasses.replace(W[1], n_tokens=300, heads=6, kv_heads=3))


def rotated(w, inp):
    cu = inp["cu"]
    qr = oracle.rope(f64(inp["q"]), cu, w.rope, w.rope_base, 0)
    kr = oracle.rope(f64(inp["k"]), cu, w.rope, w.rope_base, 0)
    return qr, kr, torch.from_numpy(qr).to(w.torch_dtype), torch.from_numpy(kr).to(w.torch_dtype)


@pytest.mark.parametrize("case", CASES + [FP32], ids=IDS + [FP32[0]])
def test_gqa_rope_and_forward(case):
    name, w = case
    inp = wl.generate(w)
    say(f"gqa forward {name}")
    plan = make_plan(w, inp["cu"])
    q2, k2 = tca.rope_qkv(plan, inp["q"].cuda(), inp["k"].cuda())
    o, lse = tca.attn_fwd(plan, q2, k2, inp["v"].cuda())
    torch.cuda.synchronize()
    qr, kr, qt, kt = rotated(w, inp)
    assert tuple(k2.shape) == (w.n_tokens, w.kv_heads, w.head_dim)
    assert_close(q2.cpu().double().numpy(), qr, tol(w), "rope q")
    assert_close(k2.cpu().double().numpy(), kr, tol(w), "rope k")
    o_ref, lse_ref = oracle.attn_fwd_gqa(f64(qt), f64(kt), f64(inp["v"]), inp["cu"], w.causal,
                                         w.window, w.scale)
    assert_close(o.cpu().double().numpy(), o_ref, tol(w), "O")
    assert_close(lse.cpu().double().numpy(), lse_ref, LSE_TOL, "LSE")


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_gqa_backward(case):
    name, w = case
    w = dataclasses.replace(w, backward=True)
    inp = wl.generate(w, with_grad=True)
    say(f"gqa backward {name}")
    _, _, qt, kt = rotated(w, inp)
    plan = make_plan(w, inp["cu"])
    q, k, v, do = qt.cuda(), kt.cuda(), inp["v"].cuda(), inp["do"].cuda()
    o, lse = tca.attn_fwd(plan, q, k, v)
    dq, dk, dv = tca.attn_bwd(plan, q, k, v, o, lse, do)
    torch.cuda.synchronize()
    assert tuple(dk.shape) == (w.n_tokens, w.kv_heads, w.head_dim)
    ref = oracle.attn_bwd_gqa(f64(qt), f64(kt), f64(inp["v"]), f64(inp["do"]), inp["cu"],
                              w.causal, w.window, w.scale)
    for g, r, n in zip((dq, dk, dv), ref, ("dQ", "dK", "dV")):
        assert_close(g.cpu().double().numpy(), r, tol(w), n)


def test_gqa_group_of_one_equals_mha():
    """num_kv_heads = H runs the ungrouped path: bit-identical to leaving it 0."""
    w = dataclasses.replace(W[5], n_tokens=700, heads=4)
    inp = wl.generate(w)
    outs = []
    for kvh in (0, 4):
        plan = make_plan(dataclasses.replace(w, kv_heads=kvh), inp["cu"])
        q2, k2 = tca.rope_qkv(plan, inp["q"].cuda(), inp["k"].cuda())
        o, lse = tca.attn_fwd(plan, q2, k2, inp["v"].cuda())
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_gqa_full_size_sampled():
    """The long-context shape (T = 16384, H = 12, d = 64) with 4 K/V heads, in
    the launch configuration the benchmark times; forward rows and backward
    rows/columns sampled, the oracle's dK/dV columns summed over the group."""
    w = dataclasses.replace(W[5], kv_heads=4)
    inp = wl.generate(w)
    say("gqa full long-context problem, 4 K/V heads")
    _, _, qt, kt = rotated(w, inp)
    plan = make_plan(w, inp["cu"])
    q, k, v, do = qt.cuda(), kt.cuda(), inp["v"].cuda(), inp["do"].cuda()
    o, lse = tca.attn_fwd(plan, q, k, v)
    dq, dk, dv = tca.attn_bwd(plan, q, k, v, o, lse, do)
    torch.cuda.synchronize()
    o, lse, dq, dk, dv = (x.cpu().double().numpy() for x in (o, lse, dq, dk, dv))
    rng = np.random.default_rng(12)
    T, H, G = w.n_tokens, w.heads, w.heads // w.kv_heads
    rows = [(int(rng.integers(H)), int(s)) for s in list(rng.integers(0, T, 24)) + [0, 1, T - 1]]
    o_ref, lse_ref = oracle.attn_fwd_rows_gqa(f64(qt), f64(kt), f64(inp["v"]), inp["cu"], rows)
    assert_close(np.stack([o[s, j] for j, s in rows]), o_ref, tol(w), "O rows")
    assert_close(np.array([lse[j, s] for j, s in rows]), lse_ref, LSE_TOL, "LSE rows")
    kv_cols = [(int(rng.integers(w.kv_heads)), int(s)) for s in
               list(rng.integers(0, T, 8)) + [0, T - 1]]
    k_cols = [(kh * G + g, s) for kh, s in kv_cols for g in range(G)]
    ek, ev = oracle.expand_kv(f64(kt), H), oracle.expand_kv(f64(inp["v"]), H)
    sq, sk, sv = oracle.attn_bwd_sampled(f64(qt), ek, ev, f64(inp["do"]), inp["cu"], rows,
                                         k_cols, 0, 1, 0, 0.0)
    assert_close(np.stack([dq[s, j] for j, s in rows]), sq, tol(w), "dQ rows")
    sk = sk.reshape(len(kv_cols), G, -1).sum(1)
    sv = sv.reshape(len(kv_cols), G, -1).sum(1)
    assert_close(np.stack([dk[s, kh] for kh, s in kv_cols]), sk, tol(w), "dK cols")
    assert_close(np.stack([dv[s, kh] for kh, s in kv_cols]), sv, tol(w), "dV cols")
