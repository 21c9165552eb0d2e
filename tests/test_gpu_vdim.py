"""GPU parity with a value width dv different from the query/key width d ("Paired
Head Attention" article, section "Source 1: model configuration": each
attention module has its own qk_dim and v_dim) against the fp64 oracle, which
takes dv as a dimension of its own.  V, O, dO and dV rows carry dv elements;
Q, K, dQ, dK keep d.  The rotary pass copies V rows of dv elements (adjacent
pairing, FP8 inputs); attention and its backward contract over d for the
scores and over dv for the value products.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import transformer_causal_self_amd as tca
from transformer_causal_self_amd import workloads as wl
from parity import (LSE_TOL, assert_close, f64, from_slot_layout, make_plan, oracle_rotated,
                    sample_rows, say, slot_to_token, to_slot_layout, tol)

pytestmark = pytest.mark.gpu

W = wl.WORKLOADS

CASES = [
    ("d64 dv128 causal two docs", dataclasses.replace(W[5], n_tokens=1500, heads=4, batch=2,
                                                       v_dim=128)),
    ("d128 dv64 window 700 varlen", dataclasses.replace(W[4].scaled(2000, doc_range=(300, 900)),
                                                         window=700, v_dim=64)),
    ("d64 dv128 paired window 128 varlen",
     dataclasses.replace(W[3].scaled(1600, doc_range=(100, 700)), head_dim=64, v_dim=128)),
    ("d64 dv128 adjacent pairing H4", dataclasses.replace(W[5], n_tokens=700, heads=4, paired=2,
                                                           v_dim=128)),
    ("d64 dv128 grouped Hkv2", dataclasses.replace(W[5], n_tokens=900, heads=6, kv_heads=2,
                                                    v_dim=128)),
    ("d128 dv64 window 300 (short-window items)",
     dataclasses.replace(W[4].scaled(1200, doc_range=(200, 700)), window=300, v_dim=64)),
]
IDS = [c[0] for c in CASES]


def oracle_fwd(w, inp, qt, kt):
    if w.kv_heads:
        return oracle.attn_fwd_gqa(f64(qt), f64(kt), f64(inp["v"]), inp["cu"], w.causal,
                                   w.window, w.scale)
    return oracle.attn_fwd(f64(qt), f64(kt), f64(inp["v"]), inp["cu"], w.paired, w.causal,
                           w.window, w.scale)


def oracle_bwd(w, inp, qt, kt):
    if w.kv_heads:
        return oracle.attn_bwd_gqa(f64(qt), f64(kt), f64(inp["v"]), f64(inp["do"]), inp["cu"],
                                   w.causal, w.window, w.scale)
    return oracle.attn_bwd(f64(qt), f64(kt), f64(inp["v"]), f64(inp["do"]), inp["cu"], w.paired,
                           w.causal, w.window, w.scale)


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_vdim_rope_and_forward(case):
    name, w = case
    inp = wl.generate(w)
    say(f"v_dim forward {name}")
    plan = make_plan(w, inp["cu"])
    H, Hk = w.heads, w.kv_heads or w.heads
    q, k, v = inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda()
    if w.paired == 2:
        q2, k2, v2 = tca.rope_qkv(plan, q, k, v, v_out=torch.empty_like(v))
        assert torch.equal(from_slot_layout(v2.cpu(), Hk, 2), inp["v"])
    else:
        q2, k2 = tca.rope_qkv(plan, q, k)
        v2 = v
    o, lse = tca.attn_fwd(plan, q2, k2, v2)
    torch.cuda.synchronize()
    qr, kr, qt, kt = oracle_rotated(w, inp)
    assert tuple(o.shape) == (w.n_tokens, H, w.v_dim)
    assert_close(from_slot_layout(q2.cpu().double().numpy(), H, w.paired), qr, tol(w), "rope q")
    assert_close(from_slot_layout(k2.cpu().double().numpy(), Hk, w.paired), kr, tol(w), "rope k")
    o_ref, lse_ref = oracle_fwd(w, inp, qt, kt)
    assert_close(from_slot_layout(o.cpu().double().numpy(), H, w.paired), o_ref, tol(w), "O")
    assert_close(lse.cpu().double().numpy(), lse_ref, LSE_TOL, "LSE")


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_vdim_backward(case):
    name, w = case
    w = dataclasses.replace(w, backward=True)
    inp = wl.generate(w, with_grad=True)
    say(f"v_dim backward {name}")
    _, _, qt, kt = oracle_rotated(w, inp)
    plan = make_plan(w, inp["cu"])
    H, Hk = w.heads, w.kv_heads or w.heads
    q, k = to_slot_layout(qt, H, w.paired).cuda(), to_slot_layout(kt, Hk, w.paired).cuda()
    v = to_slot_layout(inp["v"], Hk, w.paired).cuda()
    do = to_slot_layout(inp["do"], H, w.paired).cuda()
    o, lse = tca.attn_fwd(plan, q, k, v)
    dq, dk, dv = tca.attn_bwd(plan, q, k, v, o, lse, do)
    torch.cuda.synchronize()
    assert tuple(dv.shape) == (w.n_tokens, Hk, w.v_dim)
    ref = oracle_bwd(w, inp, qt, kt)
    for g, r, n, h in zip((dq, dk, dv), ref, ("dQ", "dK", "dV"), (H, Hk, Hk)):
        assert_close(from_slot_layout(g.cpu().double().numpy(), h, w.paired), r, tol(w), n)


def test_vdim_rope_backward_and_fp8_value_rows():
    """rope_qkv_bwd moves dV rows of dv floats; rope_qkv_fp8 decodes V rows of dv
    codes (adjacent pairing, so both permute heads)."""
    w = dataclasses.replace(W[5], n_tokens=500, heads=4, paired=2, v_dim=128)
    inp = wl.fp8_tensors(w)
    say("v_dim rope backward and fp8")
    plan = make_plan(w, inp["cu"])
    _, _, v2 = tca.rope_qkv_fp8(plan, inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(),
                                inp["scales"])
    torch.cuda.synchronize()
    want = torch.from_numpy(oracle.dequant_fp8(inp["v"].numpy(), inp["scales"][2])).float()
    assert torch.equal(from_slot_layout(v2.cpu(), 4, 2), want.bfloat16())
    rng = np.random.default_rng(5)
    gq = torch.from_numpy(rng.standard_normal((500, 4, 64)).astype(np.float32))
    gv = torch.from_numpy(rng.standard_normal((500, 4, 128)).astype(np.float32))
    dq, dk, dv = tca.rope_qkv_bwd(plan, to_slot_layout(gq, 4, 2).cuda(),
                                  to_slot_layout(gq, 4, 2).cuda(),
                                  d_v=to_slot_layout(gv, 4, 2).cuda())
    torch.cuda.synchronize()
    assert torch.equal(dv.cpu(), gv)
    want_q = oracle.rope_bwd(gq.double().numpy(), inp["cu"], w.rope, w.rope_base, 2)
    assert_close(dq.cpu().double().numpy(), want_q, 1e-4, "dq")


def test_vdim_full_size_sampled():
    """The long causal problem's full size (16384 tokens, H = 12) with d = 64 and
    dv = 128, in the launch configuration the benchmark times: sampled rows."""
    w = dataclasses.replace(W[5], v_dim=128)
    inp = wl.generate(w, with_grad=False)
    say(f"v_dim full size N={w.n_tokens}")
    plan = make_plan(w, inp["cu"])
    q2, k2 = tca.rope_qkv(plan, inp["q"].cuda(), inp["k"].cuda())
    o, lse = tca.attn_fwd(plan, q2, k2, inp["v"].cuda())
    torch.cuda.synchronize()
    _, _, qt, kt = oracle_rotated(w, inp)
    rows = sample_rows(w, inp["cu"], np.random.default_rng(9))
    o_ref, lse_ref = oracle.attn_fwd_rows(f64(qt), f64(kt), f64(inp["v"]), inp["cu"], rows, 0,
                                          w.causal, w.window, w.scale)
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    for r, (j, s) in enumerate(rows):
        t, h = slot_to_token(s, j, w.heads, 0)
        assert_close(o[t, h], o_ref[r], tol(w), f"O row {(j, s)}")
        assert abs(lse[j, s] - lse_ref[r]) <= LSE_TOL
