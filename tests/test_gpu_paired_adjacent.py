"""GPU parity of the adjacent pairing (partner h ^ 1: head h at slot
2t + (h mod 2), attention head h // 2) against the fp64 oracle, which maps the
pairing itself from its definition.  rope_qkv writes Q', K', V' in the slot
layout (heads of a token in the order 0, 2, 4, ..., 1, 3, 5, ...); attention
and its backward read and write that layout.  The tests move host tensors
between head order and slot order with a plain index permutation and compare
in head order.
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
ADJ = 2

CASES = [
    ("H6 window 128 d128 varlen",
     dataclasses.replace(W[3].scaled(3000, doc_range=(256, 1024)), paired=ADJ)),
    ("H4 causal d64 half-split",
     dataclasses.replace(W[5], n_tokens=700, heads=4, paired=ADJ)),
    ("H2 window 600 d128 two docs",
     dataclasses.replace(W[4], n_tokens=1000, heads=2, paired=ADJ, window=600,
                         doc_range=None, batch=2)),
]
IDS = [c[0] for c in CASES]


def rope_all(w, inp, plan):
    v_out = torch.empty_like(inp["v"], device="cuda")
    q2, k2, v2 = tca.rope_qkv(plan, inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(),
                              v_out=v_out)
    torch.cuda.synchronize()
    return q2, k2, v2


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_rope_adjacent(case):
    name, w = case
    inp = wl.generate(w)
    say(f"rope adjacent pairing {name}")
    plan = make_plan(w, inp["cu"])
    q2, k2, v2 = rope_all(w, inp, plan)
    qr, kr, _, _ = oracle_rotated(w, inp)
    H = w.heads
    assert_close(from_slot_layout(q2.cpu().double().numpy(), H, ADJ), qr, tol(w), "rope q")
    assert_close(from_slot_layout(k2.cpu().double().numpy(), H, ADJ), kr, tol(w), "rope k")
    # V is copied with the same head permutation, bit for bit
    assert torch.equal(from_slot_layout(v2.cpu(), H, ADJ), inp["v"])


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_fwd_adjacent_end_to_end(case):
    name, w = case
    inp = wl.generate(w)
    say(f"fwd adjacent pairing {name}")
    plan = make_plan(w, inp["cu"])
    q2, k2, v2 = rope_all(w, inp, plan)
    o, lse = tca.attn_fwd(plan, q2, k2, v2)
    torch.cuda.synchronize()
    _, _, qt, kt = oracle_rotated(w, inp)
    o_ref, lse_ref = oracle.attn_fwd(f64(qt), f64(kt), f64(inp["v"]), inp["cu"], ADJ, w.causal,
                                     w.window, w.scale)
    assert_close(from_slot_layout(o.cpu().double().numpy(), w.heads, ADJ), o_ref, tol(w), "O")
    assert_close(lse.cpu().double().numpy(), lse_ref, LSE_TOL, "LSE")


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_bwd_adjacent(case):
    name, w = case
    w = dataclasses.replace(w, backward=True)
    inp = wl.generate(w, with_grad=True)
    say(f"bwd adjacent pairing {name}")
    _, _, qt, kt = oracle_rotated(w, inp)
    H = w.heads
    plan = make_plan(w, inp["cu"])
    q, k, v, do = (to_slot_layout(x, H, ADJ).cuda() for x in (qt, kt, inp["v"], inp["do"]))
    o, lse = tca.attn_fwd(plan, q, k, v)
    dq, dk, dv = tca.attn_bwd(plan, q, k, v, o, lse, do)
    torch.cuda.synchronize()
    ref = oracle.attn_bwd(f64(qt), f64(kt), f64(inp["v"]), f64(inp["do"]), inp["cu"], ADJ,
                          w.causal, w.window, w.scale)
    for g, r, n in zip((dq, dk, dv), ref, ("dQ", "dK", "dV")):
        assert_close(from_slot_layout(g.cpu().double().numpy(), H, ADJ), r, tol(w), n)


def test_two_heads_adjacent_equals_memory_view():
    """With H = 2 the partner h ^ 1 is h + H/2: both pairings give the same
    slots, so the two GPU paths agree bit for bit."""
    w = dataclasses.replace(W[3].scaled(1500, doc_range=(200, 600)), heads=2)
    inp = wl.generate(w)
    outs = []
    for paired in (1, 2):
        wp = dataclasses.replace(w, paired=paired)
        plan = make_plan(wp, inp["cu"])
        q2, k2, v2 = rope_all(wp, inp, plan)
        o, lse = tca.attn_fwd(plan, q2, k2, v2)
        torch.cuda.synchronize()
        outs.append((q2.cpu(), k2.cpu(), o.cpu(), lse.cpu()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_adjacent_rope_needs_v_out_and_no_alias():
    w = dataclasses.replace(W[5], n_tokens=300, heads=4, paired=ADJ)
    inp = wl.generate(w)
    plan = make_plan(w, inp["cu"])
    q, k, v = inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda()
    with pytest.raises(tca.AttnError) as e:
        tca.rope_qkv(plan, q, k)                              # no v_out
    assert e.value.status == -1
    with pytest.raises(tca.AttnError) as e:
        tca.rope_qkv(plan, q, k, v, q_out=q, v_out=torch.empty_like(v))   # in place
    assert e.value.status == -1


def test_fwd_adjacent_full_size_sampled():
    """Problem 3's full size (65536 tokens, H = 6, d = 128, window 128) with the
    adjacent pairing, in the launch configuration the benchmark times."""
    w = dataclasses.replace(W[3], paired=ADJ)
    inp = wl.generate(w, with_grad=False)
    say(f"fwd adjacent pairing full size N={w.n_tokens}")
    plan = make_plan(w, inp["cu"])
    q2, k2, v2 = rope_all(w, inp, plan)
    o, lse = tca.attn_fwd(plan, q2, k2, v2)
    torch.cuda.synchronize()
    qr, kr, qt, kt = oracle_rotated(w, inp)
    H = w.heads
    assert_close(from_slot_layout(q2.cpu().double().numpy(), H, ADJ), qr, tol(w), "rope q")
    o = from_slot_layout(o.cpu().double().numpy(), H, ADJ)
    lse = lse.cpu().double().numpy()
    rows = sample_rows(w, inp["cu"], np.random.default_rng(33))
    o_ref, lse_ref = oracle.attn_fwd_rows(f64(qt), f64(kt), f64(inp["v"]), inp["cu"], rows,
                                          ADJ, w.causal, w.window, w.scale)
    got_o = np.stack([o[slot_to_token(s, j, H, ADJ)] for j, s in rows])
    got_l = np.array([lse[j, s] for j, s in rows])
    assert_close(got_o, o_ref, tol(w), "O rows")
    assert_close(got_l, lse_ref, LSE_TOL, "LSE rows")
