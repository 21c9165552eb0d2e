"""GPU parity of rope_qkv_fp8: FP8 e4m3 Q/K/V codes with per-tensor scales,
dequantised in the rotary kernel ("Paired Head Attention" article, section 5:
the FP8 packed-QKV path), against the fp64 oracle, which decodes every code
from the format's definition, scales it, and then runs the same QK norm and
rotation as for bf16 inputs.

V is only decoded, scaled and stored as bf16, so it is compared bit for bit
with the oracle's value rounded once to float32 (the product of a decoded
code and a float32 scale is exact in fp64) and then to bf16; Q' and K' keep
the 2e-2 bound of bf16 outputs.
"""
import ctypes
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import transformer_causal_self_amd as tca
from transformer_causal_self_amd import workloads as wl
from parity import LSE_TOL, assert_close, from_slot_layout, say, tol

pytestmark = pytest.mark.gpu

W = wl.WORKLOADS

CASES = [
    ("half d64 unpaired two docs", dataclasses.replace(W[5], n_tokens=900, batch=2)),
    ("adjacent d128 paired varlen window 128", W[3].scaled(2000, doc_range=(200, 900))),
    ("half d64 adjacent pairing H4", dataclasses.replace(W[5], n_tokens=700, heads=4, paired=2)),
    ("adjacent d128 grouped Hkv2 window 700",
     dataclasses.replace(W[4].scaled(1500, doc_range=(300, 800)), heads=6, kv_heads=2,
                         window=700)),
]
IDS = [c[0] for c in CASES]


def plan_of(w, cu, norm=False):
    return tca.attn_plan_create(w.n_tokens, w.heads, w.head_dim, "bf16", cu, causal=w.causal,
                                window=w.window, softmax_scale=w.scale, rope=w.rope,
                                rope_base=w.rope_base, paired=w.paired, num_kv_heads=w.kv_heads,
                                qk_norm=int(norm)).bind("cuda")


def dequant(codes, scale):
    return oracle.dequant_fp8(codes.numpy(), scale)


def v_expected(codes, scale):
    return torch.from_numpy(dequant(codes, scale)).float().bfloat16()


def prepared(w, inp, norm):
    """Oracle Q', K' (fp64, head order) and V (fp64) from the codes."""
    q = dequant(inp["q"], inp["scales"][0])
    k = dequant(inp["k"], inp["scales"][1])
    v = dequant(inp["v"], inp["scales"][2])
    prep = lambda x: oracle.qk_prep(x, inp["cu"], w.rope, w.rope_base, w.paired, norm, 1e-6)
    return prep(q), prep(k), v


def run(w, inp, plan):
    out = tca.rope_qkv_fp8(plan, inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(),
                           inp["scales"])
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("norm", [False, True], ids=["rope", "norm+rope"])
@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_fp8_rope(case, norm):
    name, w = case
    inp = wl.fp8_tensors(w)
    say(f"fp8 rope {name} norm={norm}")
    plan = plan_of(w, inp["cu"], norm)
    q2, k2, v2 = run(w, inp, plan)
    qr, kr, _ = prepared(w, inp, norm)
    H, Hk = w.heads, w.kv_heads or w.heads
    assert_close(from_slot_layout(q2.cpu().double().numpy(), H, w.paired), qr, tol(w), "q'")
    assert_close(from_slot_layout(k2.cpu().double().numpy(), Hk, w.paired), kr, tol(w), "k'")
    assert torch.equal(from_slot_layout(v2.cpu(), Hk, w.paired),
                       v_expected(inp["v"], inp["scales"][2]))


def test_fp8_every_code():
    """All 256 codes (both NaNs included) through the V path, at two scales."""
    w = dataclasses.replace(W[4], n_tokens=64, heads=4, doc_range=None, batch=1)
    say("fp8 every code")
    cu = np.array([0, 64], np.int32)
    plan = plan_of(w, cu)
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    v = codes.repeat(64 * 4 * 128 // 256).reshape(64, 4, 128)
    g = torch.Generator().manual_seed(11)
    q = torch.randint(0, 0x70, (64, 4, 128), generator=g, dtype=torch.uint8)
    for scale in (1.0, float(np.float32(0.37))):
        _, _, v2 = tca.rope_qkv_fp8(plan, q.cuda(), q.cuda(), v.cuda(), (1.0, 1.0, scale))
        torch.cuda.synchronize()
        got = v2.cpu().float()
        want = v_expected(v, scale).float()
        nan = torch.isnan(want)
        assert int(nan.sum()) == 2 * v.numel() // 256
        assert torch.equal(torch.isnan(got), nan)
        assert torch.equal(got[~nan], want[~nan]), f"scale {scale}"


@pytest.mark.parametrize("case", CASES[:3], ids=IDS[:3])
def test_fp8_inputs_end_to_end_forward(case):
    name, w = case
    inp = wl.fp8_tensors(w)
    say(f"fp8 end to end {name}")
    plan = plan_of(w, inp["cu"])
    q2, k2, v2 = run(w, inp, plan)
    o, lse = tca.attn_fwd(plan, q2, k2, v2)
    torch.cuda.synchronize()
    qr, kr, v = prepared(w, inp, False)
    bf = lambda x: torch.from_numpy(x).bfloat16().double().numpy()
    o_ref, lse_ref = oracle.attn_fwd(bf(qr), bf(kr), bf(v), inp["cu"], w.paired, w.causal,
                                     w.window, w.scale)
    assert_close(from_slot_layout(o.cpu().double().numpy(), w.heads, w.paired), o_ref, tol(w),
                 "O")
    assert_close(lse.cpu().double().numpy(), lse_ref, LSE_TOL, "LSE")


def test_fp8_strided_inputs():
    """Q, K, V as column slices of one packed [N, (H + 2 Hkv) d] code buffer."""
    w = dataclasses.replace(W[5], n_tokens=500, heads=6, kv_heads=2, batch=1)
    inp = wl.fp8_tensors(w)
    say("fp8 packed qkv slices")
    plan = plan_of(w, inp["cu"])
    N, d = w.n_tokens, w.head_dim
    packed = torch.cat([inp["q"].reshape(N, -1), inp["k"].reshape(N, -1),
                        inp["v"].reshape(N, -1)], dim=1).cuda()
    q = packed[:, :6 * d].view(N, 6, d)
    k = packed[:, 6 * d:8 * d].view(N, 2, d)
    v = packed[:, 8 * d:].view(N, 2, d)
    q2, k2, v2 = tca.rope_qkv_fp8(plan, q, k, v, inp["scales"])
    torch.cuda.synchronize()
    qr, kr, _ = prepared(w, inp, False)
    assert_close(q2.cpu().double().numpy(), qr, tol(w), "q'")
    assert_close(k2.cpu().double().numpy(), kr, tol(w), "k'")
    assert torch.equal(v2.cpu(), v_expected(inp["v"], inp["scales"][2]))


def test_fp8_rejects():
    say("fp8 rejects")
    OK, INVALID, UNSUPPORTED, ALIGN = 0, -1, -2, -3
    w = dataclasses.replace(W[5], n_tokens=64, heads=2)
    cu = np.array([0, 64], np.int32)
    plan = plan_of(w, cu)
    lib = tca.load_library()
    codes = torch.zeros((64, 2, 64), dtype=torch.uint8, device="cuda")
    outs = [torch.empty((64, 2, 64), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    c = codes.data_ptr()
    sc = lambda *v: (ctypes.c_float * 3)(*v)
    st = torch.cuda.current_stream().cuda_stream
    call = lambda qp, qs, scales, fp=plan: lib.rope_qkv_fp8(
        fp.handle, qp, qs, c, 128, c, 128, scales, *[o.data_ptr() for o in outs], st)
    assert call(c, 128, sc(1, 1, 1)) == OK
    assert call(c, 132, sc(1, 1, 1)) == ALIGN
    assert call(c + 4, 128, sc(1, 1, 1)) == ALIGN
    assert call(c, 64, sc(1, 1, 1)) == INVALID            # stride shorter than a row
    assert call(c, 128, sc(1, float("inf"), 1)) == INVALID
    assert call(c, 128, None) == INVALID
    fp32 = tca.attn_plan_create(64, 2, 64, "fp32", cu).bind("cuda")
    assert call(c, 128, sc(1, 1, 1), fp32) == UNSUPPORTED
    torch.cuda.synchronize()


def test_fp8_full_size():
    """Problem 4's full size (65536 tokens, H = 6, d = 128, ragged documents)
    with FP8 inputs, in the launch configuration the benchmark times."""
    w = W[4]
    inp = wl.fp8_tensors(w)
    say(f"fp8 rope full size N={w.n_tokens}")
    plan = plan_of(w, inp["cu"])
    q2, k2, v2 = run(w, inp, plan)
    qr, kr, _ = prepared(w, inp, False)
    assert_close(q2.cpu().double().numpy(), qr, tol(w), "q'")
    assert_close(k2.cpu().double().numpy(), kr, tol(w), "k'")
    assert torch.equal(v2.cpu(), v_expected(inp["v"], inp["scales"][2]))
