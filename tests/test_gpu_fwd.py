"""GPU parity of rope_qkv and attn_fwd against the fp64 oracle, through the C ABI.

Sizes: every problem shape at a size the oracle finishes in seconds (several
tiles plus a ragged tail), the full sizes with sampled rows for attention and
every element for RoPE, and edge cases (sequence lengths around the tile
edges, empty sequences, windows of 1..129 slots, paired head counts 2/4/6).
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
REDUCED = {
    1: W[1],
    2: W[2].scaled(600, batch=2),                          # B=2, T=300
    3: W[3].scaled(3000, doc_range=(256, 1024)),
    4: W[4].scaled(6000, doc_range=(512, 2600)),
    5: W[5].scaled(1000),
}


def gpu_inputs(inp):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def run_rope(w, inp, plan):
    g = gpu_inputs(inp)
    q2, k2 = tca.rope_qkv(plan, g["q"], g["k"])
    torch.cuda.synchronize()
    return q2, k2


def check_rope(w, inp, q2, k2, qr, kr):
    t = tol(w)
    assert_close(q2.cpu().double().numpy(), qr, t, "rope q")
    assert_close(k2.cpu().double().numpy(), kr, t, "rope k")
    if w.dtype == wl.DTYPE_BF16:
        # and within one bf16 step of the exact rotation everywhere, up to the
        # absolute error of the fp32 cos/sin: results near zero come from
        # cancellation, where that error exceeds a bf16 step of the tiny
        # result.  The kernels form cos/sin of p = 64 hi + lo from two
        # fp32-rounded table rows by angle addition, within 1.3e-7 of the
        # exact values (checked over every position and column); with both
        # inputs of a pair below 8 in magnitude that adds at most
        # 2 * 8 * 1.3e-7 = 2.1e-6, and the rotation's own fp32 rounding less
        # than 1e-6, together below 2^-18.
        for got, want in ((q2, qr), (k2, kr)):
            g = got.cpu().float().numpy()
            ulp = np.spacing(np.abs(torch.from_numpy(want).to(torch.bfloat16).float().numpy())) \
                * 2 ** 16
            assert (np.abs(g - want) <= ulp + 2.0 ** -18).all()


@pytest.mark.parametrize("num", [1, 2, 3, 4, 5])
def test_rope_reduced(num):
    w = REDUCED[num]
    inp = wl.generate(w)
    say(f"rope reduced problem {num}: N={w.n_tokens} H={w.heads} d={w.head_dim}")
    plan = make_plan(w, inp["cu"])
    q2, k2 = run_rope(w, inp, plan)
    qr, kr, _, _ = oracle_rotated(w, inp)
    check_rope(w, inp, q2, k2, qr, kr)


@pytest.mark.parametrize("num", [2, 3, 4, 5])
def test_rope_full_size(num):
    w = W[num]
    inp = wl.generate(w, with_grad=False)
    say(f"rope full problem {num}: N={w.n_tokens}")
    plan = make_plan(w, inp["cu"])
    q2, k2 = run_rope(w, inp, plan)
    qr, kr, _, _ = oracle_rotated(w, inp)
    check_rope(w, inp, q2, k2, qr, kr)


def test_rope_strided_inplace_and_v_copy():
    """Packed [N, 3, H, d] input read with token strides, V densified in the same
    pass; then an in-place rotation of a dense tensor."""
    w = REDUCED[3]
    inp = wl.generate(w)
    plan = make_plan(w, inp["cu"])
    qkv = torch.stack([inp["q"], inp["k"], inp["v"]], dim=1).cuda()   # [N, 3, H, d]
    q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    v_out = torch.empty_like(inp["v"], device="cuda")
    q2, k2, v2 = tca.rope_qkv(plan, q, k, v, v_out=v_out)
    qd = inp["q"].cuda().contiguous()
    tca.rope_qkv(plan, qd, inp["k"].cuda(), q_out=qd)                 # in place
    torch.cuda.synchronize()
    qr, kr, _, _ = oracle_rotated(w, inp)
    check_rope(w, inp, q2, k2, qr, kr)
    assert torch.equal(v2.cpu(), inp["v"])
    assert torch.equal(qd.cpu(), q2.cpu())


def run_fwd(w, plan, q, k, v):
    o, lse = tca.attn_fwd(plan, q.cuda(), k.cuda(), v.cuda())
    torch.cuda.synchronize()
    return o.cpu().double().numpy(), lse.cpu().double().numpy()


def oracle_fwd(w, inp, qt, kt):
    return oracle.attn_fwd(f64(qt), f64(kt), f64(inp["v"]), inp["cu"], w.paired, w.causal,
                           w.window, w.scale)


@pytest.mark.parametrize("num", [1, 2, 3, 4, 5])
def test_fwd_reduced_isolated(num):
    """Attention alone, on the oracle's rotated (and I/O-rounded) Q', K'."""
    w = REDUCED[num]
    inp = wl.generate(w)
    say(f"fwd reduced problem {num}")
    plan = make_plan(w, inp["cu"])
    _, _, qt, kt = oracle_rotated(w, inp)
    o, lse = run_fwd(w, plan, qt, kt, inp["v"])
    o_ref, lse_ref = oracle_fwd(w, inp, qt, kt)
    assert_close(o, o_ref, tol(w), "O")
    assert_close(lse, lse_ref, LSE_TOL, "LSE")


@pytest.mark.parametrize("num", [1, 2, 3, 4, 5])
def test_fwd_reduced_end_to_end(num):
    """rope_qkv then attn_fwd on the GPU against oracle RoPE then attention."""
    w = REDUCED[num]
    inp = wl.generate(w)
    say(f"fwd end-to-end reduced problem {num}")
    plan = make_plan(w, inp["cu"])
    q2, k2 = run_rope(w, inp, plan)
    o, lse = tca.attn_fwd(plan, q2, k2, inp["v"].cuda())
    torch.cuda.synchronize()
    _, _, qt, kt = oracle_rotated(w, inp)
    o_ref, lse_ref = oracle_fwd(w, inp, qt, kt)
    assert_close(o.cpu().double().numpy(), o_ref, tol(w), "O")
    assert_close(lse.cpu().double().numpy(), lse_ref, LSE_TOL, "LSE")


@pytest.mark.parametrize("num", [2, 3, 4, 5])
def test_fwd_full_size_sampled(num):
    """The full problem in the same launch configuration the benchmark times;
    the oracle computes sampled rows one by one."""
    w = W[num]
    inp = wl.generate(w, with_grad=False)
    say(f"fwd full problem {num}: N={w.n_tokens}")
    plan = make_plan(w, inp["cu"])
    q2, k2 = run_rope(w, inp, plan)
    o, lse = tca.attn_fwd(plan, q2, k2, inp["v"].cuda())
    torch.cuda.synchronize()
    o = o.cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    _, _, qt, kt = oracle_rotated(w, inp)
    rows = sample_rows(w, inp["cu"], np.random.default_rng(num))
    o_ref, lse_ref = oracle.attn_fwd_rows(f64(qt), f64(kt), f64(inp["v"]), inp["cu"], rows,
                                          w.paired, w.causal, w.window, w.scale)
    got_o = np.stack([o[slot_to_token(s, j, w.heads, w.paired)] for j, s in rows])
    got_l = np.array([lse[j, s] for j, s in rows])
    assert_close(got_o, o_ref, tol(w), "O rows")
    assert_close(got_l, lse_ref, LSE_TOL, "LSE rows")


def test_fwd_full_size_every_row_of_two_heads():
    """The long causal problem at full size (T = 16384, H = 12, d = 64) in the
    benchmark's launch configuration (long query tiles cut into merged parts):
    every O row and LSE of the first and the last head against the oracle.
    Late rows have |O| near 0.01, so besides the absolute bound each row's
    largest error must stay within 5% of that row's RMS: a tile of keys read
    from the wrong V rows moves a late row by about a quarter of its RMS."""
    w = W[5]
    inp = wl.generate(w, with_grad=False)
    say("fwd full problem 5, heads 0 and 11, every row")
    plan = make_plan(w, inp["cu"])
    assert plan.info["fwd_split_items"] > 0
    q2, k2 = run_rope(w, inp, plan)
    o, lse = tca.attn_fwd(plan, q2, k2, inp["v"].cuda())
    torch.cuda.synchronize()
    o = o.cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    _, _, qt, kt = oracle_rotated(w, inp)
    for head in (0, w.heads - 1):
        rows = [(head, s) for s in range(w.n_tokens)]
        o_ref, lse_ref = oracle.attn_fwd_rows(f64(qt), f64(kt), f64(inp["v"]), inp["cu"], rows,
                                              w.paired, w.causal, w.window, w.scale)
        assert_close(o[:, head], o_ref, tol(w), f"O head {head}", row_bound=5e-2)
        assert_close(lse[head], lse_ref, LSE_TOL, f"LSE head {head}")


EDGE = [
    # name, H, d, dtype, cu, paired, window, rope
    ("tile-edge lengths", 2, 64, wl.DTYPE_BF16, [0, 1, 64, 127, 191, 319, 448, 577], 0, 0, 1),
    ("empty sequences", 4, 128, wl.DTYPE_BF16, [0, 0, 65, 65, 194, 194], 0, 0, 2),
    ("window 1", 2, 64, wl.DTYPE_BF16, [0, 300], 0, 1, 1),
    ("window 2", 2, 64, wl.DTYPE_BF16, [0, 130, 300], 0, 2, 1),
    ("window 64", 2, 128, wl.DTYPE_BF16, [0, 250, 400], 0, 64, 2),
    ("window 129", 2, 64, wl.DTYPE_BF16, [0, 500], 0, 129, 1),
    ("paired H2 window 128", 2, 128, wl.DTYPE_BF16, [0, 200, 333], 1, 128, 2),
    ("paired H4", 4, 64, wl.DTYPE_BF16, [0, 150, 290], 1, 0, 1),
    ("paired H6 window 129", 6, 128, wl.DTYPE_BF16, [0, 97, 301], 1, 129, 2),
    ("fp32 varlen window", 3, 128, wl.DTYPE_FP32, [0, 70, 200, 333], 0, 100, 2),
    ("fp32 paired", 4, 64, wl.DTYPE_FP32, [0, 129, 200], 1, 0, 1),
    ("single token", 2, 64, wl.DTYPE_BF16, [0, 1], 0, 0, 1),
    # at head width 128, windows past 512 slots over sequences past 2048
    # slots run the 256-query items of the bf16 kernel (shorter ones, and
    # every problem at width 64, run 128-query items)
    ("window 513", 2, 128, wl.DTYPE_BF16, [0, 2200], 0, 513, 1),
    ("window 513 d64", 2, 64, wl.DTYPE_BF16, [0, 2200], 0, 513, 1),
    ("paired H2 window 600", 2, 128, wl.DTYPE_BF16, [0, 300, 1400], 1, 600, 2),
    ("causal 2300 slots d64", 2, 64, wl.DTYPE_BF16, [0, 150, 2450], 0, 0, 1),
    ("causal 2049 slots d128", 2, 128, wl.DTYPE_BF16, [0, 2049], 0, 0, 2),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_fwd_edge_cases(case):
    name, H, d, dt, cu, paired, window, rope = case
    N = cu[-1]
    w = dataclasses.replace(W[2], n_tokens=N, heads=H, head_dim=d, dtype=dt, paired=paired,
                            window=window, rope=rope, doc_range=None, batch=1)
    inp = wl.tensors(w, seed=11)
    inp["cu"] = np.array(cu, np.int32)
    say(f"fwd edge case {name}")
    plan = make_plan(w, inp["cu"])
    q2, k2 = run_rope(w, inp, plan)
    o, lse = tca.attn_fwd(plan, q2, k2, inp["v"].cuda())
    torch.cuda.synchronize()
    qr, kr, qt, kt = oracle_rotated(w, inp)
    check_rope(w, inp, q2, k2, qr, kr)
    o_ref, lse_ref = oracle_fwd(w, inp, qt, kt)
    assert_close(o.cpu().double().numpy(), o_ref, tol(w), "O")
    assert_close(lse.cpu().double().numpy(), lse_ref, LSE_TOL, "LSE")


# problems whose plans cut long query tiles along their keys into parts that
# separate blocks run and the last of them merges (d = 64 and 128, GQA, a
# window longer than the cut, a separate value width)
CUT = [
    ("causal T=4000 H=2 d64", dataclasses.replace(W[5], n_tokens=4000, heads=2)),
    ("causal T=2500 H=2 d128", dataclasses.replace(W[5], n_tokens=2500, heads=2, head_dim=128,
                                                   rope=2)),
    ("GQA T=3000 H=4 Hkv=1", dataclasses.replace(W[5], n_tokens=3000, heads=4, kv_heads=1)),
    ("window 2500 T=4000", dataclasses.replace(W[5], n_tokens=4000, heads=2, window=2500)),
    ("dv 128 T=3000", dataclasses.replace(W[5], n_tokens=3000, heads=2, v_dim=128)),
]


@pytest.mark.parametrize("case", CUT, ids=[c[0] for c in CUT])
def test_fwd_cut_tiles(case):
    name, w = case
    w = dataclasses.replace(w, backward=False)
    inp = wl.generate(w)
    say(f"fwd with cut query tiles: {name}")
    plan = make_plan(w, inp["cu"])
    assert plan.info["fwd_split_items"] > 0
    _, _, qt, kt = oracle_rotated(w, inp)
    o, lse = run_fwd(w, plan, qt, kt, inp["v"])
    if w.kv_heads:
        o_ref, lse_ref = oracle.attn_fwd_gqa(f64(qt), f64(kt), f64(inp["v"]), inp["cu"], w.causal,
                                             w.window, w.scale)
    else:
        o_ref, lse_ref = oracle_fwd(w, inp, qt, kt)
    assert_close(o, o_ref, tol(w), "O", row_bound=5e-2)
    assert_close(lse, lse_ref, LSE_TOL, "LSE")


@pytest.mark.parametrize("w", [REDUCED[4], CUT[0][1]], ids=["varlen window", "cut tiles"])
def test_fwd_deterministic(w):
    """Bit-identical results on a second launch, also where the plan cuts
    query tiles into parts that merge in whichever order they finish."""
    inp = wl.generate(w)
    plan = make_plan(w, inp["cu"])
    q, k, v = inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda()
    o1, l1 = tca.attn_fwd(plan, q, k, v)
    o2, l2 = tca.attn_fwd(plan, q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fwd_rejects_unbound_and_misaligned():
    w = REDUCED[2]
    inp = wl.generate(w)
    plan = tca.attn_plan_create(w.n_tokens, w.heads, w.head_dim, "bf16", inp["cu"])
    lib = tca.load_library()
    assert lib.attn_fwd(plan.handle, 16, 16, 16, 16, 16, None) == -4   # not bound
    plan.bind("cuda")
    q = inp["q"].cuda()
    assert lib.attn_fwd(plan.handle, q.data_ptr() + 2, q.data_ptr(), q.data_ptr(),
                        q.data_ptr(), q.data_ptr(), None) == -3


@pytest.mark.parametrize("d", [64, 128])
def test_empty_problem_every_entry_point(d):
    """No tokens at all: a valid plan whose launches enqueue nothing and return
    OK, with zero-size (possibly NULL) buffers, for every entry point."""
    say(f"empty problem d{d}")
    plan = tca.attn_plan_create(0, 4, d, "bf16", [0, 0], causal=1, rope="half").bind("cuda")
    e = lambda *shape, dt=torch.bfloat16: torch.empty(shape, dtype=dt, device="cuda")
    q, k, v = e(0, 4, d), e(0, 4, d), e(0, 4, d)
    q2, k2, v2 = tca.rope_qkv(plan, q, k, v, v_out=e(0, 4, d))
    o, lse = tca.attn_fwd(plan, q2, k2, v2)
    dq, dk, dv = tca.attn_bwd(plan, q2, k2, v2, o, lse, e(0, 4, d))
    gq, gk = tca.rope_qkv_bwd(plan, dq, dk)[:2]
    torch.cuda.synchronize()
    for x in (q2, k2, v2, o, dq, dk, dv, gq, gk):
        assert x.shape[0] == 0
    assert lse.numel() == 0

