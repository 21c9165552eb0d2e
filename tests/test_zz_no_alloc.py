"""attn_bwd_noalloc (the backward with its scratch in the library's static
device array) through the C ABI against attn_bwd on the same inputs: two
calls in a row, the second on a smaller problem; plus the size limit."""
import ctypes
import dataclasses

import numpy as np
import pytest
import torch

import transformer_causal_self_amd as tca
from transformer_causal_self_amd import workloads as wl
from parity import make_plan, say

pytestmark = pytest.mark.gpu


def run_both(w, seed):
    inp = wl.generate(w, seed=seed, with_grad=True)
    plan = make_plan(w, inp["cu"])
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "do"))
    o, lse = tca.attn_fwd(plan, q, k, v)
    ref = tca.attn_bwd(plan, q, k, v, o, lse, do)
    out = tuple(torch.full_like(x, float("nan")) for x in ref)
    lib = tca.load_library()
    st = lib.attn_bwd_noalloc(plan.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                              o.data_ptr(), lse.data_ptr(), do.data_ptr(), out[0].data_ptr(),
                              out[1].data_ptr(), out[2].data_ptr(),
                              torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0, tca.STATUS.get(st)
    return ref, out


def test_noalloc_backward_matches_attn_bwd_twice():
    big = dataclasses.replace(wl.WORKLOADS[5].scaled(3000), heads=8)
    small = dataclasses.replace(wl.WORKLOADS[4].scaled(700, doc_range=(100, 400)),
                                backward=True, heads=2)
    for name, w, seed in (("T=3000 H=8 d=64", big, 51), ("varlen N=700 H=2 d=128", small, 52)):
        say(f"noalloc backward vs attn_bwd: {name}")
        ref, out = run_both(w, seed)
        for r, g, n in zip(ref, out, ("dQ", "dK", "dV")):
            assert torch.equal(r, g), n


def test_noalloc_rejects_a_problem_beyond_its_scratch():
    # 16 heads x 600 000 slots x 4 bytes = 38.4 MB > 32 MiB: rejected before any launch
    N = 600_000
    plan = tca.attn_plan_create(N, 16, 64, "bf16", [0, N], causal=1, rope="half").bind("cuda")
    x = torch.zeros(64, dtype=torch.float32, device="cuda")
    lib = tca.load_library()
    p = x.data_ptr()
    st = lib.attn_bwd_noalloc(plan.handle, p, p, p, p, p, p, p, p, p, None)
    assert st == -4
