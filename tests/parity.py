"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI and
the fp64 oracle on the same seeded host inputs, and compare.

Tolerances (stated once): max-abs 1e-4 for fp32 outputs, 2e-2 for outputs of
bf16 problems (the rotated Q', K', O, and the fp32-stored gradients of a bf16
problem, whose arithmetic is bf16 MFMA), and 1e-3 for the per-row softmax
statistic LSE.  Every comparison is against the unrounded fp64 oracle, except
that the oracle's rotated Q', K' are rounded to the problem's I/O type before
its attention, because rope_qkv stores them in that type and attention
consumes them from there.
"""
import sys

import numpy as np
import torch

import oracle
import transformer_causal_self_amd as tca
from transformer_causal_self_amd import workloads as wl

LSE_TOL = 1e-3


def tol(w):
    return 1e-4 if w.dtype == wl.DTYPE_FP32 else 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def make_plan(w, cu, device="cuda"):
    return tca.attn_plan_create(w.n_tokens, w.heads, w.head_dim,
                                "fp32" if w.dtype == wl.DTYPE_FP32 else "bf16", cu,
                                causal=w.causal, window=w.window, softmax_scale=w.scale,
                                rope=w.rope, rope_base=w.rope_base, paired=w.paired,
                                num_kv_heads=w.kv_heads, v_head_dim=w.v_dim).bind(device)


def f64(t):
    return t.double().numpy() if isinstance(t, torch.Tensor) else np.asarray(t, np.float64)


def oracle_rotated(w, inp):
    """Oracle RoPE (fp64) of Q and K, and the same rounded to the I/O type."""
    cu = inp["cu"]
    qr = oracle.rope(f64(inp["q"]), cu, w.rope, w.rope_base, w.paired)
    kr = oracle.rope(f64(inp["k"]), cu, w.rope, w.rope_base, w.paired)
    qt = torch.from_numpy(qr).to(w.torch_dtype)
    kt = torch.from_numpy(kr).to(w.torch_dtype)
    return qr, kr, qt, kt


def error_figures(got, want):
    """max-abs error; max-rel error over the elements with |want| >= 1e-3 of
    the largest |want| (smaller ones only measure cancellation); and the
    largest error of a row (last axis) divided by that row's RMS in the
    oracle (rows with an RMS below 1e-3 of the largest row RMS skipped)."""
    err = np.abs(got - want)
    if not err.size:
        return 0.0, 0.0, 0.0
    mag = np.abs(want)
    big = mag >= 1e-3 * mag.max() if mag.max() > 0 else np.zeros_like(mag, bool)
    rel = float((err[big] / mag[big]).max()) if big.any() else 0.0
    if want.ndim >= 2:
        rms = np.sqrt((want * want).mean(axis=-1))
        keep = rms >= 1e-3 * rms.max() if rms.max() > 0 else np.zeros_like(rms, bool)
        row = float((err.max(axis=-1)[keep] / rms[keep]).max()) if keep.any() else 0.0
    else:
        row = rel
    return float(err.max()), rel, row


def assert_close(got, want, bound, what, row_bound=None):
    """Element-by-element comparison against the oracle: the max-abs error must
    stay within `bound` (and, when given, every row's max error within
    `row_bound` times that row's RMS).  Prints max-abs, max-rel and the
    row-relative figure."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    m, rel, row = error_figures(got, want)
    say(f"  {what}: max-abs {m:.2e} (bound {bound:.0e}), max-rel {rel:.2e}, "
        f"max err / row RMS {row:.2e}")
    if m > bound:
        err = np.abs(got - want)
        idx = np.unravel_index(int(err.argmax()), err.shape)
        raise AssertionError(f"{what}: max-abs error {m:.3e} > {bound:.1e} at {idx} "
                             f"(got {got[idx]:.6f}, want {want[idx]:.6f})")
    if row_bound is not None and row > row_bound:
        raise AssertionError(f"{what}: a row's error is {row:.3e} of its RMS > {row_bound:.1e}")
    return m


def slot_to_token(s, j, H, paired):
    """Inverse of the paired slot map: (slot, attention head) -> (token, head)."""
    if not paired:
        return s, j
    if paired == 2:
        return s // 2, 2 * j + s % 2
    return s // 2, j + (s % 2) * (H // 2)


def adjacent_order(H):
    """Position of head h inside a token's row in the adjacent-pairing layout
    (slot 2t + h mod 2, attention head h // 2, read as [2N, H/2, d])."""
    return np.array([(h % 2) * (H // 2) + h // 2 for h in range(H)])


def to_slot_layout(x, H, paired):
    """[N, H, d] in head order -> the library's slot-layout memory."""
    if paired != 2:
        return x
    y = torch.empty_like(x)
    y[:, torch.from_numpy(adjacent_order(H))] = x
    return y


def from_slot_layout(x, H, paired):
    """Inverse of to_slot_layout (numpy or torch, [N, H, d])."""
    if paired != 2:
        return x
    return x[:, adjacent_order(H)]


def sample_rows(w, cu, rng, n_random=48):
    """(attention head, slot) rows: sequence starts and ends, tile edges, random."""
    mult = 2 if w.paired else 1
    Hs = w.heads // mult
    Ns = w.n_tokens * mult
    bounds = np.asarray(cu, np.int64) * mult
    rows = set()
    for b, e in list(zip(bounds[:-1], bounds[1:]))[:12]:
        if e > b:
            for s in (b, b + 1, e - 1, min(e - 1, b + 127), min(e - 1, b + 128)):
                rows.add((int(rng.integers(Hs)), int(s)))
    for s in rng.integers(0, Ns, n_random):
        rows.add((int(rng.integers(Hs)), int(s)))
    rows.add((Hs - 1, Ns - 1))
    return sorted(rows)
