"""CPU tests of the C-ABI library: it loads, exports every declared entry point,
validates problems on the host, and its plan (work lists, exact counts) covers
every visible (query, key) pair exactly as the dense mask does.  No GPU call
is made here."""
import os
import re

import numpy as np
import pytest

import transformer_causal_self_amd as tca
from transformer_causal_self_amd import workloads as wl
import brute

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_mi355.h")


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"^(?:attn_status|size_t|const char|void)\s*\**\s*(\w+)\s*\(", text, re.M)


def test_header_declares_the_boundary():
    names = set(declared_functions())
    assert {"attn_plan_create", "attn_plan_workspace_bytes", "attn_plan_bind", "attn_plan_stats",
            "attn_plan_work_items", "rope_qkv", "rope_qkv_bwd", "attn_fwd", "attn_bwd",
            "attn_status_str",
            "attn_plan_destroy"} <= names


def test_library_exports_every_declared_symbol():
    lib = tca.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    lib = tca.load_library()
    for code in range(-6, 1):
        assert lib.attn_status_str(code)


def plan(**kw):
    args = dict(num_tokens=16, num_heads=2, head_dim=64, dtype="bf16", cu_seqlens=[0, 16],
                causal=1, window=0, rope="half", paired=0)
    args.update(kw)
    return tca.attn_plan_create(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(num_heads=3, paired=1), -1),                 # odd heads paired
    (dict(causal=0, window=4), -1),                    # window needs causal
    (dict(cu_seqlens=[0, 15]), -1),                    # does not end at N
    (dict(cu_seqlens=[1, 16]), -1),                    # does not start at 0
    (dict(cu_seqlens=[0, 10, 8, 16]), -1),             # decreasing
    (dict(num_tokens=-1, cu_seqlens=[0, -1]), -1),
    (dict(num_heads=0), -1),
    (dict(dtype=7), -1),
    (dict(rope=3), -1),
    (dict(rope_base=0.0), -1),
    (dict(softmax_scale=float("nan")), -1),
    (dict(softmax_scale=-1.0), -1),
    (dict(paired=3, num_heads=4), -1),
    (dict(paired=2, num_heads=3), -1),                 # odd heads, adjacent pairing
    (dict(num_heads=6, num_kv_heads=4), -1),           # K/V heads must divide H
    (dict(num_heads=6, num_kv_heads=-1), -1),
    (dict(num_heads=6, num_kv_heads=3, paired=1), -2), # grouped K/V heads are unpaired only
    (dict(qk_norm=2), -1),
    (dict(qk_norm=1, rope=0), -1),                     # the norm runs inside rope_qkv
    (dict(qk_norm=1, norm_eps=-1e-6), -1),
    (dict(head_dim=32), -2),                           # valid, not covered by the kernels
    (dict(head_dim=96), -2),
    (dict(v_head_dim=-64), -1),
    (dict(v_head_dim=63), -1),
    (dict(v_head_dim=96), -2),                         # value width not covered
    (dict(v_head_dim=128, dtype="fp32"), -2),          # separate value width: bf16 only
    (dict(num_heads=8194, head_dim=128), -2),          # tile offsets would pass 2^31
    (dict(num_heads=16386, head_dim=64, paired=1), -2),
    (dict(num_heads=16386, num_kv_heads=2, v_head_dim=128), -2),
])
def test_plan_rejects(kw, status):
    with pytest.raises(tca.AttnError) as e:
        plan(**kw)
    assert e.value.status == status


def test_head_count_limit_is_inclusive():
    assert plan(num_heads=8192, head_dim=128).info["attn_heads"] == 8192
    assert plan(num_heads=16384, head_dim=64).info["attn_heads"] == 16384


@pytest.mark.parametrize("d,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_value_width_counts(d, dv):
    p = plan(num_tokens=100, cu_seqlens=[0, 40, 100], head_dim=d, v_head_dim=dv)
    pairs = p.info["visible_pairs"]
    assert pairs == 2 * (40 * 41 // 2 + 60 * 61 // 2)
    assert p.info["v_head_dim"] == dv
    assert p.info["fwd_flops"] == 2 * (d + dv) * pairs
    assert p.info["bwd_flops"] == 2 * (3 * d + 2 * dv) * pairs
    # Q, K read and written by the rotary pass; V is not part of it
    assert p.info["rope_bytes"] == 2 * 2 * (100 * 2 * d) * 2
    # forward: Q, K, V read, O written (bf16), LSE written (fp32)
    assert p.info["fwd_bytes"] == 2 * 100 * 2 * (2 * d + 2 * dv) + 4 * 100 * 2
    assert plan(v_head_dim=0).info["v_head_dim"] == 64


def test_empty_problem_is_valid():
    p = plan(num_tokens=0, cu_seqlens=[0, 0])
    assert p.info["visible_pairs"] == 0
    assert p.info["fwd_items"] == 0
    assert p.workspace_bytes >= 256


def test_item_sizes_follow_the_dtype():
    # bf16: 256-query forward items at a head width of 128, 128-query ones at
    # widths of 64, 128-row backward dK/dV (keys) and dQ (queries) items;
    # fp32 (no backward): 128-query forward items and empty backward lists
    cu = [0, 2100]
    pb = plan(num_tokens=2100, cu_seqlens=cu)
    pb128 = plan(num_tokens=2100, cu_seqlens=cu, head_dim=128)
    pf = plan(num_tokens=2100, cu_seqlens=cu, dtype="fp32")
    rows = lambda p, which: np.diff(p.work_items(which)[:, 1:3], axis=1).max()
    assert rows(pb, 0) == 128 and rows(pb, 1) == 128 and rows(pb, 2) == 128
    assert rows(pb128, 0) == 256 and rows(pb128, 1) == 128 and rows(pb128, 2) == 128
    for d, dv in ((64, 128), (128, 64)):
        pm = plan(num_tokens=2100, cu_seqlens=cu, head_dim=d, v_head_dim=dv)
        assert rows(pm, 0) == 256 and rows(pm, 1) == 128 and rows(pm, 2) == 128
    assert rows(pf, 0) == 128
    # at width 128 a short window keeps 128-query forward items (a longer one
    # does not)
    wide = dict(num_tokens=2100, cu_seqlens=cu, head_dim=128)
    assert rows(plan(window=512, **wide), 0) == 128
    assert rows(plan(window=513, **wide), 0) == 256
    # so do problems whose sequences all have at most 2048 slots (paired: 1024 tokens)
    assert rows(plan(num_tokens=2048, cu_seqlens=[0, 2048], head_dim=128), 0) == 128
    assert rows(plan(num_tokens=2049, cu_seqlens=[0, 2049], head_dim=128), 0) == 256
    assert rows(plan(num_tokens=1025, cu_seqlens=[0, 1025], paired=1, head_dim=128), 0) == 256
    assert len(pf.work_items(1)) == 0 and len(pf.work_items(2)) == 0
    for bad in (-1, 3):
        with pytest.raises(tca.AttnError):
            pb.work_items(bad)


@pytest.mark.parametrize("H,Hkv,window", [(6, 2, 0), (8, 1, 100), (4, 4, 0)])
def test_grouped_kv_work_lists(H, Hkv, window):
    # forward, dQ and dK/dV items all run per query head (the dK/dV items of a
    # group add into their K/V head's rows); the query heads of a group are
    # interleaved so items reading the same K/V rows share an XCD (position i
    # runs on XCD i % 8)
    cu = list(range(0, 3073, 256)) + [3300]
    N = cu[-1]
    p = plan(num_tokens=N, num_heads=H, num_kv_heads=Hkv, cu_seqlens=cu, window=window)
    mask = brute.dense_mask(cu, 1, 1, window)
    assert p.info["kv_heads"] == Hkv and p.info["attn_heads"] == H
    assert p.info["visible_pairs"] == H * int(mask.sum())
    elems, kv = N * H * 64, N * Hkv * 64
    assert p.info["rope_bytes"] == 2 * (elems + kv) * 2
    for which, heads in ((0, H), (2, H), (1, H)):
        seen = np.zeros((heads, N), dtype=int)
        for head, r0, r1, *_ in p.work_items(which):
            seen[head, r0:r1] += 1
        assert (seen == 1).all(), which
    bwd = p.work_items(1)
    xcds = {}
    for i, it in enumerate(bwd):
        xcds.setdefault((int(it[5]), int(it[1])), set()).add(i % 8)
    # (the tail of the list borrows items across XCDs to balance load)
    assert sum(len(x) == 1 for x in xcds.values()) >= 0.6 * len(xcds)
    assert {int(it[0]) // (H // Hkv) for it in bwd if it[5] == bwd[0][5]} == {bwd[0][0] // (H // Hkv)}


def whole_items(fwd):
    """The forward list with the parts of every cut query tile joined back:
    checks that parts of one group share the head and query tile, number
    0..n-1 once each, hold consecutive partial slots, and tile the key range
    in part order without gaps or overlaps."""
    groups = {}
    whole = []
    for it in fwd:
        g, slot, pp = int(it[5]), int(it[6]), int(it[7])
        part, parts = pp >> 16, pp & 0xFFFF
        if g < 0:
            assert parts == 1 and part == 0
            whole.append(tuple(int(x) for x in it[:5]))
            continue
        assert parts >= 2 and 0 <= part < parts
        groups.setdefault(g, []).append((part, parts, slot, tuple(int(x) for x in it[:5])))
    slots = set()
    for g, ps in groups.items():
        ps.sort()
        assert [p[0] for p in ps] == list(range(ps[0][1]))
        assert len({p[1] for p in ps}) == 1
        first = ps[0][2]
        assert [p[2] for p in ps] == list(range(first, first + len(ps)))
        slots.update(p[2] for p in ps)
        items = [p[3] for p in ps]
        assert len({it[:3] for it in items}) == 1
        for a, b in zip(items, items[1:]):
            assert a[4] == b[3] and (b[3] - items[0][3]) % 64 == 0
        whole.append(items[0][:4] + (items[-1][4],))
    assert sorted(groups) == list(range(len(groups)))
    assert len(slots) == sum(len(ps) for ps in groups.values())
    return np.array(sorted(whole), dtype=np.int64).reshape(-1, 5)


def test_long_causal_forward_is_cut_and_balanced_one_is_not():
    # the schedule cuts the key range of the longest query tiles of a long
    # causal sequence into parts (the tail of a longest-first list of whole
    # tiles is the last query tile alone); a list that already balances stays
    # whole, and so does every fp32 list (its kernel has no merge)
    p = plan(num_tokens=16384, cu_seqlens=[0, 16384], num_heads=12)
    fwd = p.work_items(0)
    assert p.info["fwd_split_items"] > 0
    assert p.info["fwd_split_items"] == len({int(g) for g in fwd[:, 5] if g >= 0})
    whole = whole_items(fwd)
    assert len(whole) == 12 * 16384 // 128  # 128-query tiles at head width 64
    steps = (fwd[:, 4] - fwd[:, 3] + 63) // 64
    assert steps.max() < 256
    # many tiles of similar length over the whole chip: nothing to gain
    w = wl.WORKLOADS[4]
    q = plan(num_tokens=w.n_tokens, cu_seqlens=wl.cu_seqlens(w), num_heads=w.heads,
             head_dim=w.head_dim, window=w.window, rope="adjacent")
    assert q.info["fwd_split_items"] == 0 and (q.work_items(0)[:, 5] == -1).all()
    fp = plan(num_tokens=16384, cu_seqlens=[0, 16384], num_heads=12, dtype="fp32")
    assert fp.info["fwd_split_items"] == 0


def dense_pairs(cu, mult, causal, window):
    return int(brute.dense_mask(list(cu), mult, causal, window).sum())


CASES = [
    ([0, 300], 2, 0, 1, 0),
    ([0, 1, 64, 65, 193, 193, 322], 2, 0, 1, 0),      # tile-edge lengths and an empty doc
    ([0, 200, 450], 4, 1, 1, 0),
    ([0, 130, 400], 6, 1, 1, 128),
    ([0, 70, 271], 2, 0, 1, 64),
    ([0, 50, 300], 2, 0, 1, 1),
    ([0, 129, 300], 4, 1, 1, 129),
    ([0, 90, 300], 2, 0, 0, 0),
    ([0, 130, 400], 6, 2, 1, 128),                      # adjacent pairing: same slots
]


@pytest.mark.parametrize("cu,H,paired,causal,window", CASES)
def test_counts_and_work_lists_cover_the_mask(cu, H, paired, causal, window):
    N = cu[-1]
    p = plan(num_tokens=N, num_heads=H, cu_seqlens=cu, paired=paired, causal=causal,
             window=window)
    mult = 2 if paired else 1
    Hs = H // 2 if paired else H
    mask = brute.dense_mask(cu, mult, causal, window)
    assert p.info["visible_pairs"] == Hs * int(mask.sum())
    assert p.info["fwd_flops"] == 4 * 64 * p.info["visible_pairs"]
    assert p.info["slots"] == N * mult and p.info["attn_heads"] == Hs
    fwd = p.work_items(0)
    bwd = p.work_items(1)
    dq = p.work_items(2)
    # forward (128- or 256-query items for bf16) and dQ (256-query items): every
    # (head, query) row exactly once; its visible keys inside [k0, k1)
    bounds = np.array(cu) * mult
    def seq_of(slot):
        s = np.searchsorted(bounds, slot, side="right") - 1
        return bounds[s], bounds[s + 1]
    for lst, rows_max in ((whole_items(fwd), 256), (dq, 128)):
        seen = np.zeros((Hs, N * mult), dtype=int)
        for head, q0, q1, k0, k1, *_ in lst:
            assert 0 < q1 - q0 <= rows_max
            seen[head, q0:q1] += 1
            rows = mask[q0:q1]
            cols = np.nonzero(rows.any(axis=0))[0]
            assert cols.min() >= k0 and cols.max() < k1
            b, e = seq_of(q0)          # the item stays inside one sequence
            assert b <= q0 < q1 <= e and b <= k0 < k1 <= e
        assert (seen == 1).all()
    # backward: every (head, key) column exactly once; the queries that see it in [s0, s1)
    seen = np.zeros((Hs, N * mult), dtype=int)
    for head, r0, r1, s0, s1, *_ in bwd:
        assert 0 < r1 - r0 <= 128
        seen[head, r0:r1] += 1
        cols = mask[:, r0:r1]
        rows = np.nonzero(cols.any(axis=1))[0]
        assert rows.min() >= s0 and rows.max() < s1
        b, e = seq_of(r0)
        assert b <= r0 < r1 <= e and b <= s0 < s1 <= e
    assert (seen == 1).all()
    # XCD order: position i runs on XCD i % 8; a chunk of one stream's tiles
    # stays on one XCD unless borrowed at the tail, and each XCD runs its items
    # roughly longest first
    for lst, step in ((fwd, 64), (bwd, 64), (dq, 64)):
        steps = np.ceil((lst[:, 4] - lst[:, 3]) / step)
        if lst is not fwd:      # the backward lists carry the stream
            per_stream = {}
            for i, it in enumerate(lst):
                per_stream.setdefault(int(it[5]), set()).add(i % 8)
            n_streams = len(per_stream)
            assert n_streams == len({(int(a), int(b)) for a, b in zip(lst[:, 0], lst[:, 5])})
        for x in range(8):
            sub = steps[x::8]
            if len(sub) > 2:
                assert sub[0] >= np.median(sub)


@pytest.mark.parametrize("num,pairs", [(1, 33024), (2, 50380800), (5, 1610711040)])
def test_exact_visible_pairs_of_fixed_layouts(num, pairs):
    w = wl.WORKLOADS[num]
    cu = wl.cu_seqlens(w)
    p = plan(num_tokens=w.n_tokens, num_heads=w.heads, head_dim=w.head_dim,
             dtype="fp32" if w.dtype else "bf16", cu_seqlens=cu, paired=w.paired,
             window=w.window)
    assert p.info["visible_pairs"] == pairs
    assert p.info["fwd_flops"] == 4 * w.head_dim * pairs


@pytest.mark.parametrize("num", [3, 4])
def test_varlen_layouts_count_like_the_closed_form(num):
    w = wl.WORKLOADS[num]
    cu = wl.cu_seqlens(w)
    assert cu[0] == 0 and cu[-1] == w.n_tokens and (np.diff(cu) > 0).all()
    lens = np.diff(cu)
    lo, hi = w.doc_range
    assert (lens[:-1] >= lo).all() and (lens <= hi).all()
    p = plan(num_tokens=w.n_tokens, num_heads=w.heads, head_dim=w.head_dim, cu_seqlens=cu,
             paired=w.paired, window=w.window, rope="adjacent")
    mult = 2 if w.paired else 1
    Hs = w.heads // mult
    # sum over sequences of the per-row count min(i + 1, W), i = row inside the sequence
    total = 0
    for L in lens * mult:
        i = np.arange(L)
        total += int(np.minimum(i + 1, w.window).sum())
    assert p.info["visible_pairs"] == Hs * total


@pytest.mark.parametrize("window,same", [(2147483647, True), (1600, True), (1599, False)])
def test_window_spanning_every_sequence_is_no_window(window, same):
    # a window at least as long as the longest sequence (here 1600 slots)
    # hides no key: the plan drops it, so the kernels never add a huge window
    # to a slot index
    cu = [0, 700, 2300]
    a = plan(num_tokens=2300, cu_seqlens=cu, window=window)
    b = plan(num_tokens=2300, cu_seqlens=cu, window=0)
    if same:
        assert all(np.array_equal(a.work_items(i), b.work_items(i)) for i in range(3))
    assert (a.info["visible_pairs"] == b.info["visible_pairs"]) == same
    assert a.info["visible_pairs"] == 2 * int(brute.dense_mask(cu, 1, 1, window).sum())
