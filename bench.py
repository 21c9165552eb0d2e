"""Benchmark of the rotary causal self-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 5] [--paired P]
                    [--kv-heads G] [--v-dim DV] [--qk-norm] [--rope-bwd] [--fp8-inputs]
                    [--no-rows] [--no-cpu-baseline]

One step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM: rope_qkv (Q, K rotated), attn_fwd (O, LSE) and, for
the long-context problem, attn_bwd (dQ, dK, dV).  The plan (work lists and
rotary table) is built once per batch layout, before the timed region.

Printed: ONE JSON line.  `value` is the metric's quantity: attention-forward
TFLOP/s on causal FLOPs (the exact visible-pair FLOPs of attn_fwd, 2 (d + dv)
per pair, 4 d when dv = d, over the mean attn_fwd kernel time of the timed
steps).  `step_tflops` is the whole step's rate: forward plus backward FLOPs
(2 (3 d + 2 dv) per pair) over the step's wall time.  Per-kernel figures
(mean, median and min) come from HIP events recorded on the launch stream
around every launch of the timed steps.  Each kernel is held to the roofline
that binds it: rotary passes to HBM bandwidth, attention to the bf16 (or
fp32) MFMA peak when its FLOPs per algorithmic byte exceed the ridge point,
else to HBM bandwidth (short windows).  `roofline` is for the kernel that
takes the most time; every kernel's own roofline is under `kernels`.
`rows` (default run only) times rope_qkv and attn_fwd of the two varlen
problems (65536 tokens, 6 heads, d = 128: paired window 128, and window 2048)
with three input/output sets used in turn, so that each launch finds its data
outside the 256 MiB last-level cache: per launch (an event pair around each;
`frac` is from their median) and back to back (one event pair around the
run of launches, `*_back_to_back`, which pays the launch gap once).  `copy_gbs` is a plain 1 GiB device
copy (read + write bytes over its time), the practical HBM ceiling.
`cpu_baseline` times the fp64 oracle on a bounded sample of the same
workload on the host cores.
"""
import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 matrix / vector
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
METRIC = "attention fwd TFLOP/s (causal FLOPs) + % bf16 MFMA peak; rope_qkv HBM GB/s"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the rope_qkv / attn_fwd rows of the two varlen problems")
    ap.add_argument("--cpu-seconds", type=float, default=30.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--paired", type=int, choices=(0, 1, 2), default=None,
                    help="override the workload's head pairing (2: adjacent partner h^1, "
                         "where rope_qkv also copies V in the slot layout)")
    ap.add_argument("--kv-heads", type=int, default=None,
                    help="grouped-query attention: number of K/V heads (divides the heads)")
    ap.add_argument("--v-dim", type=int, default=None,
                    help="width of V, O and dO rows (64 or 128) when it differs from head_dim")
    ap.add_argument("--qk-norm", action="store_true",
                    help="RMS-normalise Q and K rows inside rope_qkv")
    ap.add_argument("--rope-bwd", action="store_true",
                    help="add rope_qkv_bwd (gradients back to the raw Q, K) to a backward step")
    ap.add_argument("--fp8-inputs", action="store_true",
                    help="Q, K, V arrive as e4m3 codes with per-tensor scales: the rotary "
                         "step is rope_qkv_fp8 (dequantise, rotate, bf16 Q', K', V')")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain device copy of known size (counter calibration)")
    return ap.parse_args()


def code_text(src):
    """A source file's code without comments, trailing blanks or empty lines:
    what the compiler sees, so that editing a comment does not change it."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in src.splitlines())
    return "\n".join(ln for ln in lines if ln)


def kernel_sources_digest(files=None):
    """Digest of the HIP sources' code (comments ignored), to tie stored
    counter readings to a kernel version.  `files` maps name -> text (default:
    the sources in the package's csrc directory)."""
    if files is None:
        csrc = os.path.join(ROOT, "transformer_causal_self_amd", "csrc")
        files = {}
        for name in sorted(os.listdir(csrc)):
            if name.endswith((".hip", ".h", ".cpp")):   # build by-products are not sources
                with open(os.path.join(csrc, name)) as f:
                    files[name] = f.read()
    h = hashlib.sha256()
    for name in sorted(files):
        h.update(name.encode() + code_text(files[name]).encode())
    return h.hexdigest()[:16]


def stored_traffic(kernel, workload, digest):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    r = rec.get(f"{kernel}@{workload}")
    if not r or r.get("sources") != digest:
        return None
    return r.get("bytes_per_launch")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def stats_ms(pairs):
    """mean, median and min of the elapsed times (ms) of (start, end) event pairs."""
    import numpy as np
    t = np.array([a.elapsed_time(b) for a, b in pairs])
    return float(t.mean()), float(np.median(t)), float(t.min())


def copy_gbs(dev, reps=5):
    """Read + write GB/s of a plain 1 GiB device-to-device copy (median of reps)."""
    import numpy as np
    import torch
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    ev = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    del src, dst
    return 2.0 * (1 << 30) / (ms * 1e-3) / 1e9


def varlen_rows(dev, reps=10, sets=3):
    """rope_qkv and attn_fwd of the two varlen problems, each launch on one of
    `sets` copies of its inputs and outputs in turn (the launch's data was last
    touched `sets - 1` launches earlier: beyond the last-level cache)."""
    import torch
    import transformer_causal_self_amd as tca
    from transformer_causal_self_amd import workloads as wl
    out = {}
    for num in (3, 4):
        w = wl.WORKLOADS[num]
        inp = wl.generate(w)
        plan = tca.attn_plan_create(w.n_tokens, w.heads, w.head_dim, "bf16", inp["cu"],
                                    causal=w.causal, window=w.window, softmax_scale=w.scale,
                                    rope=w.rope, rope_base=w.rope_base,
                                    paired=w.paired).bind(dev)
        info = plan.info
        base = {n: inp[n].to(dev) for n in ("q", "k", "v")}
        bufs = []
        for i in range(sets):
            q, k, v = (base[n] if i == 0 else base[n].clone() for n in ("q", "k", "v"))
            bufs.append(dict(q=q, k=k, v=v, q2=torch.empty_like(q), k2=torch.empty_like(k),
                             o=torch.empty_like(q),
                             lse=torch.empty((info["attn_heads"], info["slots"]),
                                             dtype=torch.float32, device=dev)))
        def launch(name, b):
            if name == "rope_qkv":
                tca.rope_qkv(plan, b["q"], b["k"], q_out=b["q2"], k_out=b["k2"])
            else:
                tca.attn_fwd(plan, b["q2"], b["k2"], b["v"], b["o"], b["lse"])

        ev = {"rope_qkv": [], "attn_fwd": []}
        for r in range(2 + reps):
            b = bufs[r % sets]
            for name in ev:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                launch(name, b)
                e1.record()
                if r >= 2:
                    ev[name].append((e0, e1))
        # the same launches back to back, one event pair around the run: the
        # launch gap that each single-launch event pair includes is paid once
        batch = {}
        for name in ev:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for r in range(reps):
                launch(name, bufs[r % sets])
            e1.record()
            batch[name] = (e0, e1)
        torch.cuda.synchronize()
        row = {"workload": w.name, "sets": sets, "reps": reps}
        for name in ev:
            mean, med, mn = stats_ms(ev[name])
            bt = batch[name][0].elapsed_time(batch[name][1]) / reps
            if name == "rope_qkv":
                by = info["rope_bytes"]
                row[name] = {"bound": "hbm", "gbs_median": by / (med * 1e-3) / 1e9,
                             "gbs_best": by / (mn * 1e-3) / 1e9,
                             "frac": by / (med * 1e-3) / 1e9 / PEAK_HBM_GBS,
                             "gbs_back_to_back": by / (bt * 1e-3) / 1e9,
                             "frac_back_to_back": by / (bt * 1e-3) / 1e9 / PEAK_HBM_GBS,
                             "ms_mean": mean, "ms_median": med, "ms_min": mn,
                             "ms_back_to_back": bt}
            else:
                fl, by = info["fwd_flops"], info["fwd_bytes"]
                if fl / by >= PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
                    row[name] = {"bound": "mfma", "tflops_median": fl / (med * 1e-3) / 1e12,
                                 "frac": fl / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
                else:
                    row[name] = {"bound": "hbm", "gbs_median": by / (med * 1e-3) / 1e9,
                                 "frac": by / (med * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                 "tflops_median": fl / (med * 1e-3) / 1e12}
                row[name].update(ms_mean=mean, ms_median=med, ms_min=mn, ms_back_to_back=bt)
        out[f"problem{num}"] = row
        del bufs, base, plan
        torch.cuda.empty_cache()
    return out


def cpu_baseline(w, inp, seconds, norm=False, fp8=None):
    """fp64 oracle on a bounded random sample of the forward's query rows (plus
    its RoPE of every token), scaled to causal TFLOP/s."""
    import numpy as np
    import oracle

    mult = 2 if w.paired else 1
    Hs, Ns = w.heads // mult, w.n_tokens * mult
    cu = inp["cu"]
    bounds = np.asarray(cu, np.int64) * mult

    def visible(s):
        k = np.searchsorted(bounds, s, side="right") - 1
        if not w.causal:
            return bounds[k + 1] - bounds[k]
        n = s - bounds[k] + 1
        return min(n, w.window) if w.window > 0 else n

    rng = np.random.default_rng(0)
    if fp8 is None:
        q = inp["q"].double().numpy()
        k = inp["k"].double().numpy()
        v = inp["v"].double().numpy()
    else:
        q, k, v = (oracle.dequant_fp8(fp8[n].numpy(), s)
                   for n, s in zip(("q", "k", "v"), fp8["scales"]))

    def rows_sample(nrows):
        return np.stack([rng.integers(0, Hs, nrows), rng.integers(0, Ns, nrows)], 1)

    def fwd_rows(qr, kr, rows):
        if w.kv_heads and w.kv_heads != w.heads:
            return oracle.attn_fwd_rows_gqa(qr, kr, v, cu, rows, w.causal, w.window, w.scale)
        return oracle.attn_fwd_rows(qr, kr, v, cu, rows, w.paired, w.causal, w.window, w.scale)

    # calibrate: the RoPE of every token is a fixed cost, rows scale linearly
    t0 = time.perf_counter()
    qr = oracle.qk_prep(q, cu, w.rope, w.rope_base, w.paired, norm)
    kr = oracle.qk_prep(k, cu, w.rope, w.rope_base, w.paired, norm)
    t_rope = time.perf_counter() - t0
    # each call has a fixed gather cost plus a per-row cost: two probe sizes
    t_probe = []
    for probe in (512, 2048):
        t0 = time.perf_counter()
        fwd_rows(qr, kr, rows_sample(probe))
        t_probe.append(time.perf_counter() - t0)
    per_row = max((t_probe[1] - t_probe[0]) / 1536, 1e-7)
    fixed = max(t_probe[0] - 512 * per_row, 0.0)
    n = int(min(Ns * Hs, max(512, (seconds - t_rope - fixed) / per_row)))

    rows = rows_sample(n)
    t0 = time.perf_counter()
    qr = oracle.qk_prep(q, cu, w.rope, w.rope_base, w.paired, norm)
    kr = oracle.qk_prep(k, cu, w.rope, w.rope_base, w.paired, norm)
    fwd_rows(qr, kr, rows)
    dt = time.perf_counter() - t0
    flops = sum(2.0 * (w.head_dim + (w.v_dim or w.head_dim)) * visible(int(s))
                for s in rows[:, 1])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"{n} random (head, query) rows of this workload's forward (causal FLOPs "
                      f"{flops / 1e9:.1f} GFLOP) plus the RoPE of every token, fp64, {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path runs on one GPU; across GPUs it would shard by attention head and by "
              "sequence, with no exchange)", file=sys.stderr)
        sys.exit(2)

    import torch
    import transformer_causal_self_amd as tca
    from transformer_causal_self_amd import workloads as wl

    w = wl.WORKLOADS[args.workload]
    if args.paired is not None:
        import dataclasses
        w = dataclasses.replace(w, paired=args.paired)
    if args.kv_heads is not None:
        import dataclasses
        w = dataclasses.replace(w, kv_heads=args.kv_heads)
    if args.v_dim is not None:
        import dataclasses
        w = dataclasses.replace(w, v_dim=args.v_dim)
    if args.fp8_inputs and (w.dtype != wl.DTYPE_BF16 or args.rope_bwd):
        sys.exit("--fp8-inputs needs a bf16 problem and no --rope-bwd")
    # V' is written when it must be in the slot layout, or dequantised from FP8
    copy_v = w.paired == 2 or args.fp8_inputs
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = wl.generate(w)
    plan = tca.attn_plan_create(w.n_tokens, w.heads, w.head_dim,
                                "fp32" if w.dtype == wl.DTYPE_FP32 else "bf16", inp["cu"],
                                causal=w.causal, window=w.window, softmax_scale=w.scale,
                                rope=w.rope, rope_base=w.rope_base, paired=w.paired,
                                num_kv_heads=w.kv_heads, qk_norm=int(args.qk_norm),
                                v_head_dim=w.v_dim).bind(dev)
    info = plan.info
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    fp8 = wl.fp8_tensors(w) if args.fp8_inputs else None
    if fp8 is not None:
        q8, k8, v8 = (fp8[n].to(dev) for n in ("q", "k", "v"))
    do = inp["do"].to(dev) if w.backward else None
    q2, k2 = torch.empty_like(q), torch.empty_like(k)
    v2 = torch.empty_like(v) if copy_v else v
    o = torch.empty((q.shape[0], q.shape[1], v.shape[2]), dtype=q.dtype, device=dev)
    lse = torch.empty((info["attn_heads"], info["slots"]), dtype=torch.float32, device=dev)
    grads = None
    def rope():
        if fp8 is not None:
            tca.rope_qkv_fp8(plan, q8, k8, v8, fp8["scales"], q_out=q2, k_out=k2, v_out=v2)
        elif copy_v:
            tca.rope_qkv(plan, q, k, v, q_out=q2, k_out=k2, v_out=v2)
        else:
            tca.rope_qkv(plan, q, k, q_out=q2, k_out=k2)

    rope()
    tca.attn_fwd(plan, q2, k2, v2, o, lse)
    if w.backward:
        grads = tuple(torch.empty(x.shape, dtype=torch.float32, device=dev) for x in (q, k, v))
        try:
            tca.attn_bwd(plan, q2, k2, v2, o, lse, do, *grads)
        except tca.AttnError as e:
            if e.status != -2:
                raise
            grads = None        # backward kernels not built into this library

    rope_bwd = args.rope_bwd and grads is not None
    if rope_bwd:
        raw_grads = (torch.empty_like(grads[0]), torch.empty_like(grads[1]))
        tca.rope_qkv_bwd(plan, grads[0], grads[1], q, k, dq_out=raw_grads[0],
                         dk_out=raw_grads[1])
    names = ["rope_qkv", "attn_fwd"] + (["attn_bwd"] if grads is not None else []) + (
        ["rope_qkv_bwd"] if rope_bwd else [])
    events = {n: [] for n in names}

    def step(record):
        def timed(name, fn):
            if record:
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                fn()
                b.record()
                events[name].append((a, b))
            else:
                fn()
        timed("rope_qkv", rope)
        timed("attn_fwd", lambda: tca.attn_fwd(plan, q2, k2, v2, o, lse))
        if grads is not None:
            timed("attn_bwd", lambda: tca.attn_bwd(plan, q2, k2, v2, o, lse, do, *grads))
        if rope_bwd:
            timed("rope_qkv_bwd", lambda: tca.rope_qkv_bwd(plan, grads[0], grads[1], q, k,
                                                            dq_out=raw_grads[0],
                                                            dk_out=raw_grads[1]))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps

    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    kern_stats = {n: stats_ms(events[n]) for n in names}
    kern_ms = {n: kern_stats[n][0] for n in names}
    digest = kernel_sources_digest()
    wname = f"problem{w.num}" + ("" if args.paired is None else f"-paired{w.paired}") + (
        "" if args.kv_heads is None else f"-kv{w.kv_heads}") + (
        "" if args.v_dim is None else f"-dv{w.v_dim}") + (
        "-qknorm" if args.qk_norm else "") + ("-fp8" if fp8 is not None else "")
    # rope_qkv algorithmic bytes: Q, K read and written (plus V when copied);
    # with FP8 inputs one byte read and two written per element of Q, K, V
    kvh = w.kv_heads or w.heads
    dv = w.v_dim or w.head_dim
    es = 2 if w.dtype == wl.DTYPE_BF16 else 4
    rope_bytes = info["rope_bytes"] + (2.0 * w.n_tokens * kvh * dv * es if copy_v else 0.0)
    if fp8 is not None:
        rope_bytes = 3.0 * w.n_tokens * ((w.heads + kvh) * w.head_dim + kvh * dv)
    # rope_qkv_bwd: fp32 gradients of Q', K' read and of Q, K written, plus the
    # raw Q, K read again for the norm's gradient
    qk_elems = info["rope_bytes"] / 2 / (2 if w.dtype == wl.DTYPE_BF16 else 4)
    rope_bwd_bytes = qk_elems * (8 + ((2 if w.dtype == wl.DTYPE_BF16 else 4) if args.qk_norm
                                      else 0))
    step_flops = info["fwd_flops"] + (info["bwd_flops"] if grads is not None else 0.0)
    kernels = {}
    peak_mm = PEAK_BF16_TFLOPS if w.dtype == wl.DTYPE_BF16 else PEAK_FP32_TFLOPS
    for n in names:
        t = kern_ms[n] * 1e-3
        if n in ("rope_qkv", "rope_qkv_bwd"):
            ach = (rope_bytes if n == "rope_qkv" else rope_bwd_bytes) / t / 1e9
            rl = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                  "frac": ach / PEAK_HBM_GBS}
        else:
            fl = info["fwd_flops"] if n == "attn_fwd" else info["bwd_flops"]
            by = info["fwd_bytes"] if n == "attn_fwd" else info["bwd_bytes"]
            # the roofline that binds: MFMA above the ridge point (peak FLOP/s
            # over peak bytes/s), HBM below it (short windows)
            if fl / by >= peak_mm * 1e12 / (PEAK_HBM_GBS * 1e9):
                ach = fl / t / 1e12
                rl = {"bound": "mfma", "achieved": ach, "peak": peak_mm, "unit": "TFLOP/s",
                      "frac": ach / peak_mm}
            else:
                ach = by / t / 1e9
                rl = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                      "frac": ach / PEAK_HBM_GBS, "tflops": fl / t / 1e12}
        rl["traffic"] = stored_traffic(n, wname, digest)
        rl["ms"] = kern_ms[n]
        rl["ms_median"], rl["ms_min"] = kern_stats[n][1], kern_stats[n][2]
        kernels[n] = rl
    dominant = max(names, key=lambda n: kern_ms[n])
    roof = {k2_: v_ for k2_, v_ in kernels[dominant].items() if not k2_.startswith("ms")}
    roof["kernel"] = dominant

    out = {
        "metric": METRIC,
        "value": info["fwd_flops"] / (kern_ms["attn_fwd"] * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == wl.DTYPE_BF16 else "fp32",
        "data": "synthetic (seeded N(0,1) Q, K, V, dO; fixed sequence layout"
                + ("; Q, K, V quantised to e4m3 per tensor)" if fp8 is not None else ")"),
        "config": {"workload": w.name, "tokens": w.n_tokens, "heads": w.heads,
                   "head_dim": w.head_dim, "sequences": len(inp["cu"]) - 1,
                   "window": w.window, "paired": w.paired, "v_copied_by_rope": copy_v,
                   "kv_heads": w.kv_heads or w.heads, "v_dim": dv,
                   "qk_norm": bool(args.qk_norm),
                   "inputs": "fp8 e4m3 + per-tensor scales" if fp8 is not None else "bf16",
                   "rope": {1: "half-split", 2: "adjacent"}.get(w.rope, "none"),
                   "step": "+".join(names), "parallelism": "single GPU"},
        "roofline": roof,
        "kernels": kernels,
        "fwd_frac_bf16_peak": info["fwd_flops"] / (kern_ms["attn_fwd"] * 1e-3) / 1e12 / peak_mm,
        "step_tflops": step_flops / (ms_step * 1e-3) / 1e12,
        "rope_gbs": kernels["rope_qkv"]["achieved"],
        "step_flops": step_flops,
        "visible_pairs": info["visible_pairs"],
        "kernel_sources": digest,
    }
    if not args.no_rows and args.workload == 5:
        out["rows"] = varlen_rows(dev)
    out["copy_gbs"] = copy_gbs(dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds, args.qk_norm, fp8)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
