"""Python binding of libattn_mi355.so: rotary causal self-attention on MI355X.

Thin ctypes marshalling over the C ABI declared in include/attn_mi355.h; the
functions keep the C names (attn_plan_create, rope_qkv, attn_fwd, attn_bwd).
Every step of the computation runs in the library's gfx950 kernels; PyTorch
only provides device memory and the current stream.  There is no fallback:
if the library is missing or fails to load, every call raises.

Typical use::

    plan = attn_plan_create(num_tokens=N, num_heads=H, head_dim=d, dtype="bf16",
                            cu_seqlens=cu, causal=1, window=0, rope="half")
    plan.bind(device)                      # workspace + host-to-device copy
    q2, k2 = rope_qkv(plan, q, k)          # rotated Q', K' [N, H, d]
    o, lse = attn_fwd(plan, q2, k2, v)     # O [N, H, d], LSE [H', N']
    dq, dk, dv = attn_bwd(plan, q2, k2, v, o, lse, do)
"""
import ctypes
import os
from typing import Optional

import numpy as np
import torch

__all__ = ["AttnError", "Plan", "attn_plan_create", "rope_qkv", "attn_fwd", "attn_bwd",
           "library_path", "load_library"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libattn_mi355.so"

ATTN_BF16, ATTN_FP32 = 0, 1
ROPE = {"none": 0, "half": 1, "adjacent": 2, 0: 0, 1: 1, 2: 2}
STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported problem", -3: "misaligned pointer or stride",
          -4: "plan not bound or workspace too small", -5: "HIP runtime error",
          -6: "host allocation failed"}


class AttnError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {STATUS.get(status, 'unknown')} (status {status})")


class _Problem(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int64), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("cu_seqlens", ctypes.POINTER(ctypes.c_int32)), ("num_seqs", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("window", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("rope", ctypes.c_int32),
                ("rope_base", ctypes.c_double), ("paired", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("qk_norm", ctypes.c_int32),
                ("norm_eps", ctypes.c_float), ("v_head_dim", ctypes.c_int32)]


class _Info(ctypes.Structure):
    _fields_ = [("visible_pairs", ctypes.c_int64), ("fwd_flops", ctypes.c_double),
                ("bwd_flops", ctypes.c_double), ("rope_bytes", ctypes.c_double),
                ("fwd_bytes", ctypes.c_double), ("bwd_bytes", ctypes.c_double),
                ("fwd_items", ctypes.c_int64), ("bwd_items", ctypes.c_int64),
                ("slots", ctypes.c_int64), ("attn_heads", ctypes.c_int32),
                ("max_positions", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("v_head_dim", ctypes.c_int32), ("fwd_split_items", ctypes.c_int32)]


_lib = None


def library_path() -> str:
    return os.path.join(_HERE, LIB_NAME)


def load_library():
    """Load libattn_mi355.so (built by transformer_causal_self_amd/build.py)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: run `python -m transformer_causal_self_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.attn_plan_create.argtypes = [ctypes.POINTER(_Problem), ctypes.POINTER(vp)]
    lib.attn_plan_workspace_bytes.argtypes = [vp]
    lib.attn_plan_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_plan_bind.argtypes = [vp, vp, ctypes.c_size_t, vp]
    lib.attn_plan_stats.argtypes = [vp, ctypes.POINTER(_Info)]
    lib.attn_plan_work_items.argtypes = [vp, i32, ctypes.POINTER(i32), i64, ctypes.POINTER(i64)]
    lib.rope_qkv.argtypes = [vp, vp, i64, vp, i64, vp, i64, vp, vp, vp, vp]
    lib.rope_qkv_bwd.argtypes = [vp, vp, i64, vp, i64, vp, vp, vp, vp, vp, vp, vp]
    lib.rope_qkv_fp8.argtypes = [vp, vp, i64, vp, i64, vp, i64, ctypes.POINTER(ctypes.c_float),
                                 vp, vp, vp, vp]
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.attn_bwd_noalloc.argtypes = lib.attn_bwd.argtypes
    lib.attn_status_str.argtypes = [ctypes.c_int]
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_plan_destroy.argtypes = [vp]
    lib.attn_plan_destroy.restype = None
    for f in ("attn_plan_create", "attn_plan_bind", "attn_plan_stats", "attn_plan_work_items",
              "rope_qkv", "rope_qkv_bwd", "rope_qkv_fp8", "attn_fwd", "attn_bwd",
              "attn_bwd_noalloc"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(fn, status):
    if status != 0:
        raise AttnError(fn, status)


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


class Plan:
    """Host plan (owned by the library) plus its device workspace (owned here)."""

    def __init__(self, handle, problem: dict):
        self._h = ctypes.c_void_p(handle)
        self.problem = problem
        self.workspace: Optional[torch.Tensor] = None
        info = _Info()
        _check("attn_plan_stats", load_library().attn_plan_stats(self._h, ctypes.byref(info)))
        self.info = {f: getattr(info, f) for f, _ in _Info._fields_}

    @property
    def handle(self):
        return self._h

    @property
    def dtype(self):
        return torch.bfloat16 if self.problem["dtype"] == ATTN_BF16 else torch.float32

    @property
    def workspace_bytes(self) -> int:
        return load_library().attn_plan_workspace_bytes(self._h)

    def bind(self, device=None, stream=None):
        """Allocate the workspace on `device` and copy the plan into it."""
        device = torch.device(device if device is not None else "cuda")
        n = max(256, self.workspace_bytes)
        ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
        off = (-ws.data_ptr()) % 256
        self.workspace = ws
        self._ws_ptr = ws.data_ptr() + off
        st = stream if stream is not None else _stream(device)
        _check("attn_plan_bind", load_library().attn_plan_bind(self._h, self._ws_ptr, n, st))
        self.device = device
        return self

    def work_items(self, which: int) -> np.ndarray:
        lib = load_library()
        count = ctypes.c_int64()
        _check("attn_plan_work_items",
               lib.attn_plan_work_items(self._h, which, None, 0, ctypes.byref(count)))
        out = np.zeros((count.value, 8), dtype=np.int32)
        if count.value:
            _check("attn_plan_work_items",
                   lib.attn_plan_work_items(self._h, which,
                                            out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                            count.value, ctypes.byref(count)))
        return out

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.attn_plan_destroy(h)
            self._h = ctypes.c_void_p(None)


def attn_plan_create(num_tokens: int, num_heads: int, head_dim: int, dtype, cu_seqlens,
                     causal: int = 1, window: int = 0, softmax_scale: float = 0.0, rope="half",
                     rope_base: float = 10000.0, paired: int = 0,
                     num_kv_heads: int = 0, qk_norm: int = 0, norm_eps: float = 0.0,
                     v_head_dim: int = 0) -> Plan:
    if isinstance(dtype, str):
        dtype = {"bf16": ATTN_BF16, "fp32": ATTN_FP32}[dtype]
    elif isinstance(dtype, torch.dtype):
        dtype = ATTN_BF16 if dtype == torch.bfloat16 else ATTN_FP32
    cu = np.ascontiguousarray(np.asarray(cu_seqlens), dtype=np.int32)
    pr = _Problem(num_tokens=num_tokens, num_heads=num_heads, head_dim=head_dim, dtype=dtype,
                  cu_seqlens=cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                  num_seqs=len(cu) - 1, causal=causal, window=window,
                  softmax_scale=softmax_scale, rope=ROPE.get(rope, rope), rope_base=rope_base,
                  paired=paired, num_kv_heads=num_kv_heads, qk_norm=qk_norm, norm_eps=norm_eps,
                  v_head_dim=v_head_dim)
    h = ctypes.c_void_p()
    _check("attn_plan_create", load_library().attn_plan_create(ctypes.byref(pr), ctypes.byref(h)))
    problem = dict(num_tokens=num_tokens, num_heads=num_heads, head_dim=head_dim, dtype=dtype,
                   cu_seqlens=cu.copy(), causal=causal, window=window,
                   softmax_scale=softmax_scale, rope=ROPE.get(rope, rope), rope_base=rope_base,
                   paired=paired, num_kv_heads=num_kv_heads or num_heads, qk_norm=qk_norm,
                   norm_eps=norm_eps, v_head_dim=v_head_dim or head_dim)
    return Plan(h.value, problem)


def _token_stride(x: torch.Tensor, H: int, d: int) -> int:
    if x.dim() != 3 or x.shape[1] != H or x.shape[2] != d or x.stride(2) != 1 or x.stride(1) != d:
        raise ValueError(f"expected [N, {H}, {d}] with contiguous [H, d] rows, got "
                         f"{tuple(x.shape)} strides {x.stride()}")
    return x.stride(0)


def _need(plan: Plan, x: torch.Tensor, name: str, dtype=None, dense=True, kv=False, vd=False):
    """Check device, dtype and (dense) shape [N, H or Hkv (kv), d or dv (vd)]."""
    p = plan.problem
    heads = p["num_kv_heads"] if kv else p["num_heads"]
    width = p["v_head_dim"] if vd else p["head_dim"]
    if plan.workspace is None:
        raise AttnError(name, -4)
    if not x.is_cuda or x.device != plan.workspace.device:
        raise ValueError(f"{name} must be on {plan.workspace.device}")
    if x.dtype != (dtype or plan.dtype):
        raise ValueError(f"{name} must be {dtype or plan.dtype}, got {x.dtype}")
    if dense and (tuple(x.shape) != (p["num_tokens"], heads, width) or not x.is_contiguous()):
        raise ValueError(f"{name} must be contiguous [N, {'Hkv' if kv else 'H'}, "
                         f"{'dv' if vd else 'd'}]")


def rope_qkv(plan: Plan, q, k, v=None, q_out=None, k_out=None, v_out=None):
    """Rotate Q and K (and densify V if v_out is given).  Returns (q', k'[, v'])."""
    p = plan.problem
    H, Hkv, d = p["num_heads"], p["num_kv_heads"], p["head_dim"]
    for name, x in (("q", q), ("k", k)) + ((("v", v),) if v_out is not None else ()):
        _need(plan, x, name, dense=False)
    qs, ks = _token_stride(q, H, d), _token_stride(k, Hkv, d)
    vs = _token_stride(v, Hkv, p["v_head_dim"]) if v_out is not None else 0
    q_out = torch.empty((q.shape[0], H, d), dtype=q.dtype, device=q.device) if q_out is None else q_out
    k_out = torch.empty((k.shape[0], Hkv, d), dtype=k.dtype, device=k.device) if k_out is None \
        else k_out
    for name, x, kv in (("q_out", q_out, False), ("k_out", k_out, True)):
        _need(plan, x, name, kv=kv)
    if v_out is not None:
        _need(plan, v_out, "v_out", kv=True, vd=True)
    _check("rope_qkv", load_library().rope_qkv(
        plan.handle, q.data_ptr(), qs, k.data_ptr(), ks,
        v.data_ptr() if v_out is not None else None, vs, q_out.data_ptr(), k_out.data_ptr(),
        v_out.data_ptr() if v_out is not None else None, _stream(q.device)))
    return (q_out, k_out) if v_out is None else (q_out, k_out, v_out)


def rope_qkv_fp8(plan: Plan, q, k, v, scales, q_out=None, k_out=None, v_out=None):
    """rope_qkv on FP8 e4m3 inputs (uint8 codes or torch.float8_e4m3fn, [N, H, d] /
    [N, Hkv, d] rows) with per-tensor scales (q, k, v).  Returns bf16 (q', k', v')."""
    p = plan.problem
    H, Hkv, d = p["num_heads"], p["num_kv_heads"], p["head_dim"]
    codes = []
    for name, x in (("q", q), ("k", k), ("v", v)):
        if x.dtype == torch.float8_e4m3fn:
            x = x.view(torch.uint8)
        _need(plan, x, name, torch.uint8, dense=False)
        codes.append(x)
    q, k, v = codes
    dv = p["v_head_dim"]
    qs, ks, vs = _token_stride(q, H, d), _token_stride(k, Hkv, d), _token_stride(v, Hkv, dv)
    mk = lambda t, heads, w: torch.empty((q.shape[0], heads, w), dtype=torch.bfloat16,
                                         device=q.device) if t is None else t
    q_out, k_out, v_out = mk(q_out, H, d), mk(k_out, Hkv, d), mk(v_out, Hkv, dv)
    for name, x, kv, vd in (("q_out", q_out, False, False), ("k_out", k_out, True, False),
                            ("v_out", v_out, True, True)):
        _need(plan, x, name, kv=kv, vd=vd)
    sc = (ctypes.c_float * 3)(*[float(x) for x in scales])
    _check("rope_qkv_fp8", load_library().rope_qkv_fp8(
        plan.handle, q.data_ptr(), qs, k.data_ptr(), ks, v.data_ptr(), vs, sc,
        q_out.data_ptr(), k_out.data_ptr(), v_out.data_ptr(), _stream(q.device)))
    return q_out, k_out, v_out


def rope_qkv_bwd(plan: Plan, d_q, d_k, q=None, k=None, d_v=None, dq_out=None, dk_out=None,
                 dv_out=None):
    """Gradients with respect to rope_qkv's inputs (before the QK norm and the
    rotation), given float32 gradients of its outputs in the slot layout.
    q, k (the forward inputs) are needed when the plan normalises.  Returns
    (dq, dk[, dv]) float32 in head order."""
    p = plan.problem
    H, Hkv, d = p["num_heads"], p["num_kv_heads"], p["head_dim"]
    _need(plan, d_q, "d_q", torch.float32)
    _need(plan, d_k, "d_k", torch.float32, kv=True)
    if d_v is not None:
        _need(plan, d_v, "d_v", torch.float32, kv=True, vd=True)
    dq_out = torch.empty_like(d_q) if dq_out is None else dq_out
    dk_out = torch.empty_like(d_k) if dk_out is None else dk_out
    if d_v is not None and dv_out is None:
        dv_out = torch.empty_like(d_v)
    _need(plan, dq_out, "dq_out", torch.float32)
    _need(plan, dk_out, "dk_out", torch.float32, kv=True)
    if d_v is not None:
        _need(plan, dv_out, "dv_out", torch.float32, kv=True, vd=True)
    qs = ks = 0
    if p["qk_norm"]:
        if q is None or k is None:
            raise ValueError("the QK norm's backward needs the forward inputs q and k")
        _need(plan, q, "q", dense=False)
        _need(plan, k, "k", dense=False)
        qs, ks = _token_stride(q, H, d), _token_stride(k, Hkv, d)
    ptr = lambda t: t.data_ptr() if t is not None else None
    _check("rope_qkv_bwd", load_library().rope_qkv_bwd(
        plan.handle, ptr(q) if p["qk_norm"] else None, qs, ptr(k) if p["qk_norm"] else None, ks,
        d_q.data_ptr(), d_k.data_ptr(), ptr(d_v), dq_out.data_ptr(), dk_out.data_ptr(),
        ptr(dv_out) if d_v is not None else None, _stream(d_q.device)))
    return (dq_out, dk_out) if d_v is None else (dq_out, dk_out, dv_out)


def attn_fwd(plan: Plan, q, k, v, o=None, lse=None):
    """O [N, H, dv] (plan dtype) and LSE float32 [H', N']."""
    for name, x, kv, vd in (("q", q, False, False), ("k", k, True, False), ("v", v, True, True)):
        _need(plan, x, name, kv=kv, vd=vd)
    info = plan.info
    o = torch.empty((q.shape[0], q.shape[1], v.shape[2]), dtype=q.dtype, device=q.device) \
        if o is None else o
    lse = torch.empty((info["attn_heads"], info["slots"]), dtype=torch.float32,
                      device=q.device) if lse is None else lse
    _need(plan, o, "o", vd=True)
    _need(plan, lse, "lse", torch.float32, dense=False)
    if tuple(lse.shape) != (info["attn_heads"], info["slots"]) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [H', N']")
    _check("attn_fwd", load_library().attn_fwd(plan.handle, q.data_ptr(), k.data_ptr(),
                                               v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                               _stream(q.device)))
    return o, lse


def attn_bwd(plan: Plan, q, k, v, o, lse, do, dq=None, dk=None, dv=None, noalloc=False):
    """dQ float32 [N, H, d]; dK float32 [N, Hkv, d], dV float32 [N, Hkv, dv] (gradients
    with respect to the rotated q, k and v).  noalloc=True calls attn_bwd_noalloc (its
    scratch in the library's device array instead of the plan's workspace); pass
    dq, dk, dv to keep the call itself free of allocations."""
    for name, x, kv, vd in (("q", q, False, False), ("k", k, True, False), ("v", v, True, True),
                            ("o", o, False, True), ("do", do, False, True)):
        _need(plan, x, name, kv=kv, vd=vd)
    _need(plan, lse, "lse", torch.float32, dense=False)
    mk = lambda t, ref: torch.empty(ref.shape, dtype=torch.float32, device=q.device) \
        if t is None else t
    dq, dk, dv = mk(dq, q), mk(dk, k), mk(dv, v)
    for name, x, kv, vd in (("dq", dq, False, False), ("dk", dk, True, False),
                            ("dv", dv, True, True)):
        _need(plan, x, name, torch.float32, kv=kv, vd=vd)
    name = "attn_bwd_noalloc" if noalloc else "attn_bwd"
    _check(name, getattr(load_library(), name)(plan.handle, q.data_ptr(), k.data_ptr(),
                                               v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                               do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                               dv.data_ptr(), _stream(q.device)))
    return dq, dk, dv
