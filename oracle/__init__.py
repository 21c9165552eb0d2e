"""fp64 CPU oracle for rotary causal self-attention -- TEST INFRASTRUCTURE.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product library never loads it, and it shares no code with
the GPU path.  The arithmetic lives in oracle.c (plain C, fp64, OpenMP); this
module only marshals numpy arrays through ctypes.

All tensors are numpy float64 arrays of logical shape [N, H, d]; cu_seqlens is
an int32 array of S + 1 sequence boundaries.  LSE has shape [H', N'], where
H' = H/2 and N' = 2N when paired, else H and N.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I32 = ctypes.POINTER(ctypes.c_int32)
_I64 = ctypes.POINTER(ctypes.c_int64)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = _build.LIB
    if not os.path.exists(path) or (getattr(_build, "SRC_CHECK", True) and
                                    os.path.getmtime(path) < os.path.getmtime(_build.SRC)):
        _build.build()
    lib = ctypes.CDLL(path)
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_slot_map.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    _I64, ctypes.POINTER(ctypes.c_int)]
    lib.oracle_rope.argtypes = [_D, ctypes.c_int64, ctypes.c_int, ctypes.c_int, _I32, ctypes.c_int,
                                ctypes.c_int, ctypes.c_double, ctypes.c_int, _D]
    common = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, _I32, ctypes.c_int,
              ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double]
    lib.oracle_attn_fwd.argtypes = [_D, _D, _D] + common + [_D, _D]
    lib.oracle_attn_fwd_rows.argtypes = [_D, _D, _D] + common + [ctypes.c_int64, _I64, _D, _D]
    lib.oracle_attn_bwd.argtypes = [_D, _D, _D, _D] + common + [_D, _D, _D]
    lib.oracle_attn_bwd_sampled.argtypes = ([_D, _D, _D, _D] + common +
                                            [ctypes.c_int64, _I64, _D, ctypes.c_int64, _I64, _D, _D])
    lib.oracle_rope_bwd.argtypes = lib.oracle_rope.argtypes
    lib.oracle_rms_norm.argtypes = [_D, ctypes.c_int64, ctypes.c_int, ctypes.c_double, _D]
    lib.oracle_rms_norm_bwd.argtypes = [_D, _D, ctypes.c_int64, ctypes.c_int, ctypes.c_double, _D]
    for f in (lib.oracle_rope, lib.oracle_attn_fwd, lib.oracle_attn_fwd_rows,
              lib.oracle_attn_bwd, lib.oracle_attn_bwd_sampled, lib.oracle_rope_bwd,
              lib.oracle_rms_norm, lib.oracle_rms_norm_bwd):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _p(a, t=_D):
    return a.ctypes.data_as(t)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name} failed with status {rc}")


def num_threads() -> int:
    return _load().oracle_num_threads()


def slot_map(n: int, h: int, H: int, paired: int):
    """(slot, attention head) of logical token n, head h."""
    s = ctypes.c_int64()
    j = ctypes.c_int()
    _check(_load().oracle_slot_map(n, h, H, paired, ctypes.byref(s), ctypes.byref(j)), "slot_map")
    return s.value, j.value


def rope(x, cu, convention: int, base: float = 10000.0, paired: int = 0):
    """RoPE of x [N, H, d]; convention 1 = half-split, 2 = adjacent pairs."""
    x = _f64(x)
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    N, H, d = x.shape
    y = np.empty_like(x)
    _check(_load().oracle_rope(_p(x), N, H, d, _p(cu, _I32), len(cu) - 1, convention, base,
                               paired, _p(y)), "oracle_rope")
    return y


def rope_bwd(dy, cu, convention: int, base: float = 10000.0, paired: int = 0):
    """Transpose of rope: rotation by -phi at the same positions."""
    dy = _f64(dy)
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    N, H, d = dy.shape
    dx = np.empty_like(dy)
    _check(_load().oracle_rope_bwd(_p(dy), N, H, d, _p(cu, _I32), len(cu) - 1, convention, base,
                                   paired, _p(dx)), "oracle_rope_bwd")
    return dx


def rms_norm(x, eps: float = 1e-6):
    """x / sqrt(mean(x^2) + eps) over the last axis (no gain)."""
    x = _f64(x)
    y = np.empty_like(x)
    d = x.shape[-1]
    _check(_load().oracle_rms_norm(_p(x), x.size // d, d, eps, _p(y)), "oracle_rms_norm")
    return y


def rms_norm_bwd(x, dy, eps: float = 1e-6):
    """Gradient of rms_norm with respect to x."""
    x, dy = _f64(x), _f64(dy)
    dx = np.empty_like(x)
    d = x.shape[-1]
    _check(_load().oracle_rms_norm_bwd(_p(x), _p(dy), x.size // d, d, eps, _p(dx)),
           "oracle_rms_norm_bwd")
    return dx


def qk_prep(x, cu, convention: int, base: float = 10000.0, paired: int = 0, norm: bool = False,
            eps: float = 1e-6):
    """What rope_qkv makes of Q or K: the RMS-norm (when enabled), then RoPE."""
    return rope(rms_norm(x, eps) if norm else x, cu, convention, base, paired)


def qk_prep_bwd(x, dy, cu, convention: int, base: float = 10000.0, paired: int = 0,
                norm: bool = False, eps: float = 1e-6):
    """Gradient of qk_prep with respect to x, given the gradient dy of its output."""
    g = rope_bwd(dy, cu, convention, base, paired)
    return rms_norm_bwd(x, g, eps) if norm else g


def _heads(H, N, paired):
    return (H // 2, 2 * N) if paired else (H, N)


def _vdim(q, k, v):
    N, H, d = q.shape
    if k.shape != q.shape or v.ndim != 3 or v.shape[:2] != (N, H):
        raise ValueError("q, k must be [N, H, d] and v [N, H, dv]")
    return v.shape[2]


def attn_fwd(q, k, v, cu, paired=0, causal=1, window=0, scale=0.0):
    """O [N, H, dv] and LSE [H', N'] of softmax(scale q k^T + mask) v (q, k: [N, H, d])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    N, H, d = q.shape
    dv = _vdim(q, k, v)
    Hs, Ns = _heads(H, N, paired)
    o = np.empty((N, H, dv), dtype=np.float64)
    lse = np.empty((Hs, Ns), dtype=np.float64)
    _check(_load().oracle_attn_fwd(_p(q), _p(k), _p(v), N, H, d, dv, _p(cu, _I32), len(cu) - 1,
                                   paired, causal, window, scale, _p(o), _p(lse)),
           "oracle_attn_fwd")
    return o, lse


def attn_fwd_rows(q, k, v, cu, rows, paired=0, causal=1, window=0, scale=0.0):
    """Forward at selected (attention head, slot) rows: O rows [R, dv], LSE [R]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 2)
    N, H, d = q.shape
    dv = _vdim(q, k, v)
    o = np.empty((len(rows), dv), dtype=np.float64)
    lse = np.empty(len(rows), dtype=np.float64)
    _check(_load().oracle_attn_fwd_rows(_p(q), _p(k), _p(v), N, H, d, dv, _p(cu, _I32),
                                        len(cu) - 1, paired, causal, window, scale, len(rows),
                                        _p(rows, _I64), _p(o), _p(lse)), "oracle_attn_fwd_rows")
    return o, lse


def attn_bwd(q, k, v, dout, cu, paired=0, causal=1, window=0, scale=0.0):
    """dQ, dK [N, H, d] and dV [N, H, dv] of L = sum(O * dout)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    N, H, d = q.shape
    w = _vdim(q, k, v)
    if dout.shape != v.shape:
        raise ValueError("dout must be shaped like v")
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(v)
    _check(_load().oracle_attn_bwd(_p(q), _p(k), _p(v), _p(dout), N, H, d, w, _p(cu, _I32),
                                   len(cu) - 1, paired, causal, window, scale, _p(dq), _p(dk),
                                   _p(dv)), "oracle_attn_bwd")
    return dq, dk, dv


def attn_bwd_sampled(q, k, v, dout, cu, q_rows, k_cols, paired=0, causal=1, window=0, scale=0.0):
    """dQ at (head, slot) rows [R, d]; dK [C, d], dV [C, dv] at (head, slot) key columns."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    q_rows = np.ascontiguousarray(q_rows, dtype=np.int64).reshape(-1, 2)
    k_cols = np.ascontiguousarray(k_cols, dtype=np.int64).reshape(-1, 2)
    N, H, d = q.shape
    w = _vdim(q, k, v)
    if dout.shape != v.shape:
        raise ValueError("dout must be shaped like v")
    dq = np.empty((len(q_rows), d), dtype=np.float64)
    dk = np.empty((len(k_cols), d), dtype=np.float64)
    dv = np.empty((len(k_cols), w), dtype=np.float64)
    _check(_load().oracle_attn_bwd_sampled(_p(q), _p(k), _p(v), _p(dout), N, H, d, w,
                                           _p(cu, _I32),
                                           len(cu) - 1, paired, causal, window, scale,
                                           len(q_rows), _p(q_rows, _I64), _p(dq), len(k_cols),
                                           _p(k_cols, _I64), _p(dk), _p(dv)),
           "oracle_attn_bwd_sampled")
    return dq, dk, dv


# ------------------------------------------------------------ grouped query --
# "Upgrading a textbook decoder" (juejin.cn), section 4 "GQA & FlashAttention":
# the query heads form groups that share one K/V head; the module repeats each
# of the Hkv K/V heads H / Hkv times along the head axis (repeat_interleave) and
# then runs ordinary multi-head attention.  The oracle takes the same two
# steps: expand (a plain index copy), then the fp64 attention above.  The
# backward of the expansion sums the expanded heads' gradients over each group.

def expand_kv(x, H):
    """[N, Hkv, d] -> [N, H, d]: query head h reads K/V head h // (H / Hkv)."""
    x = _f64(x)
    Hkv = x.shape[1]
    if H % Hkv:
        raise ValueError("query heads must be a multiple of K/V heads")
    return np.repeat(x, H // Hkv, axis=1)


def attn_fwd_gqa(q, k, v, cu, causal=1, window=0, scale=0.0):
    """O [N, H, d], LSE [H, N] with K, V of shape [N, Hkv, d]."""
    H = np.shape(q)[1]
    return attn_fwd(q, expand_kv(k, H), expand_kv(v, H), cu, 0, causal, window, scale)


def attn_fwd_rows_gqa(q, k, v, cu, rows, causal=1, window=0, scale=0.0):
    """Forward at selected (query head, token) rows with K, V of shape [N, Hkv, d]."""
    H = np.shape(q)[1]
    return attn_fwd_rows(q, expand_kv(k, H), expand_kv(v, H), cu, rows, 0, causal, window, scale)


def attn_bwd_gqa(q, k, v, dout, cu, causal=1, window=0, scale=0.0):
    """dQ [N, H, d]; dK, dV [N, Hkv, d] (each K/V head gathers its group's gradients)."""
    H = np.shape(q)[1]
    N, Hkv, d = np.shape(k)
    dv = np.shape(v)[2]
    dq, dke, dve = attn_bwd(q, expand_kv(k, H), expand_kv(v, H), dout, cu, 0, causal, window,
                            scale)
    G = H // Hkv
    return dq, dke.reshape(N, Hkv, G, d).sum(axis=2), dve.reshape(N, Hkv, G, dv).sum(axis=2)


# ------------------------------------------------------------------ fp8 in --
# FP8 Q/K/V inputs ("Paired Head Attention", section 5 on the interplay with
# other mechanisms: in FP8 training the paired layers take Q/K/V from a packed
# FP8 projection).  The e4m3 format
# (OCP FP8, "fn" variant): sign bit, 4 exponent bits with bias 7, 3 mantissa
# bits; exponent field 0 gives subnormals m/8 * 2^-6; the code S.1111.111 is
# NaN; there is no infinity.  Decoded values are multiplied by a per-tensor
# scale.

def fp8_e4m3_decode(codes):
    """uint8 codes -> float64 values, from the format definition."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def dequant_fp8(codes, scale):
    """[N, H, d] uint8 e4m3 codes times the per-tensor scale (fp64)."""
    return fp8_e4m3_decode(codes) * float(scale)
