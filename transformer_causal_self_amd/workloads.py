"""Seeded synthetic workloads: the five problem shapes and their input generator.

This module holds no attention or rotary arithmetic.  It only draws random
numbers, so that the GPU path and the CPU oracle can consume the very same
host values.

Recipe (stated once, used everywhere):
  * sequence lengths: ``numpy.random.default_rng(seed).integers(lo, hi + 1)``
    drawn until the running total reaches N; the last length is clipped so the
    lengths sum to N exactly.  Fixed layouts (one sequence, or B equal
    sequences) are given directly.
  * tensors: ``torch.Generator().manual_seed(seed)``; ``randn`` in float32 of
    shape [N, H, d], drawn in the order Q, K, V, dO; cast to bfloat16 with
    round-to-nearest-even when the problem is bf16.
  * FP8 inputs (``fp8_tensors``): the same float32 draws for Q, K, V, each
    tensor divided by its scale amax / 448 (float32) and cast to
    ``torch.float8_e4m3fn`` (the codes and the scales are the inputs; the
    cast only draws them).
  * seed: the problem number 1..5 unless a test picks another.
"""
from dataclasses import dataclass, replace
from typing import Optional, Tuple

import numpy as np
import torch

ROPE_NONE, ROPE_HALF, ROPE_ADJACENT = 0, 1, 2
DTYPE_BF16, DTYPE_FP32 = 0, 1


@dataclass(frozen=True)
class Workload:
    name: str
    num: int                      # problem number, also the default seed
    dtype: int                    # DTYPE_BF16 or DTYPE_FP32
    n_tokens: int
    heads: int
    head_dim: int
    rope: int
    paired: int = 0
    kv_heads: int = 0             # K/V heads (grouped-query); 0 -> heads
    v_dim: int = 0                # width of V, O, dO rows; 0 -> head_dim
    causal: int = 1
    window: int = 0               # key slots, self included; <= 0: none
    scale: float = 0.0            # 0 -> 1/sqrt(head_dim)
    rope_base: float = 10000.0
    doc_range: Optional[Tuple[int, int]] = None   # random sequence lengths
    batch: int = 1                # equal sequences when doc_range is None
    backward: bool = False

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == DTYPE_BF16 else torch.float32

    def scaled(self, n_tokens: int, doc_range=None, batch=None) -> "Workload":
        """The same problem at another size (for oracle-sized parity runs)."""
        return replace(self, n_tokens=n_tokens,
                       doc_range=doc_range if doc_range is not None else self.doc_range,
                       batch=batch if batch is not None else self.batch)


WORKLOADS = {
    1: Workload("tiny causal fp32 T=128 H=4 d=64", 1, DTYPE_FP32, 128, 4, 64, ROPE_HALF,
                scale=0.125),
    2: Workload("gpt2-small causal bf16 B=8 T=1024 H=12 d=64", 2, DTYPE_BF16, 8192, 12, 64,
                ROPE_HALF, batch=8),
    3: Workload("paired varlen window-128 bf16 N=65536 H=6 d=128", 3, DTYPE_BF16, 65536, 6, 128,
                ROPE_ADJACENT, paired=1, window=128, doc_range=(256, 4096)),
    4: Workload("varlen window-2048 bf16 N=65536 H=6 d=128", 4, DTYPE_BF16, 65536, 6, 128,
                ROPE_ADJACENT, window=2048, doc_range=(512, 8192)),
    5: Workload("long causal fwd+bwd bf16 T=16384 H=12 d=64", 5, DTYPE_BF16, 16384, 12, 64,
                ROPE_HALF, backward=True),
}


def cu_seqlens(w: Workload, seed: Optional[int] = None) -> np.ndarray:
    """Sequence boundaries (int32, S + 1 entries, 0 .. n_tokens)."""
    seed = w.num if seed is None else seed
    if w.doc_range is None:
        b = max(1, w.batch)
        if w.n_tokens % b:
            raise ValueError("n_tokens must be a multiple of batch")
        return np.arange(0, w.n_tokens + 1, w.n_tokens // b, dtype=np.int32) if w.n_tokens else \
            np.zeros(b + 1, dtype=np.int32)
    lo, hi = w.doc_range
    rng = np.random.default_rng(seed)
    lengths = []
    total = 0
    while total < w.n_tokens:
        n = int(rng.integers(lo, hi + 1))
        n = min(n, w.n_tokens - total)
        lengths.append(n)
        total += n
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def tensors(w: Workload, seed: Optional[int] = None, with_grad: Optional[bool] = None):
    """Q, K, V (and dO) as CPU tensors [N, H, d] (K, V: [N, Hkv, d] when grouped;
    V and dO rows have v_dim elements when it is set) in the workload's dtype."""
    seed = w.num if seed is None else seed
    with_grad = w.backward if with_grad is None else with_grad
    g = torch.Generator().manual_seed(seed)
    dv = w.v_dim or w.head_dim
    hk = w.kv_heads or w.heads
    shapes = {"q": (w.n_tokens, w.heads, w.head_dim), "k": (w.n_tokens, hk, w.head_dim),
              "v": (w.n_tokens, hk, dv), "do": (w.n_tokens, w.heads, dv)}
    names = ["q", "k", "v"] + (["do"] if with_grad else [])
    out = {}
    for n in names:
        out[n] = torch.randn(shapes[n], generator=g, dtype=torch.float32).to(w.torch_dtype)
    return out


def generate(w: Workload, seed: Optional[int] = None, with_grad: Optional[bool] = None):
    """All inputs of one problem: dict with cu (numpy int32) and the tensors."""
    out = tensors(w, seed, with_grad)
    out["cu"] = cu_seqlens(w, seed)
    return out


def fp8_tensors(w: Workload, seed: Optional[int] = None):
    """Q, K, V as e4m3 codes (uint8 CPU tensors, shapes as in ``tensors``) and their
    per-tensor float32 scales (q, k, v)."""
    seed = w.num if seed is None else seed
    g = torch.Generator().manual_seed(seed)
    hk = w.kv_heads or w.heads
    shapes = {"q": (w.n_tokens, w.heads, w.head_dim), "k": (w.n_tokens, hk, w.head_dim),
              "v": (w.n_tokens, hk, w.v_dim or w.head_dim)}
    out, scales = {}, []
    for n in ("q", "k", "v"):
        x = torch.randn(shapes[n], generator=g, dtype=torch.float32)
        amax = float(x.abs().max()) if x.numel() else 1.0
        sc = float(np.float32(max(amax, 1e-30) / 448.0))
        out[n] = (x / sc).to(torch.float8_e4m3fn).view(torch.uint8)
        scales.append(sc)
    out["scales"] = tuple(scales)
    out["cu"] = cu_seqlens(w, seed)
    return out
