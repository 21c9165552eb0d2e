"""Dense brute-force constructions used to pin the oracle on tiny inputs.

These are deliberately built a different way from oracle.c:
  * the paired sequence is assembled by literal list construction in the order
    the "Paired Head Attention" article (hncyxsy.com, section "Core idea")
    shows -- position by position, the first head of the pair, then the
    second -- instead of through an index formula;
  * the mask is a dense boolean matrix made of a lower-triangular block per
    sequence (the "SingleHeadAttention" note, ranhao.site, slicing example)
    intersected with a band for the window;
  * rotation uses complex multiplication by exp(i * angle) instead of cos/sin
    expressions.
"""
import numpy as np


def pair_members(H, paired):
    """For each attention head, the list of logical heads, in slot order."""
    if paired == 0:
        return [[h] for h in range(H)]
    if paired == 1:   # code reading: head h pairs with h + H/2
        return [[j, j + H // 2] for j in range(H // 2)]
    if paired == 2:   # prose reading: adjacent heads 2j, 2j+1
        return [[2 * j, 2 * j + 1] for j in range(H // 2)]
    raise ValueError(paired)


def interleave(x, H, paired):
    """x [N, H, d] -> list over attention heads of arrays [N', d] plus, for
    each slot, the (token, logical head) it came from."""
    N = x.shape[0]
    out, origin = [], []
    for members in pair_members(H, paired):
        rows, orig = [], []
        for t in range(N):
            for h in members:
                rows.append(x[t, h])
                orig.append((t, h))
        out.append(np.array(rows).reshape(len(rows), x.shape[2]))
        orig_arr = np.array(orig, dtype=np.int64).reshape(len(orig), 2)
        origin.append(orig_arr)
    return out, origin


def dense_mask(cu, mult, causal, window):
    """Boolean visibility [N', N'] for sequence boundaries cu scaled by mult."""
    bounds = [c * mult for c in cu]
    n = bounds[-1]
    m = np.zeros((n, n), dtype=bool)
    for b, e in zip(bounds[:-1], bounds[1:]):
        L = e - b
        block = np.tril(np.ones((L, L), dtype=bool)) if causal else np.ones((L, L), dtype=bool)
        m[b:e, b:e] = block
    if window > 0:
        i = np.arange(n)[:, None]
        j = np.arange(n)[None, :]
        m &= (i - j) < window
    return m


def attention(q, k, v, cu, paired=0, causal=1, window=0, scale=0.0):
    """Dense fp64 forward: O [N, H, dv], LSE [H', N'], and P per attention head."""
    N, H, d = q.shape
    s = scale if scale else 1.0 / np.sqrt(d)
    qs, origin = interleave(q, H, paired)
    ks, _ = interleave(k, H, paired)
    vs, _ = interleave(v, H, paired)
    mask = dense_mask(list(cu), 2 if paired else 1, causal, window)
    o = np.zeros((N, H, v.shape[2]), dtype=np.float64)
    lses, probs = [], []
    for j in range(len(qs)):
        z = s * (qs[j] @ ks[j].T)
        z = np.where(mask, z, -np.inf)
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        l = e.sum(axis=1, keepdims=True)
        p = e / l
        oj = p @ vs[j]
        for slot, (t, h) in enumerate(origin[j]):
            o[t, h] = oj[slot]
        lses.append((m + np.log(l))[:, 0])
        probs.append(p)
    return o, np.array(lses), probs


def rope(x, cu, convention, base=10000.0, paired=0):
    """RoPE by complex multiplication: pair (a, b) -> (a + ib) * exp(i p theta)."""
    N, H, d = x.shape
    half = d // 2
    y = np.array(x, dtype=np.float64, copy=True)
    theta = base ** (-np.arange(half) * 2.0 / d)
    for b_, e_ in zip(cu[:-1], cu[1:]):
        for n in range(b_, e_):
            t = n - b_
            for h in range(H):
                p = 2 * t + (h % 2) if paired else t
                if convention == 1:
                    z = x[n, h, :half] + 1j * x[n, h, half:]
                else:
                    z = x[n, h, 0::2] + 1j * x[n, h, 1::2]
                z = z * np.exp(1j * p * theta)
                if convention == 1:
                    y[n, h, :half], y[n, h, half:] = z.real, z.imag
                else:
                    y[n, h, 0::2], y[n, h, 1::2] = z.real, z.imag
    return y
