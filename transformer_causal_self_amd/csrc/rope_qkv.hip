// rope_qkv.hip -- fused rotary embedding of Q and K (and optional dense copy of
// V) for gfx950.  Memory bound: one read and one write of every element, with
// 128-bit loads and stores.
//
// What it computes ("Upgrading a textbook decoder", section 2 "RoPE";
// "Paired Head Attention" article, sections "Zero-copy RoPE", "Staggered
// rotary" and "Source 4: Triton kernel interleave indexing"): token t of its
// sequence, head h, pair i = (a, b) becomes (a cos - b sin, b cos + a sin) at
// angle p * base^(-2i/d), p = t, or 2t + (h mod 2) for paired heads.  Pairs are
// (i, i + d/2) for the half-split convention and (2i, 2i + 1) for adjacent
// pairs; the partner is formed in registers, never re-read from HBM.  The
// dense output [N, H, d] is already the paired interleaved layout
// [2N, H/2, d], so the interleave costs no extra pass.
//
// Work split: one thread owns one token and two 16-byte units of every head
// row, and walks the H heads, so its cos/sin values (fp32, read from the table,
// L2 resident) are loaded once per token and reused for every head of Q and K.
//
// The adjacent pairing (partner h ^ 1; "Paired Head Attention", section "Core
// idea") puts head h at slot 2t + (h mod 2), attention head h / 2, which in the
// dense [2N, H/2, d] output is position (h mod 2) * H/2 + h / 2 of the token's
// row: the store permutes heads (V is copied with the same permutation).
//
// Grouped K/V heads: K (and V) carry Hkv heads; their rows are rotated after
// the H query rows.  QK norm ("Paired Head Attention", section "Source 4":
// the rotary kernel also applies the Q/K RMS-norm; "Upgrading a textbook
// decoder", section 1 "RMSNorm"): each row is divided by sqrt(mean(x^2) + eps)
// in fp32 before its rotation; the row's sum of squares is spread over the
// lanes of its token and summed across them.  The backward kernel at the end
// of this file rotates gradient rows by -phi and applies the norm's gradient.
#include "attn_internal.h"
#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

template <typename T>
struct Vec;  // 16-byte vector of T
template <>
struct Vec<__bf16> {
  static constexpr int kN = 8;
};
template <>
struct Vec<float> {
  static constexpr int kN = 4;
};

template <typename T>
__device__ __forceinline__ void unpack(const uint4 &u, float *f);
template <>
__device__ __forceinline__ void unpack<__bf16>(const uint4 &u, float *f) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(w[i]);
    f[2 * i + 1] = bf16_hi(w[i]);
  }
}
template <>
__device__ __forceinline__ void unpack<float>(const uint4 &u, float *f) {
  f[0] = __uint_as_float(u.x);
  f[1] = __uint_as_float(u.y);
  f[2] = __uint_as_float(u.z);
  f[3] = __uint_as_float(u.w);
}

template <typename T>
__device__ __forceinline__ uint4 pack(const float *f);
template <>
__device__ __forceinline__ uint4 pack<__bf16>(const float *f) {
  return make_uint4(pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]),
                    pack_bf16(f[6], f[7]));
}
template <>
__device__ __forceinline__ uint4 pack<float>(const float *f) {
  return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                    __float_as_uint(f[3]));
}

// Sum over each aligned group of L consecutive lanes (the lanes of one token).
template <int L>
__device__ __forceinline__ float lanes_sum(float v) {
#pragma unroll
  for (int m = 1; m < L; m <<= 1) v += __shfl_xor(v, m, L);
  return v;
}

// cos and sin of angle column `col` at position `pos` from the two-level
// table: rows [0, F) hold lo * theta, rows F + hi hold hi * F * theta
// (F = kRopeFine); pos = hi * F + lo by the angle-addition formulas.
template <int D>
__device__ __forceinline__ void table_angle(const float *__restrict__ tcos,
                                            const float *__restrict__ tsin, int64_t pos, int col,
                                            float &c, float &s) {
  const int64_t lo = pos & (kRopeFine - 1), hi = kRopeFine + pos / kRopeFine;
  const float c1 = tcos[lo * (D / 2) + col], s1 = tsin[lo * (D / 2) + col];
  const float c2 = tcos[hi * (D / 2) + col], s2 = tsin[hi * (D / 2) + col];
  c = fmaf(c2, c1, -s2 * s1);
  s = fmaf(s2, c1, c2 * s1);
}

// Work split: a row of D elements is U = D / V sixteen-byte units (V elements
// each).  Thread (token n, chunk c) owns units c and c + U/2 of every head row of
// that token, so each load/store instruction of a wave covers whole 128-byte
// lines.  Half-split pairs element i of unit c with element i of unit c + U/2;
// adjacent pairs stay inside a unit.
template <typename T, int D, bool HALF>
struct RopeChunk {
  static constexpr int V = Vec<T>::kN;
  static constexpr int U = D / V;
  // a thread rotates V pairs: V half-split pairs across its two units, or V/2
  // adjacent pairs inside each unit.  Table column of its pair i: half-split
  // c*V + i; adjacent u*V/2 + i' for unit u = c (i < V/2) or c + U/2.
  static constexpr int NP = V;
  __device__ static __forceinline__ int col(int c, int i) {
    if (HALF) return c * V + i;
    return (i < V / 2) ? c * (V / 2) + i : (c + U / 2) * (V / 2) + (i - V / 2);
  }
  // rotation of the unpacked pair values a (unit c) and b (unit c + U/2),
  // each first multiplied by `scale`; packed back to T
  __device__ static __forceinline__ void rotate_vals(const float *a, const float *b,
                                                     const float *cs, const float *sn, float scale,
                                                     uint4 &r0, uint4 &r1) {
    float x[V], y[V];
    if (HALF) {
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const float ai = a[i] * scale, bi = b[i] * scale;
        x[i] = fmaf(ai, cs[i], -bi * sn[i]);
        y[i] = fmaf(bi, cs[i], ai * sn[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < V / 2; ++i) {
        const float a0 = a[2 * i] * scale, a1 = a[2 * i + 1] * scale;
        const float b0 = b[2 * i] * scale, b1 = b[2 * i + 1] * scale;
        x[2 * i] = fmaf(a0, cs[i], -a1 * sn[i]);
        x[2 * i + 1] = fmaf(a1, cs[i], a0 * sn[i]);
        const int j = V / 2 + i;
        y[2 * i] = fmaf(b0, cs[j], -b1 * sn[j]);
        y[2 * i + 1] = fmaf(b1, cs[j], b0 * sn[j]);
      }
    }
    r0 = pack<T>(x);
    r1 = pack<T>(y);
  }
  __device__ static __forceinline__ void rotate(const uint4 &u0, const uint4 &u1, const float *cs,
                                                const float *sn, uint4 &r0, uint4 &r1) {
    float a[V], b[V];
    unpack<T>(u0, a);
    unpack<T>(u1, b);
    rotate_vals(a, b, cs, sn, 1.0f, r0, r1);
  }
  // RMS-norm then rotation of one head row: the sum of squares over the row is
  // spread over the U/2 lanes of the token and summed across them
  __device__ static __forceinline__ void norm_rotate(const uint4 &u0, const uint4 &u1,
                                                     const float *cs, const float *sn, float eps,
                                                     uint4 &r0, uint4 &r1) {
    float a[V], b[V];
    unpack<T>(u0, a);
    unpack<T>(u1, b);
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < V; ++i) ss = fmaf(a[i], a[i], fmaf(b[i], b[i], ss));
    ss = lanes_sum<U / 2>(ss);
    rotate_vals(a, b, cs, sn, rsqrtf(ss * (1.0f / D) + eps), r0, r1);
  }
};

// PM: 0 unpaired, 1 paired (partner h + H/2, no permutation), 2 paired
// adjacent (partner h ^ 1, heads permuted on store).
// NORM: RMS-normalise each Q and K head row (eps) before rotating it.
template <typename T, int D, bool HALF, int PM, bool NORM>
__global__ __launch_bounds__(kRopeThreads) void rope_kernel(
    const T *q, int64_t qs, const T *k, int64_t ks, const T *__restrict__ v, int64_t vs, T *qo,
    T *ko, T *__restrict__ vo, const int32_t *__restrict__ tok_pos,
    const float *__restrict__ tcos, const float *__restrict__ tsin, int64_t N, int H, int Hk,
    float eps, int dv) {
  using RC = RopeChunk<T, D, HALF>;
  constexpr int U = RC::U, NP = RC::NP;
  const int64_t gid = (int64_t)blockIdx.x * kRopeThreads + threadIdx.x;
  const int64_t n = gid / (U / 2);
  const int c = (int)(gid % (U / 2));
  if (n >= N) return;
  const int t = tok_pos[n];
  float cs[2][NP], sn[2][NP];
#pragma unroll
  for (int par = 0; par < (PM ? 2 : 1); ++par) {
    const int64_t pos = PM ? 2 * t + par : t;
#pragma unroll
    for (int i = 0; i < NP; ++i)
      table_angle<D>(tcos, tsin, pos, RC::col(c, i), cs[par][i], sn[par][i]);
  }
  const uint4 *q4 = reinterpret_cast<const uint4 *>(q + n * qs);
  const uint4 *k4 = reinterpret_cast<const uint4 *>(k + n * ks);
  uint4 *qo4 = reinterpret_cast<uint4 *>(qo + n * (int64_t)H * D);
  uint4 *ko4 = reinterpret_cast<uint4 *>(ko + n * (int64_t)Hk * D);
  auto rot = [eps](const uint4 &u0, const uint4 &u1, const float *c_, const float *s_, uint4 &r0,
                   uint4 &r1) {
    if (NORM)
      RC::norm_rotate(u0, u1, c_, s_, eps, r0, r1);
    else
      RC::rotate(u0, u1, c_, s_, r0, r1);
  };
  // output position of head hh inside the token's row
  auto out_head = [H](int hh) { return PM == 2 ? (hh & 1) * (H / 2) + hh / 2 : hh; };
  if (Hk == H) {
    int h = 0;
    // two heads per step: eight 16-byte loads in flight before any store
    for (; h + 1 < H; h += 2) {
      uint4 in[2][2][2];  // [head][q/k][unit]
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int base = (h + e) * U;
        in[e][0][0] = q4[base + c];
        in[e][0][1] = q4[base + c + U / 2];
        in[e][1][0] = k4[base + c];
        in[e][1][1] = k4[base + c + U / 2];
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int par = PM ? ((h + e) & 1) : 0;
        const int base = out_head(h + e) * U;
        uint4 r0, r1;
        rot(in[e][0][0], in[e][0][1], cs[par], sn[par], r0, r1);
        qo4[base + c] = r0;
        qo4[base + c + U / 2] = r1;
        rot(in[e][1][0], in[e][1][1], cs[par], sn[par], r0, r1);
        ko4[base + c] = r0;
        ko4[base + c + U / 2] = r1;
      }
    }
    if (h < H) {  // odd H: unpaired only
      const int par = PM ? (h & 1) : 0;
      const int base = h * U;
      const uint4 a0 = q4[base + c], a1 = q4[base + c + U / 2];
      const uint4 b0 = k4[base + c], b1 = k4[base + c + U / 2];
      uint4 r0, r1;
      rot(a0, a1, cs[par], sn[par], r0, r1);
      qo4[base + c] = r0;
      qo4[base + c + U / 2] = r1;
      rot(b0, b1, cs[par], sn[par], r0, r1);
      ko4[base + c] = r0;
      ko4[base + c + U / 2] = r1;
    }
  } else {
    // grouped K/V heads (unpaired): the H query heads, then the Hk key heads,
    // two heads (four 16-byte loads) per step
    auto rotate_heads = [&](const uint4 *src, uint4 *dst, int nh) {
      int h = 0;
      for (; h + 1 < nh; h += 2) {
        uint4 in[2][2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          in[e][0] = src[(h + e) * U + c];
          in[e][1] = src[(h + e) * U + c + U / 2];
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          uint4 r0, r1;
          rot(in[e][0], in[e][1], cs[0], sn[0], r0, r1);
          dst[(h + e) * U + c] = r0;
          dst[(h + e) * U + c + U / 2] = r1;
        }
      }
      if (h < nh) {
        uint4 r0, r1;
        rot(src[h * U + c], src[h * U + c + U / 2], cs[0], sn[0], r0, r1);
        dst[h * U + c] = r0;
        dst[h * U + c + U / 2] = r1;
      }
    };
    rotate_heads(q4, qo4, H);
    rotate_heads(k4, ko4, Hk);
  }
  if (vo) {  // V rows hold dv elements: UV units, spread over the token's U/2 lanes
    const int UV = dv / RC::V;
    const uint4 *v4 = reinterpret_cast<const uint4 *>(v + n * vs);
    uint4 *vo4 = reinterpret_cast<uint4 *>(vo + n * (int64_t)Hk * dv);
    for (int hh = 0; hh < Hk; ++hh) {
      const int ob = out_head(hh) * UV;
      for (int u = c; u < UV; u += U / 2) vo4[ob + u] = v4[hh * UV + u];
    }
  }
}

template <typename T, int D>
hipError_t launch_typed(const attn_plan *p, const void *q, int64_t qs, const void *k, int64_t ks,
                        const void *v, int64_t vs, void *qo, void *ko, void *vo,
                        hipStream_t stream) {
  constexpr int C = D / Vec<T>::kN / 2;  // threads per token
  const int64_t N = p->p.N;
  const int64_t threads = N * C;
  const dim3 grid((unsigned)((threads + kRopeThreads - 1) / kRopeThreads));
  const int32_t *pos = reinterpret_cast<const int32_t *>(p->ws + p->off_pos);
  const float *tc = reinterpret_cast<const float *>(p->ws + p->off_cos);
  const float *ts = reinterpret_cast<const float *>(p->ws + p->off_sin);
  const T *Q = static_cast<const T *>(q);
  const T *K = static_cast<const T *>(k);
  const T *Vv = static_cast<const T *>(v);
  T *QO = static_cast<T *>(qo);
  T *KO = static_cast<T *>(ko);
  T *VO = static_cast<T *>(vo);
  const bool half = p->p.rope == ATTN_ROPE_HALF;
  const int pm = p->p.paired;
  const float eps = p->p.norm_eps;
#define ROPE_LAUNCH(HF, PMV, NRM)                                                          \
  hipLaunchKernelGGL((rope_kernel<T, D, HF, PMV, NRM>), grid, dim3(kRopeThreads), 0, stream, Q, \
                     qs, K, ks, Vv, vs, QO, KO, VO, pos, tc, ts, N, p->p.H, p->p.Hkv, eps,    \
                     p->p.dv)
#define ROPE_PM(HF, NRM)                \
  do {                                  \
    if (pm == 0) ROPE_LAUNCH(HF, 0, NRM); \
    else if (pm == 1) ROPE_LAUNCH(HF, 1, NRM); \
    else ROPE_LAUNCH(HF, 2, NRM);       \
  } while (0)
  if (p->p.qk_norm) {
    if (half) ROPE_PM(true, true);
    else ROPE_PM(false, true);
  } else {
    if (half) ROPE_PM(true, false);
    else ROPE_PM(false, false);
  }
#undef ROPE_PM
#undef ROPE_LAUNCH
  return hipGetLastError();
}

// ------------------------------------------------------------------ fp8 in --
// FP8 (e4m3, OCP) inputs with per-tensor scales, bf16 outputs: the same lane
// split as the bf16 kernel (lane = token x units c, c + U/2 of 8 outputs),
// each unit read as 8 one-byte codes, decoded by v_cvt_pk_f32_fp8 and scaled
// before the norm and the rotation.  V is decoded and copied (its slot order
// under the adjacent pairing).
__device__ __forceinline__ void unpack_fp8(const uint2 &u, float scale, float *f) {
  const uint32_t w[2] = {u.x, u.y};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);  // bytes 0, 1
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);   // bytes 2, 3
    f[4 * i] = lo[0] * scale;
    f[4 * i + 1] = lo[1] * scale;
    f[4 * i + 2] = hi[0] * scale;
    f[4 * i + 3] = hi[1] * scale;
  }
}

template <int D, bool HALF, int PM, bool NORM>
__global__ __launch_bounds__(kRopeThreads) void rope_fp8_kernel(
    const uint8_t *__restrict__ q, int64_t qs, const uint8_t *__restrict__ k, int64_t ks,
    const uint8_t *__restrict__ v, int64_t vs, __bf16 *__restrict__ qo, __bf16 *__restrict__ ko,
    __bf16 *__restrict__ vo, const int32_t *__restrict__ tok_pos, const float *__restrict__ tcos,
    const float *__restrict__ tsin, int64_t N, int H, int Hk, float eps, float q_scale,
    float k_scale, float v_scale, int dv) {
  using RC = RopeChunk<__bf16, D, HALF>;
  constexpr int U = RC::U, NP = RC::NP;  // units of 8 elements
  const int64_t gid = (int64_t)blockIdx.x * kRopeThreads + threadIdx.x;
  const int64_t n = gid / (U / 2);
  const int c = (int)(gid % (U / 2));
  if (n >= N) return;  // whole token groups leave together
  const int t = tok_pos[n];
  float cs[2][NP], sn[2][NP];
#pragma unroll
  for (int par = 0; par < (PM ? 2 : 1); ++par) {
    const int64_t pos = PM ? 2 * t + par : t;
#pragma unroll
    for (int i = 0; i < NP; ++i)
      table_angle<D>(tcos, tsin, pos, RC::col(c, i), cs[par][i], sn[par][i]);
  }
  auto out_head = [H](int hh) { return PM == 2 ? (hh & 1) * (H / 2) + hh / 2 : hh; };
  auto rows = [&](const uint8_t *src, int64_t ss, float scale, __bf16 *dst, int nh) {
    const uint2 *s8 = reinterpret_cast<const uint2 *>(src + n * ss);  // 8 codes per unit
    uint4 *d4 = reinterpret_cast<uint4 *>(dst + n * (int64_t)nh * D);
    for (int hh = 0; hh < nh; ++hh) {
      const int par = PM ? (hh & 1) : 0;
      float a[8], b[8];
      unpack_fp8(s8[hh * U + c], scale, a);
      unpack_fp8(s8[hh * U + c + U / 2], scale, b);
      float r = 1.0f;
      if (NORM) {
        float ss2 = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss2 = fmaf(a[i], a[i], fmaf(b[i], b[i], ss2));
        r = rsqrtf(lanes_sum<U / 2>(ss2) * (1.0f / D) + eps);
      }
      uint4 r0, r1;
      RC::rotate_vals(a, b, cs[par], sn[par], r, r0, r1);
      const int ob = out_head(hh) * U;
      d4[ob + c] = r0;
      d4[ob + c + U / 2] = r1;
    }
  };
  rows(q, qs, q_scale, qo, H);
  rows(k, ks, k_scale, ko, Hk);
  const int UV = dv / 8;  // V rows: dv codes, UV units of 8 over the token's U/2 lanes
  const uint2 *v8 = reinterpret_cast<const uint2 *>(v + n * vs);
  uint4 *v4 = reinterpret_cast<uint4 *>(vo + n * (int64_t)Hk * dv);
  for (int hh = 0; hh < Hk; ++hh) {
    const int ob = out_head(hh) * UV;
    for (int u = c; u < UV; u += U / 2) {
      float a[8];
      unpack_fp8(v8[hh * UV + u], v_scale, a);
      v4[ob + u] = pack<__bf16>(a);
    }
  }
}

template <int D>
hipError_t launch_fp8_typed(const attn_plan *p, const void *q, int64_t qs, const void *k,
                            int64_t ks, const void *v, int64_t vs, const float *scales, void *qo,
                            void *ko, void *vo, hipStream_t stream) {
  constexpr int C = D / 16;  // lanes per token
  const int64_t N = p->p.N;
  const dim3 grid((unsigned)((N * C + kRopeThreads - 1) / kRopeThreads));
  const int32_t *pos = reinterpret_cast<const int32_t *>(p->ws + p->off_pos);
  const float *tc = reinterpret_cast<const float *>(p->ws + p->off_cos);
  const float *ts = reinterpret_cast<const float *>(p->ws + p->off_sin);
  const uint8_t *Q = static_cast<const uint8_t *>(q), *K = static_cast<const uint8_t *>(k);
  const uint8_t *Vv = static_cast<const uint8_t *>(v);
  __bf16 *QO = static_cast<__bf16 *>(qo), *KO = static_cast<__bf16 *>(ko);
  __bf16 *VO = static_cast<__bf16 *>(vo);
  const bool half = p->p.rope == ATTN_ROPE_HALF;
  const int pm = p->p.paired;
  const float eps = p->p.norm_eps;
#define F8_LAUNCH(HF, PMV, NRM)                                                                 \
  hipLaunchKernelGGL((rope_fp8_kernel<D, HF, PMV, NRM>), grid, dim3(kRopeThreads), 0, stream, Q, \
                     qs, K, ks, Vv, vs, QO, KO, VO, pos, tc, ts, N, p->p.H, p->p.Hkv, eps,       \
                     scales[0], scales[1], scales[2], p->p.dv)
#define F8_PM(HF, NRM)                         \
  do {                                         \
    if (pm == 0) F8_LAUNCH(HF, 0, NRM);        \
    else if (pm == 1) F8_LAUNCH(HF, 1, NRM);   \
    else F8_LAUNCH(HF, 2, NRM);                \
  } while (0)
  if (p->p.qk_norm) {
    if (half) F8_PM(true, true);
    else F8_PM(false, true);
  } else {
    if (half) F8_PM(true, false);
    else F8_PM(false, false);
  }
#undef F8_PM
#undef F8_LAUNCH
  return hipGetLastError();
}

// ---------------------------------------------------------------- backward --
// Backward of rope_qkv for one token per group of D/8 lanes: the incoming
// gradient rows (fp32, read from the slot layout) are rotated by -phi, the
// transpose of the forward rotation, and with NORM pushed through the RMS-norm:
// dx = r g - (r^3 / D) x (g . x), r = 1 / sqrt(mean(x^2) + eps), x the forward
// input row (plan dtype).  Lane (token n, chunk c) owns the fp32 units c and
// c + D/8 of every row (4 elements each).
template <typename T>
__device__ __forceinline__ void load4(const T *p, float *f);
template <>
__device__ __forceinline__ void load4<__bf16>(const __bf16 *p, float *f) {
  const uint2 u = *reinterpret_cast<const uint2 *>(p);
  f[0] = bf16_lo(u.x);
  f[1] = bf16_hi(u.x);
  f[2] = bf16_lo(u.y);
  f[3] = bf16_hi(u.y);
}
template <>
__device__ __forceinline__ void load4<float>(const float *p, float *f) {
  const float4 u = *reinterpret_cast<const float4 *>(p);
  f[0] = u.x;
  f[1] = u.y;
  f[2] = u.z;
  f[3] = u.w;
}

template <typename T, int D, bool HALF, int PM, bool NORM>
__global__ __launch_bounds__(kRopeThreads) void rope_bwd_kernel(
    const T *__restrict__ q, int64_t qs, const T *__restrict__ k, int64_t ks, const float *dq_in,
    const float *dk_in, const float *dv_in, float *dq, float *dk, float *dv,
    const int32_t *__restrict__ tok_pos, const float *__restrict__ tcos,
    const float *__restrict__ tsin, int64_t N, int H, int Hk, float eps, int dv_dim) {
  using RC = RopeChunk<float, D, HALF>;  // fp32 units of 4
  constexpr int U = RC::U, NP = RC::NP, L = U / 2;
  const int64_t gid = (int64_t)blockIdx.x * kRopeThreads + threadIdx.x;
  const int64_t n = gid / L;
  const int c = (int)(gid % L);
  if (n >= N) return;  // whole token groups leave together
  const int t = tok_pos[n];
  float cs[2][NP], sn[2][NP];  // sin negated: the transpose rotates by -phi
#pragma unroll
  for (int par = 0; par < (PM ? 2 : 1); ++par) {
    const int64_t pos = PM ? 2 * t + par : t;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      table_angle<D>(tcos, tsin, pos, RC::col(c, i), cs[par][i], sn[par][i]);
      sn[par][i] = -sn[par][i];
    }
  }
  auto slot_head = [H](int hh) { return PM == 2 ? (hh & 1) * (H / 2) + hh / 2 : hh; };
  auto rows = [&](const float *gin, float *gout, const T *x, int64_t xs, int nh) {
    const uint4 *g4 = reinterpret_cast<const uint4 *>(gin + n * (int64_t)nh * D);
    uint4 *o4 = reinterpret_cast<uint4 *>(gout + n * (int64_t)nh * D);
    for (int hh = 0; hh < nh; ++hh) {
      const int par = PM ? (hh & 1) : 0;
      const int sb = slot_head(hh) * U;
      uint4 r0, r1;
      RC::rotate(g4[sb + c], g4[sb + c + U / 2], cs[par], sn[par], r0, r1);
      if (NORM) {
        float ga[4], gb[4], xa[4], xb[4];
        unpack<float>(r0, ga);
        unpack<float>(r1, gb);
        const T *xr = x + n * xs + (int64_t)hh * D;
        load4<T>(xr + 4 * c, xa);
        load4<T>(xr + 4 * (c + U / 2), xb);
        float ss = 0.0f, xg = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ss = fmaf(xa[i], xa[i], fmaf(xb[i], xb[i], ss));
          xg = fmaf(xa[i], ga[i], fmaf(xb[i], gb[i], xg));
        }
        ss = lanes_sum<L>(ss);
        xg = lanes_sum<L>(xg);
        const float r = rsqrtf(ss * (1.0f / D) + eps);
        const float cx = r * r * r * (1.0f / D) * xg;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ga[i] = fmaf(r, ga[i], -cx * xa[i]);
          gb[i] = fmaf(r, gb[i], -cx * xb[i]);
        }
        r0 = pack<float>(ga);
        r1 = pack<float>(gb);
      }
      o4[hh * U + c] = r0;
      o4[hh * U + c + U / 2] = r1;
    }
  };
  rows(dq_in, dq, q, qs, H);
  rows(dk_in, dk, k, ks, Hk);
  if (dv) {  // dV rows: dv_dim floats, UV units of 4 over the token's L lanes
    const int UV = dv_dim / 4;
    const uint4 *v4 = reinterpret_cast<const uint4 *>(dv_in + n * (int64_t)Hk * dv_dim);
    uint4 *o4 = reinterpret_cast<uint4 *>(dv + n * (int64_t)Hk * dv_dim);
    for (int hh = 0; hh < Hk; ++hh) {
      const int sb = slot_head(hh) * UV;
      for (int u = c; u < UV; u += L) o4[hh * UV + u] = v4[sb + u];
    }
  }
}

template <typename T, int D>
hipError_t launch_bwd_typed(const attn_plan *p, const void *q, int64_t qs, const void *k,
                            int64_t ks, const float *dqi, const float *dki, const float *dvi,
                            float *dq, float *dk, float *dv, hipStream_t stream) {
  constexpr int L = D / 8;  // lanes per token
  const int64_t N = p->p.N;
  const dim3 grid((unsigned)((N * L + kRopeThreads - 1) / kRopeThreads));
  const int32_t *pos = reinterpret_cast<const int32_t *>(p->ws + p->off_pos);
  const float *tc = reinterpret_cast<const float *>(p->ws + p->off_cos);
  const float *ts = reinterpret_cast<const float *>(p->ws + p->off_sin);
  const T *Q = static_cast<const T *>(q);
  const T *K = static_cast<const T *>(k);
  const bool half = p->p.rope == ATTN_ROPE_HALF;
  const int pm = p->p.paired;
  const float eps = p->p.norm_eps;
#define RB_LAUNCH(HF, PMV, NRM)                                                                 \
  hipLaunchKernelGGL((rope_bwd_kernel<T, D, HF, PMV, NRM>), grid, dim3(kRopeThreads), 0, stream, \
                     Q, qs, K, ks, dqi, dki, dvi, dq, dk, dv, pos, tc, ts, N, p->p.H, p->p.Hkv,  \
                     eps, p->p.dv)
#define RB_PM(HF, NRM)                         \
  do {                                         \
    if (pm == 0) RB_LAUNCH(HF, 0, NRM);        \
    else if (pm == 1) RB_LAUNCH(HF, 1, NRM);   \
    else RB_LAUNCH(HF, 2, NRM);                \
  } while (0)
  if (p->p.qk_norm) {
    if (half) RB_PM(true, true);
    else RB_PM(false, true);
  } else {
    if (half) RB_PM(true, false);
    else RB_PM(false, false);
  }
#undef RB_PM
#undef RB_LAUNCH
  return hipGetLastError();
}

}  // namespace

attn_status launch_rope_fp8(const attn_plan *p, const void *q, int64_t qs, const void *k,
                            int64_t ks, const void *v, int64_t vs, const float *scales,
                            void *q_out, void *k_out, void *v_out, hipStream_t stream) {
  const hipError_t e =
      p->p.d == 64
          ? launch_fp8_typed<64>(p, q, qs, k, ks, v, vs, scales, q_out, k_out, v_out, stream)
          : launch_fp8_typed<128>(p, q, qs, k, ks, v, vs, scales, q_out, k_out, v_out, stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

attn_status launch_rope_bwd(const attn_plan *p, const void *q, int64_t qs, const void *k,
                            int64_t ks, const float *dq_in, const float *dk_in,
                            const float *dv_in, float *dq, float *dk, float *dv,
                            hipStream_t stream) {
  hipError_t e;
  const bool bf = p->p.dtype == ATTN_BF16;
  if (p->p.d == 64)
    e = bf ? launch_bwd_typed<__bf16, 64>(p, q, qs, k, ks, dq_in, dk_in, dv_in, dq, dk, dv, stream)
           : launch_bwd_typed<float, 64>(p, q, qs, k, ks, dq_in, dk_in, dv_in, dq, dk, dv, stream);
  else
    e = bf ? launch_bwd_typed<__bf16, 128>(p, q, qs, k, ks, dq_in, dk_in, dv_in, dq, dk, dv,
                                           stream)
           : launch_bwd_typed<float, 128>(p, q, qs, k, ks, dq_in, dk_in, dv_in, dq, dk, dv,
                                          stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

attn_status launch_rope(const attn_plan *p, const void *q, int64_t qs, const void *k, int64_t ks,
                        const void *v, int64_t vs, void *q_out, void *k_out, void *v_out,
                        hipStream_t stream) {
  hipError_t e;
  const bool bf = p->p.dtype == ATTN_BF16;
  if (p->p.d == 64)
    e = bf ? launch_typed<__bf16, 64>(p, q, qs, k, ks, v, vs, q_out, k_out, v_out, stream)
           : launch_typed<float, 64>(p, q, qs, k, ks, v, vs, q_out, k_out, v_out, stream);
  else
    e = bf ? launch_typed<__bf16, 128>(p, q, qs, k, ks, v, vs, q_out, k_out, v_out, stream)
           : launch_typed<float, 128>(p, q, qs, k, ks, v, vs, q_out, k_out, v_out, stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

}  // namespace attn
