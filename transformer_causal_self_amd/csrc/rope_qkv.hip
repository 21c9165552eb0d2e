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
// Work split: one thread owns one token and one chunk of PP consecutive pairs
// and walks the H heads, so the chunk's cos/sin values (fp32, read from the
// table, L2 resident) are loaded once per token and reused for every head of
// Q and K.
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

// Rotate PP pairs of one head row.  HALF: pairs (c*PP + i, c*PP + i + D/2);
// else pairs (2(c*PP + i), 2(c*PP + i) + 1).
template <typename T, int D, bool HALF>
__device__ __forceinline__ void rotate_row(const T *__restrict__ src, T *__restrict__ dst, int c,
                                           const float *cs, const float *sn) {
  constexpr int V = Vec<T>::kN;
  constexpr int PP = V;  // pairs per thread
  const uint4 *s4 = reinterpret_cast<const uint4 *>(src);
  uint4 *d4 = reinterpret_cast<uint4 *>(dst);
  float a[2 * V];
  if (HALF) {
    // first-half elements c*PP .. c*PP+PP, second half + D/2
    const uint4 u0 = s4[c];
    const uint4 u1 = s4[c + D / 2 / V];
    unpack<T>(u0, a);
    unpack<T>(u1, a + V);
    float r[2 * V];
#pragma unroll
    for (int i = 0; i < PP; ++i) {
      const float x = a[i], y = a[V + i];
      r[i] = fmaf(x, cs[i], -y * sn[i]);
      r[V + i] = fmaf(y, cs[i], x * sn[i]);
    }
    d4[c] = pack<T>(r);
    d4[c + D / 2 / V] = pack<T>(r + V);
  } else {
    // 2*PP consecutive elements = PP adjacent pairs
    const uint4 u0 = s4[2 * c];
    const uint4 u1 = s4[2 * c + 1];
    unpack<T>(u0, a);
    unpack<T>(u1, a + V);
    float r[2 * V];
#pragma unroll
    for (int i = 0; i < PP; ++i) {
      const float x = a[2 * i], y = a[2 * i + 1];
      r[2 * i] = fmaf(x, cs[i], -y * sn[i]);
      r[2 * i + 1] = fmaf(y, cs[i], x * sn[i]);
    }
    d4[2 * c] = pack<T>(r);
    d4[2 * c + 1] = pack<T>(r + V);
  }
}

template <typename T, int D, bool HALF, bool PAIRED>
__global__ __launch_bounds__(kRopeThreads) void rope_kernel(
    const T *__restrict__ q, int64_t qs, const T *__restrict__ k, int64_t ks,
    const T *__restrict__ v, int64_t vs, T *__restrict__ qo, T *__restrict__ ko,
    T *__restrict__ vo, const int32_t *__restrict__ tok_pos, const float *__restrict__ tcos,
    const float *__restrict__ tsin, int64_t N, int H) {
  constexpr int V = Vec<T>::kN;
  constexpr int PP = V;
  constexpr int C = D / 2 / PP;  // chunks per head row
  const int64_t gid = (int64_t)blockIdx.x * kRopeThreads + threadIdx.x;
  const int64_t n = gid / C;
  const int c = (int)(gid % C);
  if (n >= N) return;
  const int t = tok_pos[n];
  // cos/sin of the chunk's PP pairs at the (one or two) positions used here.
  float cs[2][PP], sn[2][PP];
#pragma unroll
  for (int par = 0; par < (PAIRED ? 2 : 1); ++par) {
    const int pos = PAIRED ? 2 * t + par : t;
    const float4 *c4 = reinterpret_cast<const float4 *>(tcos + (int64_t)pos * (D / 2) + c * PP);
    const float4 *s4 = reinterpret_cast<const float4 *>(tsin + (int64_t)pos * (D / 2) + c * PP);
#pragma unroll
    for (int i = 0; i < PP / 4; ++i) {
      const float4 cc = c4[i], ss = s4[i];
      cs[par][4 * i] = cc.x;
      cs[par][4 * i + 1] = cc.y;
      cs[par][4 * i + 2] = cc.z;
      cs[par][4 * i + 3] = cc.w;
      sn[par][4 * i] = ss.x;
      sn[par][4 * i + 1] = ss.y;
      sn[par][4 * i + 2] = ss.z;
      sn[par][4 * i + 3] = ss.w;
    }
  }
  const int64_t row = (int64_t)H * D;
  for (int h = 0; h < H; ++h) {
    const int par = PAIRED ? (h & 1) : 0;
    rotate_row<T, D, HALF>(q + n * qs + h * D, qo + n * row + h * D, c, cs[par], sn[par]);
    rotate_row<T, D, HALF>(k + n * ks + h * D, ko + n * row + h * D, c, cs[par], sn[par]);
    if (vo) {
      // dense copy of this thread's two 16-byte pieces of V
      const uint4 *s4 = reinterpret_cast<const uint4 *>(v + n * vs + h * D);
      uint4 *d4 = reinterpret_cast<uint4 *>(vo + n * row + h * D);
      if (HALF) {
        d4[c] = s4[c];
        d4[c + D / 2 / V] = s4[c + D / 2 / V];
      } else {
        d4[2 * c] = s4[2 * c];
        d4[2 * c + 1] = s4[2 * c + 1];
      }
    }
  }
}

template <typename T, int D>
hipError_t launch_typed(const attn_plan *p, const void *q, int64_t qs, const void *k, int64_t ks,
                        const void *v, int64_t vs, void *qo, void *ko, void *vo,
                        hipStream_t stream) {
  constexpr int C = D / 2 / Vec<T>::kN;
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
  const bool paired = p->p.paired != 0;
  if (half && paired)
    hipLaunchKernelGGL((rope_kernel<T, D, true, true>), grid, dim3(kRopeThreads), 0, stream, Q,
                       qs, K, ks, Vv, vs, QO, KO, VO, pos, tc, ts, N, p->p.H);
  else if (half)
    hipLaunchKernelGGL((rope_kernel<T, D, true, false>), grid, dim3(kRopeThreads), 0, stream, Q,
                       qs, K, ks, Vv, vs, QO, KO, VO, pos, tc, ts, N, p->p.H);
  else if (paired)
    hipLaunchKernelGGL((rope_kernel<T, D, false, true>), grid, dim3(kRopeThreads), 0, stream, Q,
                       qs, K, ks, Vv, vs, QO, KO, VO, pos, tc, ts, N, p->p.H);
  else
    hipLaunchKernelGGL((rope_kernel<T, D, false, false>), grid, dim3(kRopeThreads), 0, stream, Q,
                       qs, K, ks, Vv, vs, QO, KO, VO, pos, tc, ts, N, p->p.H);
  return hipGetLastError();
}

}  // namespace

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
