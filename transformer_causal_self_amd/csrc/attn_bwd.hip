// attn_bwd.hip -- attention backward for gfx950 (bf16 inputs, fp32 gradients).
//
// What it computes: the gradients of L = sum(O * dO) through
// O = softmax(s Q K^T + mask) V with respect to Q, K, V (the rotated inputs
// of the forward), from the chain rule with the softmax Jacobian
// diag(P) - P P^T:
//     D_i  = dO_i . O_i
//     P    = exp(s q_i . k_j - LSE_i)           (recomputed from the forward's LSE)
//     dS   = P o (dO V^T - D)
//     dV   = P^T dO,   dK = s dS^T Q,   dQ = s dS K.
// The softmax derivative is the standard one, P o (dP - rowsum(dP o P)) with
// rowsum(dP o P) = D_i, not the variant printed in the "mHC module" article
// (lshu.cn, section 4.1), which is not the derivative of softmax.
//
// Two launches, deterministic without grouped K/V heads (no atomics):
//   1. delta:  D_i for every (attention head, slot).
//   2. one grid of two item kinds (the dQ items fill the CUs that the dK/dV
//      tail leaves idle):
//      dK/dV:  one block per 128-key tile of one attention head (four
//              waves, 32 keys each), looping over the 64-query tiles that
//              can see it.  S is formed as Q K^T so that every accumulator
//              lane belongs to one key; P^T and dS^T then feed the MFMA A
//              operand straight from registers, and the Q and dO B operands
//              are read transposed (ds_read_b64_tr_b16) from the same
//              row-major tiles that serve S and dP.
//      dQ:     one block per 128-query tile, looping over key tiles;
//              S^T = K Q^T as in the forward, and K^T for dQ^T = K^T dS^T
//              read transposed from the row-major K tile.
//   The streamed tiles (Q, dO; K, V) go from global memory straight into LDS
//   (buffer loads with the LDS flag), double buffered: the next tile's loads
//   are issued before the current tile's MMAs and waited for after them, and
//   no staging register or LDS store instruction is spent on them.
#include <mutex>

#include "attn_internal.h"
#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float dot8(const uint4 &a, const uint4 &b) {
  const uint32_t x[4] = {a.x, a.y, a.z, a.w}, y[4] = {b.x, b.y, b.z, b.w};
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s = fmaf(bf16_lo(x[i]), bf16_lo(y[i]), s);
    s = fmaf(bf16_hi(x[i]), bf16_hi(y[i]), s);
  }
  return s;
}

// D[head][slot] = dO . O over the head dimension.
template <int D>
__global__ __launch_bounds__(256) void delta_kernel(const __bf16 *__restrict__ O,
                                                    const __bf16 *__restrict__ dO,
                                                    float *__restrict__ delta, int Hs,
                                                    int64_t Ns) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;  // slot * Hs + head
  if (r >= Ns * Hs) return;
  const uint4 *o4 = reinterpret_cast<const uint4 *>(O + r * D);
  const uint4 *g4 = reinterpret_cast<const uint4 *>(dO + r * D);
  float acc = 0.0f;
#pragma unroll
  for (int c = 0; c < D / 8; ++c) acc += dot8(o4[c], g4[c]);
  delta[(r % Hs) * Ns + r / Hs] = acc;
}

__device__ __forceinline__ bf16x8 to_bf16x8(const floatx16 &x, int first) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[first + e];
  return r;
}

__device__ __forceinline__ bf16x8 load_bf16x8(const __bf16 *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}

// MFMA operand with k running down the rows of a row-major bf16 tile (row
// stride `stride` elements): for lane (l32, h), column n = l32 of the tile
// (relative to p) and rows 4h + 0..3, then 8 + 4h + 0..3 -- the row order of
// a 32x32 accumulator's registers 8m .. 8m + 7 -- by two ds_read_b64_tr_b16.
// Inside each group of 16 lanes, lane 4e + g addresses row e and columns
// 4g .. 4g + 3 (plus 16 for the upper 16 lanes of each half-wave).
__device__ __forceinline__ int tr_lane(int h, int l32, int stride) {
  return (4 * h + ((l32 & 15) >> 2)) * stride + 16 * (l32 >> 4) + 4 * (l32 & 3);
}
__device__ __forceinline__ bf16x8 tr_operand(const __bf16 *p, int stride) {
  const uint2 lo = lds_read_tr16(p), hi = lds_read_tr16(p + 8 * stride);
  return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// waves per SIMD the register budget is sized for: three four-wave blocks
// per CU when both widths are 64 (at most 168 VGPRs), else two (256 VGPRs)
template <int D, int DV>
constexpr int bwd_waves_per_simd() {
  return D == 64 && DV == 64 ? 3 : 2;
}

// The lane index as the DMA offsets are formed from it.  With both widths 128
// it is hidden from loop-invariant code motion, so the offsets are recomputed
// per tile rather than held across the loop: there the registers are short,
// a held offset is spilled, and reloading it before a DMA waits for every
// load issued before (2-4% faster).  With a width of 64 the recomputation
// costs more VALU time than it saves (2% at 64/64, 6% with mixed widths).
template <int D, int DV>
__device__ __forceinline__ int offset_lane(int lane) {
  if constexpr (D == 128 && DV == 128) asm volatile("" : "+v"(lane));
  return lane;
}

// With both widths 64, a wave raises its issue priority while it issues the
// S and dP MFMAs, so that the matrix unit is fed while the other waves of the
// SIMD compute their exponentials (-2.8% backward time at d = 64; with a
// width of 128, where the registers are already short, it costs 2-8%).
template <int D, int DV, int LEVEL>
__device__ __forceinline__ void mfma_priority() {
  if constexpr (D == 64 && DV == 64) __builtin_amdgcn_s_setprio(LEVEL);
}

// ---------------------------------------------------------------- dK, dV --

// D: width of Q, K (and their gradients); DV: width of V, O, dO, dV.
template <int D, int DV>
struct DkvBuf {
  static constexpr int RS = D + 8, RSV = DV + 8, BQ = kBwdBQ;
  __bf16 q[BQ * RS];
  __bf16 g[BQ * RSV];
  float lse2[BQ];  // LSE * log2(e)
  float dl[BQ];    // -D (the start value of the dP accumulator)
};
template <int D, int DV>
struct DkvSmem {
  DkvBuf<D, DV> b[2];  // double buffered: one barrier per query tile
};

// One dK/dV item (keys [q0, q1), queries [k0, k1)).
template <int D, int DV, int NW>
__device__ __forceinline__ void dkv_item(
    const WorkItem it, DkvSmem<D, DV> &sm, const __bf16 *__restrict__ Q,
    const __bf16 *__restrict__ K, const __bf16 *__restrict__ V, const __bf16 *__restrict__ dO,
    const float *__restrict__ LSE, const float *__restrict__ delta, float *__restrict__ dK,
    float *__restrict__ dV, int Hs, int Hks, int G, int64_t Ns, float scale, float scale_log2,
    int causal, int window) {
  constexpr int RS = DkvBuf<D, DV>::RS, RSV = DkvBuf<D, DV>::RSV;
  constexpr int BQ = kBwdBQ;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int h = lane >> 5, l32 = lane & 31;
  // the item's head is a query head; with grouped K/V heads (G > 1) its
  // K/V head is it.head / G, and the group's items add into dK and dV
  const int64_t rs = (int64_t)Hs * D;     // Q elements between consecutive slots
  const int64_t rso = (int64_t)Hs * DV;   // dO
  const int64_t rsk = (int64_t)Hks * D;   // K / dK
  const int64_t rsv = (int64_t)Hks * DV;  // V / dV
  const int64_t ho = (int64_t)it.head * D, hoo = (int64_t)it.head * DV;
  const int64_t hk = (int64_t)(it.head / G) * D, hv = (int64_t)(it.head / G) * DV;
  const int wk0 = it.q0 + 32 * w, wk1 = min(wk0 + 32, it.q1);
  const int kj = wk0 + l32;  // this lane's key (column of S)
  const bool kok = kj < it.q1;
  const int trl_q = tr_lane(h, l32, RS), trl_g = tr_lane(h, l32, RSV);
  // with both widths 128 the two 32-query halves of a tile run one after the
  // other (no overlap): the registers hold only one half's S and dP next to
  // the dK/dV accumulators (fewer spills, 2-10% faster; with mixed widths the
  // overlap wins by 2%)
  constexpr int RHO_UNROLL = D == 128 && DV == 128 ? 1 : 2;

  bf16x8 kf[D / 16], vf[DV / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    if (kok) {
      kf[c] = load_bf16x8(K + hk + kj * rsk + 16 * c + 8 * h);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[c][e] = (__bf16)0.0f;
    }
  }
#pragma unroll
  for (int c = 0; c < DV / 16; ++c) {
    if (kok) {
      vf[c] = load_bf16x8(V + hv + kj * rsv + 16 * c + 8 * h);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) vf[c][e] = (__bf16)0.0f;
    }
  }
  floatx16 dv[DV / 32], dk[D / 32];
#pragma unroll
  for (int dl = 0; dl < DV / 32; ++dl) dv[dl] = floatx16{};
#pragma unroll
  for (int dl = 0; dl < D / 32; ++dl) dk[dl] = floatx16{};

  const int nq = (it.k1 - it.k0 + BQ - 1) / BQ;
  static_assert(BQ == 64, "one DMA instruction per 64-row chunk column");
  const uint32_t rsb = (uint32_t)rs * 2u, rsbo = (uint32_t)rso * 2u;
  float st_lse = 0.0f;
  // start the loads of query tile q0 into bf (Q, dO straight into LDS; the
  // LSE / -D values into a register)
  auto issue = [&](DkvBuf<D, DV> &bf, int q0) {
    const uint32_t n = (uint32_t)max(0, min(it.k1 - q0, BQ));
    const auto rq = make_rsrc(Q + ho + (int64_t)q0 * rs, n * rsb);
    const auto rg = make_rsrc(dO + hoo + (int64_t)q0 * rso, n * rsbo);
    constexpr int NQ = DmaTile<D>::NI, NG = DmaTile<DV>::NI;
    const int ln = offset_lane<D, DV>(lane);
    if constexpr (D == DV) {
      // equal widths: Q and dO rows have the same stride (heads x width), so
      // chunk column j of both tiles uses one offset
#pragma unroll
      for (int j0 = 0; j0 < NQ; j0 += NW) {
        const int j = j0 + w;
        if (j < NQ) {
          const uint32_t off = DmaTile<D>::offset(j, ln, rsb);
          dma16(rq, &bf.q[512 * j], off);
          dma16(rg, &bf.g[512 * j], off);
        }
      }
    } else {
#pragma unroll
      for (int j0 = 0; j0 < NQ + NG; j0 += NW) {
        const int j = j0 + w;
        if (j < NQ) dma16(rq, &bf.q[512 * j], DmaTile<D>::offset(j, ln, rsb));
        else if (j < NQ + NG)
          dma16(rg, &bf.g[512 * (j - NQ)], DmaTile<DV>::offset(j - NQ, ln, rsbo));
      }
    }
    if (tid < 2 * BQ) {
      const int row = q0 + (tid % BQ);
      st_lse = row < it.k1 ? (tid < BQ ? LSE[(int64_t)it.head * Ns + row] * kLog2e
                                       : -delta[(int64_t)it.head * Ns + row])
                           : 0.0f;
    }
  };
  // store the register part and wait for this wave's LDS loads
  auto finish = [&](DkvBuf<D, DV> &bf) {
    if (tid < BQ) bf.lse2[tid] = st_lse;
    else if (tid < 2 * BQ) bf.dl[tid - BQ] = st_lse;
    wait_dma();
  };
  issue(sm.b[0], it.k0);
  finish(sm.b[0]);
  __syncthreads();
  for (int t = 0; t < nq; ++t) {
    const int qt0 = it.k0 + t * BQ;
    const DkvBuf<D, DV> &cur = sm.b[t & 1];
    if (t + 1 < nq) issue(sm.b[(t + 1) & 1], qt0 + BQ);
    const int qt1 = min(qt0 + BQ, it.k1);  // one past the last valid query
    const bool active = wk0 < wk1 && !(causal && qt1 - 1 < wk0) &&
                        !(window > 0 && qt0 - (wk1 - 1) >= window);
    if (active) {
    const bool full = (qt0 + BQ <= it.k1) && (!causal || wk1 - 1 <= qt0) &&
                      (window <= 0 || (qt0 + BQ - 1) - wk0 < window);
    // query rows (tile-relative) that see this lane's key: [qlo, qhi]; the
    // lane's key itself may be past the item end -- its column is never stored
    const int qlo = causal ? kj - qt0 : -(1 << 30);
    const int qhi = min(it.k1 - 1, window > 0 ? kj + window - 1 : (1 << 30)) - qt0;
#pragma unroll RHO_UNROLL
    for (int rho = 0; rho < BQ / 32; ++rho) {
      // rows of s: query 32*rho + 8b + 4h + i of the tile; column: key kj.
      // dP starts from -D of its rows, so the MFMA leaves dP - D.
      floatx16 s = {}, dp;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float4 d4 = *reinterpret_cast<const float4 *>(&cur.dl[32 * rho + 8 * b + 4 * h]);
        dp[4 * b] = d4.x;
        dp[4 * b + 1] = d4.y;
        dp[4 * b + 2] = d4.z;
        dp[4 * b + 3] = d4.w;
      }
      // S first: its exponentials can start while dP is multiplied
      mfma_priority<D, DV, 1>();
#pragma unroll
      for (int c = 0; c < D / 16; ++c)
        s = mfma32x32x16(load_bf16x8(&cur.q[(32 * rho + l32) * RS + 16 * c + 8 * h]), kf[c], s);
#pragma unroll
      for (int c = 0; c < DV / 16; ++c)
        dp = mfma32x32x16(load_bf16x8(&cur.g[(32 * rho + l32) * RSV + 16 * c + 8 * h]), vf[c], dp);
      mfma_priority<D, DV, 0>();
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float4 l4 = *reinterpret_cast<const float4 *>(&cur.lse2[32 * rho + 8 * b + 4 * h]);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) s[4 * b + i] = fast_exp2(fmaf(s[4 * b + i], scale_log2, -lv[i]));
      }
      if (!full) {  // tiles on the diagonal, the window edge or the range end
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = 32 * rho + 8 * (r / 4) + 4 * h + (r % 4);
          if (q > qhi || q < qlo) s[r] = 0.0f;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) dp[r] *= s[r];
      const bf16x8 pa[2] = {to_bf16x8(s, 0), to_bf16x8(s, 8)};
      const bf16x8 da[2] = {to_bf16x8(dp, 0), to_bf16x8(dp, 8)};
#pragma unroll
      for (int dl = 0; dl < (D > DV ? D : DV) / 32; ++dl)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          // B operands dO and Q with the query order of pa / da, read
          // transposed from the row-major tiles
          const int row = 32 * rho + 16 * m;
          if (dl < DV / 32)
            dv[dl] = mfma32x32x16(pa[m], tr_operand(&cur.g[trl_g + row * RSV + 32 * dl], RSV),
                                  dv[dl]);
          if (dl < D / 32)
            dk[dl] = mfma32x32x16(da[m], tr_operand(&cur.q[trl_q + row * RS + 32 * dl], RS),
                                  dk[dl]);
        }
    }
    }
    if (t + 1 < nq) finish(sm.b[(t + 1) & 1]);
    __syncthreads();
  }
  // epilogue: accumulator rows are keys 8b + 4h + i of the wave, columns d
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = wk0 + 8 * (r / 4) + 4 * h + (r % 4);
    if (key < it.q1) {
      // with grouped heads, the group's query heads share this K/V row
      // (zeroed first) and add into it
#pragma unroll
      for (int dl = 0; dl < DV / 32; ++dl) {
        const int64_t off = key * rsv + hv + 32 * dl + l32;
        if (G == 1) dV[off] = dv[dl][r];
        else unsafeAtomicAdd(&dV[off], dv[dl][r]);
      }
#pragma unroll
      for (int dl = 0; dl < D / 32; ++dl) {
        const int64_t off = key * rsk + hk + 32 * dl + l32;
        if (G == 1) dK[off] = dk[dl][r] * scale;
        else unsafeAtomicAdd(&dK[off], dk[dl][r] * scale);
      }
    }
  }
}

// -------------------------------------------------------------------- dQ --

template <int D, int DV>
struct DqBuf {
  static constexpr int RS = D + 8, RSV = DV + 8;
  __bf16 k[kFwdBK * RS];
  __bf16 v[kFwdBK * RSV];
};
template <int D, int DV>
struct DqSmem {
  DqBuf<D, DV> b[2];  // double buffered: one barrier per key tile
};

// One dQ item (queries [q0, q1), keys [k0, k1)).
template <int D, int DV, int NW>
__device__ __forceinline__ void dq_item(
    const WorkItem it, DqSmem<D, DV> &sm, const __bf16 *__restrict__ Q,
    const __bf16 *__restrict__ K, const __bf16 *__restrict__ V, const __bf16 *__restrict__ dO,
    const float *__restrict__ LSE, const float *__restrict__ delta, float *__restrict__ dQ,
    int Hs, int Hks, int G, int64_t Ns, float scale, float scale_log2, int causal, int window) {
  constexpr int RS = DqBuf<D, DV>::RS, RSV = DqBuf<D, DV>::RSV;
  constexpr int BK = kFwdBK;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t rs = (int64_t)Hs * D;     // Q / dQ elements between consecutive slots
  const int64_t rso = (int64_t)Hs * DV;   // dO
  const int64_t rsk = (int64_t)Hks * D;   // K
  const int64_t rsv = (int64_t)Hks * DV;  // V
  const int64_t ho = (int64_t)it.head * D, hoo = (int64_t)it.head * DV;
  // the query head's K/V head
  const int64_t hk = (int64_t)(it.head / G) * D, hv = (int64_t)(it.head / G) * DV;
  const int wq0 = it.q0 + 32 * w, wq1 = min(wq0 + 32, it.q1);
  const int qi = wq0 + l32;
  const bool qok = qi < it.q1;
  const int trl_k = tr_lane(h, l32, RS);

  bf16x8 qf[D / 16], gf[DV / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    if (qok) {
      qf[c] = load_bf16x8(Q + ho + qi * rs + 16 * c + 8 * h);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[c][e] = (__bf16)0.0f;
    }
  }
#pragma unroll
  for (int c = 0; c < DV / 16; ++c) {
    if (qok) {
      gf[c] = load_bf16x8(dO + hoo + qi * rso + 16 * c + 8 * h);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) gf[c][e] = (__bf16)0.0f;
    }
  }
  const float lse2 = qok ? LSE[(int64_t)it.head * Ns + qi] * kLog2e : 0.0f;
  // -D of this lane's query: the start value of every dP accumulator, so the
  // MFMA leaves dP - D
  floatx16 negd;
  {
    const float dd = qok ? delta[(int64_t)it.head * Ns + qi] : 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) negd[r] = -dd;
  }
  floatx16 dq[D / 32];
#pragma unroll
  for (int dl = 0; dl < D / 32; ++dl) dq[dl] = floatx16{};

  const int nk = (it.k1 - it.k0 + BK - 1) / BK;
  static_assert(BK == 64, "one DMA instruction per 64-row chunk column");
  const uint32_t rsbk = (uint32_t)rsk * 2u, rsbv = (uint32_t)rsv * 2u;
  // start the loads of key tile k0 into bf (K, V straight into LDS)
  auto issue = [&](DqBuf<D, DV> &bf, int k0) {
    const uint32_t n = (uint32_t)max(0, min(it.k1 - k0, BK));
    const auto rk = make_rsrc(K + hk + (int64_t)k0 * rsk, n * rsbk);
    const auto rv = make_rsrc(V + hv + (int64_t)k0 * rsv, n * rsbv);
    constexpr int NK = DmaTile<D>::NI, NV = DmaTile<DV>::NI;
    const int ln = offset_lane<D, DV>(lane);
    if constexpr (D == DV) {
#pragma unroll
      for (int j0 = 0; j0 < NK; j0 += NW) {
        const int j = j0 + w;
        if (j < NK) {  // K and V rows: the same stride at equal widths
          const uint32_t off = DmaTile<D>::offset(j, ln, rsbk);
          dma16(rk, &bf.k[512 * j], off);
          dma16(rv, &bf.v[512 * j], off);
        }
      }
    } else {
#pragma unroll
      for (int j0 = 0; j0 < NK + NV; j0 += NW) {
        const int j = j0 + w;
        if (j < NK) dma16(rk, &bf.k[512 * j], DmaTile<D>::offset(j, ln, rsbk));
        else if (j < NK + NV)
          dma16(rv, &bf.v[512 * (j - NK)], DmaTile<DV>::offset(j - NK, ln, rsbv));
      }
    }
  };
  issue(sm.b[0], it.k0);
  wait_dma();
  __syncthreads();
  for (int t = 0; t < nk; ++t) {
    const int kt0 = it.k0 + t * BK;
    const DqBuf<D, DV> &cur = sm.b[t & 1];
    if (t + 1 < nk) issue(sm.b[(t + 1) & 1], kt0 + BK);
    const bool active = wq0 < wq1 && !(causal && kt0 > wq1 - 1) &&
                        !(window > 0 && wq0 - (kt0 + BK - 1) >= window);
    if (active) {
    const bool full = (kt0 + BK <= it.k1) && (!causal || kt0 + BK - 1 <= wq0) &&
                      (window <= 0 || (wq1 - 1) - kt0 < window);
    // keys (relative to kt0 + 4h) this lane's query sees: [klo, khi]; the
    // lane's query may be past the item end -- its row is never stored
    const int kb = kt0 + 4 * h;
    const int khi = (causal ? min(it.k1 - 1, qi) : it.k1 - 1) - kb;
    const int klo = window > 0 ? qi - window + 1 - kb : -(1 << 30);
    floatx16 s[2], dp[2];
#pragma unroll
    for (int beta = 0; beta < 2; ++beta) {
      s[beta] = floatx16{};
      dp[beta] = negd;
      mfma_priority<D, DV, 1>();
#pragma unroll
      for (int c = 0; c < D / 16; ++c)
        s[beta] = mfma32x32x16(load_bf16x8(&cur.k[(32 * beta + l32) * RS + 16 * c + 8 * h]), qf[c],
                               s[beta]);
#pragma unroll
      for (int c = 0; c < DV / 16; ++c)
        dp[beta] = mfma32x32x16(load_bf16x8(&cur.v[(32 * beta + l32) * RSV + 16 * c + 8 * h]),
                                gf[c], dp[beta]);
      mfma_priority<D, DV, 0>();
#pragma unroll
      for (int r = 0; r < 16; ++r) s[beta][r] = fast_exp2(fmaf(s[beta][r], scale_log2, -lse2));
      if (!full) {  // tiles on the diagonal, the window edge or the range end
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rel = 32 * beta + 8 * (r / 4) + (r % 4);
          if (rel > khi || rel < klo) s[beta][r] = 0.0f;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) dp[beta][r] *= s[beta][r];
    }
#pragma unroll
    for (int dl = 0; dl < D / 32; ++dl)
#pragma unroll
      for (int beta = 0; beta < 2; ++beta)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          // K^T rows with the key order of dp, read transposed from the K tile
          const bf16x8 a = tr_operand(&cur.k[trl_k + (32 * beta + 16 * m) * RS + 32 * dl], RS);
          dq[dl] = mfma32x32x16(a, to_bf16x8(dp[beta], 8 * m), dq[dl]);
        }
    }
    if (t + 1 < nk) wait_dma();
    __syncthreads();
  }
  if (qok) {
    float *row = dQ + qi * rs + ho;
#pragma unroll
    for (int dl = 0; dl < D / 32; ++dl)
#pragma unroll
      for (int b = 0; b < 4; ++b)
        *reinterpret_cast<float4 *>(row + 32 * dl + 8 * b + 4 * h) =
            make_float4(dq[dl][4 * b] * scale, dq[dl][4 * b + 1] * scale,
                        dq[dl][4 * b + 2] * scale, dq[dl][4 * b + 3] * scale);
  }
}

// Both passes in one launch: blocks [0, n_dkv) run the dK/dV items, the rest
// the dQ items, so the dQ work fills the CUs the dK/dV tail leaves idle.  The
// two share one LDS allocation (the larger of the two layouts).
template <int D, int DV, int NW>
__global__ __launch_bounds__(64 * NW, (bwd_waves_per_simd<D, DV>())) void bwd_kernel(
    const WorkItem *__restrict__ dkv_items, int n_dkv, const WorkItem *__restrict__ dq_items,
    const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K, const __bf16 *__restrict__ V,
    const __bf16 *__restrict__ dO, const float *__restrict__ LSE, const float *__restrict__ delta,
    float *__restrict__ dQ, float *__restrict__ dK, float *__restrict__ dV, int Hs, int Hks, int G,
    int64_t Ns, float scale, float scale_log2, int causal, int window) {
  __shared__ __attribute__((aligned(16))) union {
    DkvSmem<D, DV> kv;
    DqSmem<D, DV> q;
  } sm;
  const int b = (int)blockIdx.x;
  if (b < n_dkv)
    dkv_item<D, DV, NW>(dkv_items[b], sm.kv, Q, K, V, dO, LSE, delta, dK, dV, Hs, Hks, G, Ns,
                        scale, scale_log2, causal, window);
  else
    dq_item<D, DV, NW>(dq_items[b - n_dkv], sm.q, Q, K, V, dO, LSE, delta, dQ, Hs, Hks, G, Ns,
                       scale, scale_log2, causal, window);
}

// Zero na floats of a and nb of b (dK and dV before the grouped heads add
// into them; a kernel rather than a memset, so the launch sequence stays
// graph-capturable).
__global__ __launch_bounds__(256) void zero_kernel(float *__restrict__ a, int64_t na,
                                                   float *__restrict__ b, int64_t nb) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < na) a[i] = 0.0f;
  if (i < nb) b[i] = 0.0f;
}

template <int D, int DV = D>
hipError_t launch_typed(const attn_plan *p, const void *q, const void *k, const void *v,
                        const void *o, const float *lse, const void *d_o, float *dq, float *dk,
                        float *dv, float *delta, hipStream_t stream) {
  const int Hs = p->p.Hs;
  const int64_t Ns = p->p.Ns;
  const float scale = p->p.scale, scale_log2 = p->p.scale * kLog2e;
  const __bf16 *Q = static_cast<const __bf16 *>(q), *K = static_cast<const __bf16 *>(k);
  const __bf16 *V = static_cast<const __bf16 *>(v), *O = static_cast<const __bf16 *>(o);
  const __bf16 *G = static_cast<const __bf16 *>(d_o);
  const int64_t rows = Ns * Hs;
  constexpr int NWK = bwd_waves(D, DV), NWQ = NWK;
  hipLaunchKernelGGL((delta_kernel<DV>), dim3((unsigned)((rows + 255) / 256)), dim3(256), 0,
                     stream, O, G, delta, Hs, Ns);
  if (p->p.G > 1) {
    const int64_t nk = p->p.Ns * p->p.Hks * D, nv = p->p.Ns * p->p.Hks * DV;
    const int64_t n = nk > nv ? nk : nv;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, dk,
                       nk, dv, nv);
  }
  static_assert(NWK == NWQ, "one launch runs both passes");
  const unsigned nb = (unsigned)(p->bwd.size() + p->dq.size());
  if (nb > 0)
    hipLaunchKernelGGL((bwd_kernel<D, DV, NWK>), dim3(nb), dim3(64 * NWK), 0, stream,
                       reinterpret_cast<const WorkItem *>(p->ws + p->off_bwd), (int)p->bwd.size(),
                       reinterpret_cast<const WorkItem *>(p->ws + p->off_dq), Q, K, V, G, lse,
                       delta, dq, dk, dv, Hs, p->p.Hks, p->p.G, Ns, scale, scale_log2,
                       p->p.causal, p->p.window);
  return hipGetLastError();
}

}  // namespace

attn_status launch_bwd(const attn_plan *p, const void *q, const void *k, const void *v,
                       const void *o, const float *lse, const void *d_o, float *dq, float *dk,
                       float *dv, float *delta, hipStream_t stream) {
  const int d = p->p.d, w = p->p.dv;
  hipError_t e;
  if (d == 64 && w == 64) e = launch_typed<64>(p, q, k, v, o, lse, d_o, dq, dk, dv, delta, stream);
  else if (d == 64) e = launch_typed<64, 128>(p, q, k, v, o, lse, d_o, dq, dk, dv, delta, stream);
  else if (w == 64) e = launch_typed<128, 64>(p, q, k, v, o, lse, d_o, dq, dk, dv, delta, stream);
  else e = launch_typed<128>(p, q, k, v, o, lse, d_o, dq, dk, dv, delta, stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

}  // namespace attn

// ------------------------------------------------------- allocation-free --
// The backward's only scratch is D (one float per attention head and slot).
// attn_bwd_noalloc keeps it in this array instead of the plan's workspace,
// for callers that cannot allocate.  Each GPU the library runs on holds its
// own copy until the process ends; host code uses the address that
// hipGetSymbolAddress returns for the current device, never the name itself
// (a host-side stand-in).
static __device__ __align__(256) float scratch[attn::kNoallocScratchBytes / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float *g_scratch[kMaxDevices] = {};  // device address of `scratch`, per device

// The address of `scratch` on the device that `stream` runs on (the current
// device for the null stream), looked up once per device with that device
// current.
hipError_t scratch_on(hipStream_t stream, float **out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream != nullptr && (e = hipStreamGetDevice(stream, &dev)) != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return e;
    g_scratch[dev] = static_cast<float *>(ptr);
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" attn_status attn_bwd_noalloc(const attn_plan *p, const void *q, const void *k,
                                        const void *v, const void *o, const float *lse,
                                        const void *d_o, float *dq, float *dk, float *dv,
                                        void *stream) {
  const attn_status st = attn::check_bwd_args(p, q, k, v, o, lse, d_o, dq, dk, dv);
  if (st != ATTN_OK || p->p.N == 0) return st;
  if ((size_t)p->p.Hs * (size_t)p->p.Ns * sizeof(float) > attn::kNoallocScratchBytes)
    return ATTN_E_WORKSPACE;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  float *delta = nullptr;
  if (scratch_on(hs, &delta) != hipSuccess) return ATTN_E_HIP;
  return attn::launch_bwd(p, q, k, v, o, lse, d_o, dq, dk, dv, delta, hs);
}
