// attn_fwd.hip -- flash-style causal / windowed / varlen attention forward for
// gfx950 (MI355X), on MFMA matrix cores.
//
// What it computes: O = softmax(s Q K^T + mask) V and LSE = log sum exp per
// query row, per attention head, with the mask of the plan (same sequence,
// causal, window of W key slots), exactly the plain definition
// ("mHC module" article, lshu.cn, section 2.1; "SingleHeadAttention" note,
// ranhao.site, forward()).  The N' x N' score matrix is never written to HBM:
// it is produced tile by tile on chip with a running max and sum
// ("Upgrading a textbook decoder", juejin.cn, section 4, FlashAttention: the
// tiling changes where the result is computed, not the result).
//
// gfx950 mapping (one work item = one block of 8 waves = 256 query slots of
// one attention head for bf16, 4 waves = 128 slots for fp32, for windows of
// at most 512 slots, when every sequence fits 2048 slots and at head widths
// of 64; each wave owns 32 query slots, and every K/V tile staged in LDS
// serves the whole block):
//   * Each wave holds its 32 queries as the B operand of
//     v_mfma_f32_32x32x16_bf16 for the whole item (registers).
//   * K tiles of 64 key slots are staged in LDS row-major.  V tiles are staged
//     transposed (V^T, d-major) for eight-wave items, row-major for four-wave
//     items, which read V^T with ds_read_b64_tr_b16 (see SmemBF).
//   * S^T = K Q^T: with keys as MFMA rows and queries as columns, every lane of
//     the accumulator holds one query's scores, so the row max and row sum are
//     in-lane reductions plus one exchange between the two half-waves.
//   * P^T goes straight from the accumulator registers to the B operand of
//     O^T += V^T P^T (no LDS round trip): V^T is read with its keys in the
//     order in which the accumulator holds them (bits 2 and 3 of the key
//     index swapped inside each group of 16).
//   * exp uses v_exp_f32 (2^x) with log2(e) folded into the scale; masking is
//     applied only on tiles that cross the causal diagonal, the window edge or
//     the end of the key range; tiles masked for a whole wave are skipped.
// The fp32 problem uses the same schedule on v_mfma_f32_32x32x2_f32, whose
// operands hold one element per lane, so no transposed staging is needed.
#include <type_traits>

#include "attn_internal.h"
#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int BK = kFwdBK;  // key slots per step
constexpr float kMinusBig = -1e30f;  // finite start value of the running max

template <typename T, int D>
struct Smem;
template <int D>
struct Smem<float, D> {
  static constexpr int KS = D + 1;   // odd stride: column reads hit 32 different banks
  static constexpr int VS = D + 4;
  float k[BK * KS];
  float v[BK * VS];
};

// Global -> register staging of one K/V tile.
template <typename T, int D>
struct Stage;

template <int D>
struct Stage<float, D> {
  static constexpr int PT = BK * D / 4 / kFwdThreadsF32;  // float4 chunks per thread (K and V)
  float4 kr[PT];
  float4 vr[PT];

  __device__ __forceinline__ void load(const float *Kh, const float *Vh, int64_t rs, int kt0,
                                       int k1, int tid) {
#pragma unroll
    for (int r = 0; r < PT; ++r) {
      const int ci = tid + kFwdThreadsF32 * r;
      const int key = ci / (D / 4), c4 = ci % (D / 4);
      const int slot = kt0 + key;
      const bool ok = slot < k1;
      kr[r] = ok ? *reinterpret_cast<const float4 *>(Kh + slot * rs + 4 * c4)
                 : make_float4(0.f, 0.f, 0.f, 0.f);
      vr[r] = ok ? *reinterpret_cast<const float4 *>(Vh + slot * rs + 4 * c4)
                 : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }

  __device__ __forceinline__ void store(Smem<float, D> &sm, int tid) {
    constexpr int KS = Smem<float, D>::KS, VS = Smem<float, D>::VS;
#pragma unroll
    for (int r = 0; r < PT; ++r) {
      const int ci = tid + kFwdThreadsF32 * r;
      const int key = ci / (D / 4), c4 = ci % (D / 4);
      float *kd = &sm.k[key * KS + 4 * c4];
      kd[0] = kr[r].x;
      kd[1] = kr[r].y;
      kd[2] = kr[r].z;
      kd[3] = kr[r].w;
      *reinterpret_cast<float4 *>(&sm.v[key * VS + 4 * c4]) = vr[r];
    }
  }
};

// The wave's 32 queries as the MFMA B operand (k = feature index).
template <typename T, int D>
struct QFrag;
template <int D>
struct QFrag<float, D> {
  float f[D / 2];
  __device__ __forceinline__ void load(const float *Qh, int64_t rs, int qi, bool ok, int h) {
#pragma unroll
    for (int c = 0; c < D / 2; ++c) f[c] = ok ? Qh[qi * rs + 2 * c + h] : 0.0f;
  }
  __device__ __forceinline__ floatx16 scores(const Smem<float, D> &sm, int beta, int l32,
                                             int h) const {
    constexpr int KS = Smem<float, D>::KS;
    floatx16 acc = {};
#pragma unroll
    for (int c = 0; c < D / 2; ++c)
      acc = mfma32x32x2f32(sm.k[(32 * beta + l32) * KS + 2 * c + h], f[c], acc);
    return acc;
  }
};

// O^T += V^T P^T for the staged tile; p[beta][r] holds the probabilities of
// key 32*beta + 8*(r/4) + 4*h + r%4 for this lane's query.
template <int D>
__device__ __forceinline__ void accumulate_pv(const Smem<float, D> &sm, const floatx16 (&p)[2],
                                              floatx16 (&o)[D / 32], int l32, int h) {
  constexpr int VS = Smem<float, D>::VS;
#pragma unroll
  for (int dl = 0; dl < D / 32; ++dl)
#pragma unroll
    for (int beta = 0; beta < 2; ++beta)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * beta + 8 * (r / 4) + 4 * h + (r % 4);
        o[dl] = mfma32x32x2f32(sm.v[key * VS + 32 * dl + l32], p[beta][r], o[dl]);
      }
}

template <typename T>
__device__ __forceinline__ void store4(T *dst, const float *x);
template <>
__device__ __forceinline__ void store4<__bf16>(__bf16 *dst, const float *x) {
  *reinterpret_cast<uint2 *>(dst) = make_uint2(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]));
}
template <>
__device__ __forceinline__ void store4<float>(float *dst, const float *x) {
  *reinterpret_cast<float4 *>(dst) = make_float4(x[0], x[1], x[2], x[3]);
}

// Two blocks per CU for bf16 (8 waves, <= 256 VGPRs each); the fp32 variant
// holds its queries as D/2 fp32 registers and runs one block per CU.
template <typename T>
constexpr int fwd_min_blocks() {
  return std::is_same<T, float>::value ? 1 : 2;
}

template <typename T, int D>
__global__ __launch_bounds__(kFwdThreadsF32, fwd_min_blocks<T>()) void fwd_kernel(
    const WorkItem *__restrict__ items, const T *__restrict__ Q, const T *__restrict__ K,
    const T *__restrict__ V, T *__restrict__ O, float *__restrict__ LSE, int Hs, int Hks, int G, int64_t Ns,
    float scale, float scale_log2, int causal, int window) {
  __shared__ __attribute__((aligned(16))) Smem<T, D> sm;
  const WorkItem it = items[blockIdx.x];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t rs = (int64_t)Hs * D;    // Q / O elements between consecutive slots
  const int64_t rsk = (int64_t)Hks * D;  // K / V elements between consecutive slots
  const T *Qh = Q + (int64_t)it.head * D;
  const T *Kh = K + (int64_t)(it.head / G) * D;  // the query head's K/V head
  const T *Vh = V + (int64_t)(it.head / G) * D;

  const int wq0 = it.q0 + 32 * w;             // first query of this wave
  const int wq1 = min(wq0 + 32, it.q1);        // one past its last valid query
  const int qi = wq0 + l32;                    // this lane's query
  const bool qok = qi < it.q1;

  QFrag<T, D> qf;
  qf.load(Qh, rs, qi, qok, h);

  floatx16 o[D / 32];
#pragma unroll
  for (int dl = 0; dl < D / 32; ++dl) o[dl] = floatx16{};
  float m = kMinusBig;  // running max of raw scores q.k
  float l = 0.0f;       // this lane's part of the running sum

  const int nk = (it.k1 - it.k0 + BK - 1) / BK;
  Stage<T, D> st;
  st.load(Kh, Vh, rsk, it.k0, it.k1, tid);
  for (int t = 0; t < nk; ++t) {
    const int kt0 = it.k0 + t * BK;
    __syncthreads();
    st.store(sm, tid);
    __syncthreads();
    if (t + 1 < nk) st.load(Kh, Vh, rsk, kt0 + BK, it.k1, tid);

    // wave-uniform tile classification
    const bool active = wq0 < wq1 && !(causal && kt0 > wq1 - 1) &&
                        !(window > 0 && wq0 - (kt0 + BK - 1) >= window);
    if (!active) continue;
    const bool full = (kt0 + BK <= it.k1) && (!causal || kt0 + BK - 1 <= wq0) &&
                      (window <= 0 || (wq1 - 1) - kt0 < window);

    floatx16 s[2];
    s[0] = qf.scores(sm, 0, l32, h);
    s[1] = qf.scores(sm, 1, l32, h);
    if (!full) {
#pragma unroll
      for (int beta = 0; beta < 2; ++beta)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kj = kt0 + 32 * beta + 8 * (r / 4) + 4 * h + (r % 4);
          const bool vis = kj < it.k1 && (!causal || kj <= qi) && (window <= 0 || qi - kj < window);
          if (!vis) s[beta][r] = -INFINITY;
        }
    }
    // online softmax: new max, rescale, probabilities
    float mx = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    mx = halves_max(mx);
    const float m_new = fmaxf(m, mx);
    const float alpha = exp2f((m - m_new) * scale_log2);
    m = m_new;
    const float mb = m_new * scale_log2;
    float ls = 0.0f;
#pragma unroll
    for (int beta = 0; beta < 2; ++beta)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = exp2f(fmaf(s[beta][r], scale_log2, -mb));
        s[beta][r] = pv;
        ls += pv;
      }
    l = fmaf(l, alpha, ls);
#pragma unroll
    for (int dl = 0; dl < D / 32; ++dl)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dl][r] *= alpha;
    accumulate_pv<D>(sm, s, o, l32, h);
  }

  // epilogue: O = O^T / l, LSE = s * m + ln l
  const float lt = halves_sum(l);
  if (qok) {
    const float inv = 1.0f / lt;
    T *orow = O + (int64_t)qi * rs + (int64_t)it.head * D;
#pragma unroll
    for (int dl = 0; dl < D / 32; ++dl)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = o[dl][4 * b + i] * inv;
        store4<T>(orow + 32 * dl + 8 * b + 4 * h, x);
      }
    if (h == 0) LSE[(int64_t)it.head * Ns + qi] = m * scale + logf(lt);
  }
}

// ------------------------------------------------------------------ bf16 --
// The production kernel (bf16 I/O, fp32 accumulate).  Differences from the
// generic schedule above: K/V/Q come in through raw buffer loads whose
// resource ends at the item's last key, so a ragged tail reads zeros without
// branches and the per-tile address update is scalar; LDS is double-buffered
// (one barrier per key tile); the reference max of the exponentials is taken
// on a wave's first tile and only moved when a lane's weights of a tile sum
// past 2^64 (a score more than 64 above the reference in the exp2 domain), so
// weights stay below 2^64 and sums of them far below the fp32 range, and
// O / l and LSE do not depend on where the reference sits.

// D: width of Q and K rows; DV: width of V and O rows.  K is kept row-major
// (one key per row).  V has two layouts (VT):
//   VT = true:  V^T, the key order permuted to the order the S accumulator
//               holds (perm16), so one 16-byte read gives the PV A operand;
//               staging it costs eight 4-byte stores and byte permutes per
//               16 bytes.
//   VT = false: row-major like K (one 16-byte store), read transposed with
//               two ds_read_b64_tr_b16, which run at half the rate of
//               16-byte reads.
// Eight-wave items read every staged tile eight times and use VT = true;
// four-wave items (short windows, short sequences, head widths of 64) use
// VT = false, where the cheaper store wins (10% on the paired window-128
// problem; the other way round costs 3-7% on eight-wave items).
template <int D, int DV, bool VT>
struct SmemBF {
  static constexpr int KS = D + 8;                 // K row stride (elements): 4-bank shift
  static constexpr int VS = VT ? BK + 8 : DV + 8;  // V^T or V row stride (elements)
  __bf16 k[2][BK * KS];
  __bf16 v[2][VT ? DV * VS : BK * VS];
};

template <int D, int DV, int NT, bool VT>
struct StageBF {
  static constexpr int KPT = BK * D / 8 / NT;  // 16-byte K chunks per thread
  static_assert(KPT >= 1 && BK * D / 8 % NT == 0, "K staging split");
  // V units: (key pair, 8 features) for VT, else 16-byte chunks of one key
  static constexpr int VR = VT ? 2 : 1;  // rows per unit
  static constexpr int VU = (BK / VR) * (DV / 8);
  static constexpr int VPT = (VU + NT - 1) / NT;
  uint4 kr[KPT];
  uint4 vr[VPT][VR];

  // Rows [kt0, kt0 + BK) of the head's K and V (row strides rsb, rsbv bytes);
  // rows past `rows` read zero.
  __device__ __forceinline__ void load(const __bf16 *Kt, const __bf16 *Vt, int rows, uint32_t rsb,
                                       uint32_t rsbv, int tid) {
    const uint32_t nr = (uint32_t)max(0, min(rows, BK));
    const auto rk = make_rsrc(Kt, nr * rsb);
    const auto rv = make_rsrc(Vt, nr * rsbv);
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int ci = tid + NT * r;
      kr[r] = buf_load16(rk, (uint32_t)(ci / (D / 8)) * rsb + 16u * (ci % (D / 8)));
    }
#pragma unroll
    for (int r = 0; r < VPT; ++r) {
      const int vi = tid + NT * r;
      if (VU % NT != 0 && vi >= VU) break;
      if (VT) {
        const uint32_t off = (uint32_t)(2 * (vi % (BK / 2))) * rsbv + 16u * (vi / (BK / 2));
        vr[r][0] = buf_load16(rv, off);
        vr[r][VR - 1] = buf_load16(rv, off + rsbv);
      } else {
        vr[r][0] = buf_load16(rv, (uint32_t)(vi / (DV / 8)) * rsbv + 16u * (vi % (DV / 8)));
      }
    }
  }

  __device__ __forceinline__ void store(__bf16 *kdst, __bf16 *vdst, int tid) const {
    constexpr int KS = SmemBF<D, DV, VT>::KS, VS = SmemBF<D, DV, VT>::VS;
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int ci = tid + NT * r;
      *reinterpret_cast<uint4 *>(&kdst[(ci / (D / 8)) * KS + 8 * (ci % (D / 8))]) = kr[r];
    }
#pragma unroll
    for (int r = 0; r < VPT; ++r) {
      const int vi = tid + NT * r;
      if (VU % NT != 0 && vi >= VU) break;
      if (VT) {
        const int kp = vi % (BK / 2), c8 = vi / (BK / 2);
        const int pos = perm16(2 * kp);  // even; key 2kp+1 lands at pos + 1
        const uint4 &ra = vr[r][0], &rb = vr[r][VR - 1];
        const uint32_t a[4] = {ra.x, ra.y, ra.z, ra.w};
        const uint32_t b[4] = {rb.x, rb.y, rb.z, rb.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t word = (e & 1) ? __byte_perm(a[e / 2], b[e / 2], 0x7632)
                                        : __byte_perm(a[e / 2], b[e / 2], 0x5410);
          *reinterpret_cast<uint32_t *>(&vdst[(8 * c8 + e) * VS + pos]) = word;
        }
      } else {
        *reinterpret_cast<uint4 *>(&vdst[(vi / (DV / 8)) * VS + 8 * (vi % (DV / 8))]) = vr[r][0];
      }
    }
  }
};

constexpr float kOverflow = 18446744073709551616.0f;  // 2^64

// Causal / window / key-range mask of one 64-key tile for this lane's query;
// the key of s[beta][r] is kt0 + 4h + 32 beta + 8 (r / 4) + r % 4.
__device__ __forceinline__ void mask_tile(floatx16 (&s)[2], int kt0, int k1, int qi, int h,
                                          int causal, int window) {
  const int kb = kt0 + 4 * h;
  const int hi = (causal ? min(k1 - 1, qi) : k1 - 1) - kb;
  const int lo = window > 0 ? qi - window + 1 - kb : -(1 << 30);
#pragma unroll
  for (int beta = 0; beta < 2; ++beta)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rel = 32 * beta + 8 * (r / 4) + (r % 4);
      if (rel > hi || rel < lo) s[beta][r] = -INFINITY;
    }
}

// S^T of the staged K tile again (rare path).
template <int D>
__device__ __forceinline__ void scores_again(const __bf16 *ks, const bf16x8 (&qf)[D / 16], int l32,
                                          int h, floatx16 (&s)[2]) {
  constexpr int KS = D + 8;
  s[0] = floatx16{};
  s[1] = floatx16{};
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    s[0] = mfma32x32x16(*reinterpret_cast<const bf16x8 *>(&ks[l32 * KS + 16 * c + 8 * h]), qf[c],
                        s[0]);
    s[1] = mfma32x32x16(*reinterpret_cast<const bf16x8 *>(&ks[(32 + l32) * KS + 16 * c + 8 * h]),
                        qf[c], s[1]);
  }
}

// NW waves (32 query slots each) per work item.
template <int D, int DV, int NW>
__global__ __launch_bounds__(64 * NW, 2) void fwd_bf16_kernel(
    const WorkItem *__restrict__ items, const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K,
    const __bf16 *__restrict__ V, __bf16 *__restrict__ O, float *__restrict__ LSE, int Hs,
    int Hks, int G, int64_t Ns, float scale, float scale_log2, int causal, int window,
    int *__restrict__ split_cnt, float *__restrict__ split_part) {
  constexpr bool VT = NW == 8;  // V layout (see SmemBF)
  constexpr int KS = SmemBF<D, DV, VT>::KS, VS = SmemBF<D, DV, VT>::VS;
  __shared__ __attribute__((aligned(16))) SmemBF<D, DV, VT> sm;
  const WorkItem it = items[blockIdx.x];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t rs = (int64_t)Hs * D;     // Q elements between consecutive slots
  const int64_t rso = (int64_t)Hs * DV;   // O
  const int64_t rsk = (int64_t)Hks * D;   // K
  const int64_t rsv = (int64_t)Hks * DV;  // V
  const uint32_t rsbq = (uint32_t)rs * 2u, rsb = (uint32_t)rsk * 2u, rsbv = (uint32_t)rsv * 2u;
  const __bf16 *Kh = K + (int64_t)(it.head / G) * D;  // the query head's K/V head
  const __bf16 *Vh = V + (int64_t)(it.head / G) * DV;

  const int wq0 = it.q0 + 32 * w;       // first query of this wave
  const int wq1 = min(wq0 + 32, it.q1);  // one past its last valid query
  const int qi = wq0 + l32;              // this lane's query
  const bool qok = qi < it.q1;
  // this lane's part of a V read: VT, row l32 of V^T at key column 8h;
  // else a transposed read, where inside its group of 16 lanes, lane 4e + g
  // addresses key row e (+ 4h) and features 4g .. 4g + 3 (+ 16 for the upper
  // 16 lanes of each half-wave)
  const int vlane = VT ? l32 * VS + 8 * h
                       : (4 * h + ((l32 & 15) >> 2)) * VS + 16 * (l32 >> 4) + 4 * (l32 & 3);

  // the wave's queries as the B operand (k = features 16c + 8h .. +8)
  bf16x8 qf[D / 16];
  {
    const auto rq = make_rsrc(Q + (int64_t)wq0 * rs + (int64_t)it.head * D,
                              (uint32_t)max(0, wq1 - wq0) * rsbq);
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      qf[c] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)l32 * rsbq + 32u * c + 16u * h));
  }

  floatx16 o[DV / 32];
#pragma unroll
  for (int dl = 0; dl < DV / 32; ++dl) o[dl] = floatx16{};
  float m = kMinusBig;  // running max of raw scores (the exponent's reference)
  float mb = m * scale_log2;
  float l = 0.0f;       // this lane's part of the running sum
  bool first = true;    // no active tile seen yet (wave-uniform)

  const int nk = (it.k1 - it.k0 + BK - 1) / BK;
  constexpr int NT = 64 * NW;
  StageBF<D, DV, NT, VT> st;
  st.load(Kh + (int64_t)it.k0 * rsk, Vh + (int64_t)it.k0 * rsv, it.k1 - it.k0, rsb, rsbv, tid);
  st.store(sm.k[0], sm.v[0], tid);
  if (nk > 1)
    st.load(Kh + (int64_t)(it.k0 + BK) * rsk, Vh + (int64_t)(it.k0 + BK) * rsv,
            it.k1 - it.k0 - BK, rsb, rsbv, tid);
  __syncthreads();

  for (int t = 0; t < nk; ++t) {
    const int buf = t & 1;
    const int kt0 = it.k0 + t * BK;
    // wave-uniform tile classification
    const bool active = wq0 < wq1 && !(causal && kt0 > wq1 - 1) &&
                        !(window > 0 && wq0 - (kt0 + BK - 1) >= window);
    if (active) {
      const __bf16 *ks = sm.k[buf];
      const __bf16 *vs = sm.v[buf];
      const bool full = (kt0 + BK <= it.k1) && (!causal || kt0 + BK - 1 <= wq0) &&
                        (window <= 0 || (wq1 - 1) - kt0 < window);
      bf16x8 a[2][D / 16];
#pragma unroll
      for (int beta = 0; beta < 2; ++beta)
#pragma unroll
        for (int c = 0; c < D / 16; ++c)
          a[beta][c] =
              *reinterpret_cast<const bf16x8 *>(&ks[(32 * beta + l32) * KS + 16 * c + 8 * h]);
      // key half 0 first: its weights can start while half 1 is multiplied
      floatx16 s[2] = {floatx16{}, floatx16{}};
#pragma unroll
      for (int beta = 0; beta < 2; ++beta)
#pragma unroll
        for (int c = 0; c < D / 16; ++c) s[beta] = mfma32x32x16(a[beta][c], qf[c], s[beta]);
      if (!full) mask_tile(s, kt0, it.k1, qi, h, causal, window);
      // weights against the current reference max; the row max is only taken
      // on the wave's first tile and when some weight would exceed 2^64 (a
      // score more than 64 above the reference in the exp2 domain)
      float ls = 0.0f;
      bool need_max = first;
      if (!need_max) {
#pragma unroll
        for (int beta = 0; beta < 2; ++beta)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pv = fast_exp2(fmaf(s[beta][r], scale_log2, -mb));
            s[beta][r] = pv;
            ls += pv;
          }
        need_max = wave_any(!(ls <= kOverflow));
        if (need_max) {  // rare: the raw scores were overwritten, form them again
          scores_again<D>(ks, qf, l32, h, s);
          if (!full) mask_tile(s, kt0, it.k1, qi, h, causal, window);
        }
      }
      if (need_max) {
        float mx = s[0][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
        mx = halves_max(mx);
        const float m_new = fmaxf(m, mx);
        const float alpha = fast_exp2((m - m_new) * scale_log2);
        m = m_new;
        mb = m_new * scale_log2;
        l *= alpha;
#pragma unroll
        for (int dl = 0; dl < DV / 32; ++dl)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dl][r] *= alpha;
        ls = 0.0f;
#pragma unroll
        for (int beta = 0; beta < 2; ++beta)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pv = fast_exp2(fmaf(s[beta][r], scale_log2, -mb));
            s[beta][r] = pv;
            ls += pv;
          }
      }
      l += ls;
      first = false;
      bf16x8 pf[2][2];
#pragma unroll
      for (int beta = 0; beta < 2; ++beta)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
#pragma unroll
          for (int e = 0; e < 8; ++e) pf[beta][mm][e] = (__bf16)s[beta][8 * mm + e];
      // A operand of O^T += V^T P^T: row d = 32 dl + l32 of V^T with the keys
      // of pf[beta][mm] (32 beta + 16 mm + 4h + 0..3, then the same + 8): one
      // 16-byte read of the permuted V^T tile, or two transposed reads of the
      // row-major V tile
#pragma unroll
      for (int beta = 0; beta < 2; ++beta)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
#pragma unroll
          for (int dl = 0; dl < DV / 32; ++dl) {
            bf16x8 va;
            if (VT) {
              va = *reinterpret_cast<const bf16x8 *>(&vs[vlane + 32 * dl * VS + 32 * beta +
                                                         16 * mm]);
            } else {
              const __bf16 *vp = vs + vlane + (32 * beta + 16 * mm) * VS + 32 * dl;
              const uint2 lo = lds_read_tr16(vp), hi = lds_read_tr16(vp + 8 * VS);
              va = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
            }
            o[dl] = mfma32x32x16(va, pf[beta][mm], o[dl]);
          }
    }
    if (t + 1 < nk) {
      st.store(sm.k[buf ^ 1], sm.v[buf ^ 1], tid);
      if (t + 2 < nk)
        st.load(Kh + (int64_t)(kt0 + 2 * BK) * rsk, Vh + (int64_t)(kt0 + 2 * BK) * rsv,
                it.k1 - kt0 - 2 * BK, rsb, rsbv, tid);
    }
    __syncthreads();
  }

  if (it.pad0 >= 0) {
    // The item's key range was cut into parts run by separate blocks (this
    // one ran [k0, k1)).  Each part leaves its unnormalised O^T, reference max
    // and sum in its partial slot, then counts itself in; the last to arrive
    // merges all parts: with M = max_p m_p and c_p = 2^((m_p - M) s log2 e),
    // O^T = sum c_p O^T_p and l = sum c_p l_p -- the rescaling of the online
    // softmax, once per part.  Nobody waits: blocks that are not last just
    // finish.  The merge folds the parts in part order whichever block does
    // it (its own part from registers, the same values it stored), so the
    // result does not depend on the order in which the parts finished.  The
    // slots are written and read with device-coherent accesses, so no
    // cache-wide write-back or invalidation is needed around the count.
    const int part = it.pad2 >> 16, parts = it.pad2 & 0xffff;
    constexpr int CH = fwd_partial_chunks(DV);
    constexpr uint32_t kWaveBytes = CH * 64 * 16;  // one wave's share of a slot
    // this wave's region of part pp's slot
    const auto region = [&](int pp) {
      const char *base = reinterpret_cast<const char *>(split_part) +
                         ((int64_t)(it.pad1 - part + pp) * NW + w) * kWaveBytes;
      return make_rsrc(base, kWaveBytes);
    };
    const uint32_t lo = 16u * lane;
    {
      const auto mine = region(part);
#pragma unroll
      for (int dl = 0; dl < DV / 32; ++dl)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          store16_coherent(mine, lo + 1024u * (4 * dl + b),
                           floatx4{o[dl][4 * b], o[dl][4 * b + 1], o[dl][4 * b + 2],
                                   o[dl][4 * b + 3]});
      store16_coherent(mine, lo + 1024u * (CH - 1), floatx4{m, l, 0.0f, 0.0f});
    }
    // The slot is complete and visible device-wide once the stores have
    // drained; only then does the block count itself in.
    wait_stores();
    __shared__ int last;
    __syncthreads();
    if (tid == 0)
      last = __hip_atomic_fetch_add(split_cnt + it.pad0, 1, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT) == parts - 1;
    __syncthreads();
    if (!last) return;
    if (tid == 0)  // every part has counted: ready for the next launch
      __hip_atomic_store(split_cnt + it.pad0, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    floatx16 acc[DV / 32];
#pragma unroll
    for (int dl = 0; dl < DV / 32; ++dl) acc[dl] = floatx16{};
    float am = kMinusBig, al = 0.0f;
    for (int pp = 0; pp < parts; ++pp) {
      const bool own = pp == part;  // block-uniform
      const auto src = region(pp);
      float pm = m, pl = l;
      if (!own) {
        const floatx4 ml = load16_coherent(src, lo + 1024u * (CH - 1));
        pm = ml[0];
        pl = ml[1];
      }
      float ca = 0.0f, cb = 1.0f;  // part 0: acc = its values
      if (pp > 0) {
        const float mx = fmaxf(am, pm);
        ca = fast_exp2((am - mx) * scale_log2);
        cb = fast_exp2((pm - mx) * scale_log2);
      }
      am = pp > 0 ? fmaxf(am, pm) : pm;
      al = al * ca + pl * cb;
#pragma unroll
      for (int dl = 0; dl < DV / 32; ++dl)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          floatx4 x;
          if (own)
            x = floatx4{o[dl][4 * b], o[dl][4 * b + 1], o[dl][4 * b + 2], o[dl][4 * b + 3]};
          else
            x = load16_coherent(src, lo + 1024u * (4 * dl + b));
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[dl][4 * b + i] = acc[dl][4 * b + i] * ca + x[i] * cb;
        }
    }
    m = am;
    l = al;
#pragma unroll
    for (int dl = 0; dl < DV / 32; ++dl) o[dl] = acc[dl];
  }

  // epilogue: O = O^T / l, LSE = s * m + ln l
  const float lt = halves_sum(l);
  if (qok) {
    const float inv = 1.0f / lt;
    __bf16 *orow = O + (int64_t)qi * rso + (int64_t)it.head * DV;
#pragma unroll
    for (int dl = 0; dl < DV / 32; ++dl)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = o[dl][4 * b + i] * inv;
        store4<__bf16>(orow + 32 * dl + 8 * b + 4 * h, x);
      }
    if (h == 0) LSE[(int64_t)it.head * Ns + qi] = m * scale + logf(lt);
  }
}

template <typename T, int D, int DV = D>
hipError_t launch_typed(const attn_plan *p, const void *q, const void *k, const void *v, void *o,
                        float *lse, hipStream_t stream) {
  static_assert(std::is_same<T, __bf16>::value || DV == D, "fp32 keeps one head width");
  const WorkItem *items = reinterpret_cast<const WorkItem *>(p->ws + p->off_fwd);
  int *split_cnt = reinterpret_cast<int *>(p->ws + p->off_split_cnt);
  float *split_part = reinterpret_cast<float *>(p->ws + p->off_split_part);
  const unsigned n = (unsigned)p->fwd.size();
  if (n == 0) return hipSuccess;
  const float scale = p->p.scale;
  const float scale_log2 = scale * 1.4426950408889634f;
  const Problem &P = p->p;
  if (std::is_same<T, __bf16>::value && p->fwd_bq == kFwdBQ)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, DV, kFwdBQ / 32>), dim3(n), dim3(2 * kFwdBQ), 0, stream,
                       items, static_cast<const __bf16 *>(q), static_cast<const __bf16 *>(k),
                       static_cast<const __bf16 *>(v), static_cast<__bf16 *>(o), lse, P.Hs, P.Hks,
                       P.G, P.Ns, scale, scale_log2, P.causal, P.window, split_cnt, split_part);
  else if (std::is_same<T, __bf16>::value)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, DV, kFwdBQShort / 32>), dim3(n),
                       dim3(2 * kFwdBQShort), 0, stream, items, static_cast<const __bf16 *>(q),
                       static_cast<const __bf16 *>(k), static_cast<const __bf16 *>(v),
                       static_cast<__bf16 *>(o), lse, P.Hs, P.Hks, P.G, P.Ns, scale, scale_log2,
                       P.causal, P.window, split_cnt, split_part);
  else
    hipLaunchKernelGGL((fwd_kernel<float, D>), dim3(n), dim3(kFwdThreadsF32), 0, stream, items,
                       static_cast<const float *>(q), static_cast<const float *>(k),
                       static_cast<const float *>(v), static_cast<float *>(o), lse, P.Hs, P.Hks,
                       P.G, P.Ns, scale, scale_log2, P.causal, P.window);
  return hipGetLastError();
}

}  // namespace

attn_status launch_fwd(const attn_plan *p, const void *q, const void *k, const void *v, void *o,
                       float *lse, hipStream_t stream) {
  hipError_t e;
  const bool bf = p->p.dtype == ATTN_BF16;
  const int d = p->p.d, dv = p->p.dv;  // the plan admits dv != d for bf16 only
  if (bf && d == 64 && dv == 128)
    e = launch_typed<__bf16, 64, 128>(p, q, k, v, o, lse, stream);
  else if (bf && d == 128 && dv == 64)
    e = launch_typed<__bf16, 128, 64>(p, q, k, v, o, lse, stream);
  else if (d == 64)
    e = bf ? launch_typed<__bf16, 64>(p, q, k, v, o, lse, stream)
           : launch_typed<float, 64>(p, q, k, v, o, lse, stream);
  else
    e = bf ? launch_typed<__bf16, 128>(p, q, k, v, o, lse, stream)
           : launch_typed<float, 128>(p, q, k, v, o, lse, stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

}  // namespace attn
