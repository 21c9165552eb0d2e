// device_common.h -- small gfx950 helpers shared by the kernels: bf16 packing,
// MFMA operand vector types, cross-half-wave exchange.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t uint32x4 __attribute__((ext_vector_type(4)));

// bf16 halves of a 32-bit word -> float (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

// Reductions of lane l with lane l ^ 32.  v_permlane32_swap applied to two
// copies of x returns one copy holding the low half-wave's values in both
// halves and one holding the high half-wave's; a symmetric operation on the
// two gives every lane op(x[l % 32], x[l % 32 + 32]), whichever copy is which.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Position of row r (0..63) of a tile inside a transposed LDS copy whose rows
// are read as the k operand of a 32x32x16 MFMA.  A 32x32 accumulator gives
// lane half h the rows 8b + 4h + i (b = 0..3, i = 0..3); the k operand wants
// 8 consecutive k per lane half.  Swapping bits 2 and 3 of the row index
// inside each group of 16 makes the accumulator's rows 16m + 8b' + 4h + i
// land at 16m + 8h + 4b' + i, i.e. eight contiguous positions per lane half.
__device__ __forceinline__ int perm16(int r) {
  return (r & ~0xC) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Raw buffer resource over [base, base + bytes): loads at byte offsets past
// `bytes` return zeros, so ragged tile tails need no branch.  (Word 3 is the
// gfx9-family raw-buffer format word.)
// Both arguments must be wave-uniform; readfirstlane states it, so the
// descriptor lives in SGPRs (no waterfall loop around the load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                           __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// 16-byte stores and loads with the device-scope coherence bit (sc1 in the
// cache-policy operand: bit 0 sc0, bit 1 nt, bit 4 sc1), the access form of
// device-scope relaxed atomics: a store is visible to every CU of every XCD
// once this wave's memory counter has drained (wait_stores), and a load reads
// around the non-coherent cache levels.  They let blocks hand data to each
// other through global memory without cache-wide write-backs or
// invalidations.
constexpr int kDeviceCoherent = 16;
__device__ __forceinline__ void store16_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                 floatx4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(uint32x4, v), r, off, 0,
                                         kDeviceCoherent);
}
__device__ __forceinline__ floatx4 load16_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0,
                                                                           kDeviceCoherent));
}

// Direct global -> LDS staging (buffer_load_dwordx4 with the LDS flag) of
// the 64 rows [t0, t0 + 64) of a [slots, heads, W] bf16 tensor into a
// row-major LDS tile of row stride W + 8 elements.  A wave instruction writes
// 1 KB of LDS, lane L at byte 16 L, so instruction i fills the padded tile's
// 16-byte chunks [64 i, 64 i + 64); a lane whose chunk is a row's pad, or
// whose row is past the buffer resource's end, reads out of range, which
// writes zeros.
template <int W>
struct DmaTile {
  static constexpr int RC = W / 8 + 1;  // 16-byte chunks per LDS row, the last one pad
  static constexpr int NI = RC;         // wave instructions per 64-row tile
  __device__ static __forceinline__ uint32_t offset(int i, int lane, uint32_t rsb) {
    const int p = 64 * i + lane, row = p / RC, c = p % RC;
    return c < W / 8 ? (uint32_t)row * rsb + 16u * (uint32_t)c : 0x80000000u;
  }
};
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, __bf16 *lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16,
                                           off, 0, 0, 0);
}
// wait for this wave's staging loads (vmcnt 0; other counters left alone)
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// wait until this wave's stores are complete (vmcnt counts them too)
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// 2^x on the transcendental unit (v_exp_f32); results below the normal range
// flush to zero, which is what softmax weights want.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

// ds_read_b64_tr_b16: inside each group of 16 lanes, lane i receives element
// (i % 4) of the 8-byte chunks addressed by lanes i/4, 4 + i/4, 8 + i/4 and
// 12 + i/4 (in that order).  If lane 4e + g of the group addresses row
// (r0 + e), columns (c0 + 4g .. c0 + 4g + 3) of a row-major bf16 tile, lane i
// receives rows r0 .. r0 + 3 of column c0 + i: a transposed read.
__device__ __forceinline__ uint2 lds_read_tr16(const __bf16 *p) {
  const shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(p));
  return __builtin_bit_cast(uint2, v);
}

__device__ __forceinline__ floatx16 mfma32x32x16(const bf16x8 &a, const bf16x8 &b,
                                                 const floatx16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx16 mfma32x32x2f32(float a, float b, const floatx16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

}  // namespace attn
