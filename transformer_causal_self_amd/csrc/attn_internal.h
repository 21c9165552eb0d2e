// attn_internal.h -- plan layout and tile sizes shared by the host plan and
// the gfx950 kernels.  Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

#include "../../include/attn_mi355.h"

namespace attn {

// Tile shapes.  The host plan cuts work items with these, the kernels assume
// them; both sides include this header.
//   forward: BQ query slots per work item, BK key slots per inner step, 32
//   queries per wave.  bf16 runs eight waves per item (each staged K/V tile
//   serves 256 queries) unless the window is short, where a 256-query item
//   would stage mostly keys that most of its waves skip, every sequence is
//   short, where twice as many items balance the CUs better, or both head
//   widths are 64: then four.  At widths of 64 four four-wave blocks share a
//   CU (two eight-wave ones otherwise), their waves independent of each
//   other on each SIMD, which beats staging each K/V tile once for 256
//   queries (+2% on the long causal problem, +3% with grouped K/V heads);
//   wider heads fit one eight-wave or two four-wave blocks per CU, and there
//   the four-wave items lose 3% (varlen window-2048 problem).  fp32 runs
//   four, its registers do not allow more.
constexpr int kFwdBQ = 256;
constexpr int kFwdBQShort = 128;
constexpr int kFwdShortWindow = 512;  // windows up to this use kFwdBQShort
constexpr int kFwdShortSeq = 2048;    // and so do problems whose sequences all fit this
constexpr int kFwdBQF32 = 128;
constexpr int kFwdThreadsF32 = 256;
constexpr int kFwdBK = 64;
//   backward: both passes run four waves of 32 rows (keys for dK/dV, queries
//   for dQ) per item and step over 64 partner rows at a time.  Several
//   independent blocks then share a CU (three at d = 64, two at d = 128) and
//   their phases interleave, which beat eight-wave items that stage each
//   partner tile once for 256 rows (-4% on the long causal problem, -18% at
//   GPT-2-small sizes, -10% on the paired window-128 problem).
constexpr int bwd_waves(int, int) { return 4; }
constexpr int kBwdBQ = 64;
//   rotary: threads per block, and the fine step of the two-level cos/sin
//   table (positions p = hi * kRopeFine + lo).
constexpr int kRopeThreads = 256;
constexpr int kRopeFine = 64;
// Work-list chunk: consecutive tiles of one head and sequence kept on one XCD.
constexpr int kXcdChunk = 16;
// Size of the device array that holds the backward's D values in
// attn_bwd_noalloc (one float per attention head and slot: 8 Mi rows).
constexpr size_t kNoallocScratchBytes = size_t(32) << 20;

// Compute units of the chip (8 XCDs of 32).
constexpr int kCUs = 256;

// Forward blocks resident on one CU, from the kernels' register use (at most
// 512 VGPRs per SIMD lane: 128 a wave at four waves per SIMD, 256 at two) and
// LDS: the d = dv = 64 kernel fits 128 registers, the wider ones do not.
// Only the plan's schedule model uses it.
constexpr int fwd_blocks_per_cu(int dtype, int d, int dv, int bq) {
  return dtype != 0 ? 1 : (bq == kFwdBQ ? (d == 64 && dv == 64 ? 2 : 1)
                                        : (d == 64 && dv == 64 ? 4 : 2));
}

// A forward item whose key range is cut into parts leaves, per part, the
// unnormalised output rows and the running max and sum of its queries in a
// partial-result slot; the last part to finish merges them.  Per wave and lane:
// dv / 8 float4 of the output accumulator, then one float4 (max, sum, 0, 0),
// stored chunk-major (chunk c of lane L at float4 64 c + L).
constexpr int fwd_partial_chunks(int dv) { return dv / 8 + 1; }
constexpr size_t fwd_partial_bytes(int dv, int bq) {
  return (size_t)(bq / 32) * 64 * 16 * (size_t)fwd_partial_chunks(dv);
}

// One work item of the forward or dQ pass: attention head `head`, query slots
// [q0, q1) inside one sequence, key slots [k0, k1) that any of those queries
// may see.  For the dK/dV pass the roles swap: keys [q0, q1) of the item,
// queries [k0, k1) that may see them.  Backward lists: pad0 = stream, the
// (attention head, sequence) index.  Forward list: pad0 = split group (-1:
// the item is whole), pad1 = its partial-result slot, pad2 = part << 16 |
// parts; the parts of a group hold consecutive slots.
struct WorkItem {
  int32_t head;
  int32_t q0, q1;
  int32_t k0, k1;
  int32_t pad0, pad1, pad2;
};
static_assert(sizeof(WorkItem) == 32, "work item is 32 bytes");

struct Problem {
  int64_t N;       // tokens
  int32_t H, d;    // heads given, head dim
  int32_t dtype;   // ATTN_BF16 / ATTN_FP32
  int32_t causal, window;
  float scale;
  int32_t rope;
  double rope_base;
  int32_t paired;
  int32_t Hs;      // attention (query) heads
  int64_t Ns;      // slots
  int32_t Hkv;     // K/V heads given (= H unless grouped)
  int32_t Hks;     // K/V attention heads (= Hs unless grouped)
  int32_t G;       // query heads per K/V head: Hs / Hks
  int32_t qk_norm; // RMS-norm of Q and K rows before the rotation
  float norm_eps;
  int32_t dv;      // V / O / dO / dV head dim (= d unless set apart)
};

}  // namespace attn

struct attn_plan {
  attn::Problem p;
  std::vector<int32_t> cu;          // token boundaries, S + 1
  std::vector<int32_t> tok_pos;     // per token: offset inside its sequence
  std::vector<float> rope_cos;      // [F + ceil(P / F), d/2]: fine rows, then coarse
  std::vector<float> rope_sin;      // same layout (F = kRopeFine)
  int32_t max_pos = 0;              // P, positions covered
  int32_t fwd_bq = 0;               // query slots per forward item
  std::vector<attn::WorkItem> fwd;  // forward items
  std::vector<attn::WorkItem> bwd;  // dK/dV items
  std::vector<attn::WorkItem> dq;   // dQ items (bf16 problems only)
  int32_t fwd_groups = 0;           // forward items cut into parts
  int32_t fwd_part_slots = 0;       // partial-result slots of their parts
  std::vector<int32_t> zero_counters;  // initial merge counters (zeros)
  attn_plan_info info{};

  // Workspace layout (byte offsets; every section 256-byte aligned).
  size_t off_pos = 0, off_cos = 0, off_sin = 0, off_fwd = 0, off_bwd = 0, off_dq = 0;
  size_t off_delta = 0;
  size_t off_split_cnt = 0, off_split_part = 0;
  size_t ws_bytes = 0;
  // Bound workspace.
  char *ws = nullptr;
};
