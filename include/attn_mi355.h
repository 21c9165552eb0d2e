/*
 * attn_mi355.h -- C ABI of the MI355X (gfx950) rotary causal self-attention
 * library (libattn_mi355.so).
 *
 * The library computes, on one GPU,
 *     O = softmax(s * Q' K'^T + mask) V,    LSE = log of the row sums,
 * with Q', K' the rotary-embedded queries and keys, over packed variable-length
 * sequences, optionally with a causal sliding window, and optionally with
 * "paired heads".  The pages this follows:
 *
 *  - "Paired Head Attention" record article (hncyxsy.com):
 *      section "Source 3: paired forward branch" -- the varlen attention call
 *        with cu_seqlens, causal=True, softmax_scale and a left window, on one
 *        packed stream;
 *      sections "Core idea" and "Source 4: Triton kernel interleave indexing"
 *        -- head h of token t becomes slot 2t + h / (H/2) of attention head
 *        h mod (H/2): the sequence doubles and the head count halves;
 *      section "Core idea" -- the K/Q/V of two adjacent heads are interleaved
 *        per position (the ATTN_PAIRED_ADJACENT reading: partner h ^ 1);
 *      section "Sequence length and window" -- sequence boundaries double,
 *        the window (in key slots) does not;
 *      sections "Zero-copy RoPE", "Staggered rotary", "Source 2: paired
 *        rotary table" -- adjacent-pair rotation and the paired position
 *        2t + (h mod 2).
 *  - "Upgrading a textbook decoder" (juejin.cn): section 2 "RoPE" -- the
 *    frequencies base^(-2i/d) and the half-split rotation; section 4 --
 *    FlashAttention computes the same result as the plain definition, and
 *    grouped-query attention: groups of query heads share one K/V head
 *    (query head h reads K/V head h / (H / Hkv), the page's repetition of
 *    each K/V head along the head axis, done here by indexing, not copying).
 *  - "SingleHeadAttention" note (ranhao.site) -- the lower-triangular causal
 *    mask; "mHC module" article (lshu.cn), sections 2.1-2.2 -- softmax with
 *    max subtraction.
 *
 * Layouts (row-major, element strides):
 *   Q, K, V, O         [N, H, d]  token-major, each token's H*d values contiguous.
 *                      When paired (ATTN_PAIRED) the same memory is read as
 *                      [2N, H/2, d]: slot 2t + h / (H/2), attention head
 *                      h mod (H/2).  With ATTN_PAIRED_ADJACENT, head h goes to
 *                      slot 2t + (h mod 2), attention head h / 2; the [2N, H/2, d]
 *                      buffers (Q', K', V' from rope_qkv, O, dQ, dK, dV) then
 *                      hold token t's heads in the order 0, 2, 4, ..., 1, 3, 5,
 *                      ...: head h at position (h mod 2) * H/2 + h / 2 of the
 *                      token's H*d row.
 *   K, V (grouped)     [N, Hkv, d] when num_kv_heads = Hkv < H (unpaired only).
 *   V, O, dO, dV       rows of dv = v_head_dim elements instead of d when the
 *                      problem sets a separate value width ("Paired Head
 *                      Attention" article, section "Source 1: model
 *                      configuration": each attention module has its own
 *                      qk_dim and v_dim); Q, K, dQ, dK keep d.
 *   LSE                float [H', N'] (attention head, slot); natural log.
 *   dQ, dK, dV         float [N, H, d] (same slot view as Q when paired);
 *                      dK, dV are [N, Hkv, d] when grouped.
 *   N' = 2N, H' = H/2 when paired; else N' = N, H' = H.
 *
 * Conventions for every call:
 *   - Every device pointer must be 16-byte aligned and every token stride a
 *     multiple of 8 elements (bf16) or 4 elements (fp32); else ATTN_E_ALIGN.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Launch functions only enqueue work; they return ATTN_E_HIP when a launch
 *     or copy is rejected.  Faults during execution surface at the caller's
 *     next synchronisation.
 *   - The caller owns every device buffer, the workspace and the stream.  The
 *     plan owns only host memory and is immutable after attn_plan_bind, so
 *     several launches may share it.  Launches that share one bound workspace
 *     may run concurrently, except two attn_fwd or two attn_bwd calls: each
 *     of those entry points keeps scratch data in the workspace (attn_fwd the
 *     merge counters and partial results of query tiles whose key range the
 *     plan cut into parts, attn_bwd the per-row D values).  The merge
 *     counters start at zero at attn_plan_bind and every attn_fwd leaves them
 *     at zero; a launch that does not run to completion leaves them
 *     undefined, and binding again resets them.
 *   - No call throws, aborts or prints.
 */
#ifndef ATTN_MI355_H
#define ATTN_MI355_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct attn_plan attn_plan; /* opaque host object */

typedef enum {
  ATTN_OK = 0,
  ATTN_E_INVALID = -1,     /* a bad argument or an inconsistent problem */
  ATTN_E_UNSUPPORTED = -2, /* a valid problem the kernels do not cover */
  ATTN_E_ALIGN = -3,       /* a pointer or stride breaks the alignment rule */
  ATTN_E_WORKSPACE = -4,   /* plan not bound, or workspace missing/too small */
  ATTN_E_HIP = -5,         /* the HIP runtime rejected a launch or copy */
  ATTN_E_NOMEM = -6        /* host allocation failed */
} attn_status;

enum { ATTN_BF16 = 0, ATTN_FP32 = 1 };
enum { ATTN_ROPE_NONE = 0, ATTN_ROPE_HALF = 1, ATTN_ROPE_ADJACENT = 2 };
enum { ATTN_UNPAIRED = 0, ATTN_PAIRED = 1, ATTN_PAIRED_ADJACENT = 2 };

typedef struct {
  int64_t num_tokens;        /* N >= 0 */
  int32_t num_heads;         /* H >= 1; even when paired */
  int32_t head_dim;          /* d: 64 or 128 */
  int32_t dtype;             /* ATTN_BF16 or ATTN_FP32 (I/O type; fp32 accumulate) */
  const int32_t *cu_seqlens; /* HOST pointer, num_seqs + 1 entries: 0 = cu[0] <= ... <= cu[S] = N */
  int32_t num_seqs;          /* S >= 1 */
  int32_t causal;            /* 0 or 1; must be 1 when window > 0 */
  int32_t window;            /* <= 0: none; else key slot j is visible from query
                                slot i only if 0 <= i - j < window (self counts) */
  float softmax_scale;       /* s; 0 selects 1/sqrt(head_dim) */
  int32_t rope;              /* ATTN_ROPE_NONE, _HALF (pairs i, i+d/2), _ADJACENT (2i, 2i+1) */
  double rope_base;          /* frequencies base^(-2i/d); e.g. 10000 */
  int32_t paired;            /* ATTN_UNPAIRED, ATTN_PAIRED (partner h + H/2, the
                                memory view) or ATTN_PAIRED_ADJACENT (partner h ^ 1) */
  int32_t num_kv_heads;      /* Hkv: 0 or H for one K/V head per query head; else a
                                divisor of H (grouped-query attention, unpaired
                                only: ATTN_E_UNSUPPORTED with pairing) */
  int32_t qk_norm;           /* 0: none; 1: rope_qkv first RMS-normalises every Q and
                                K head row over d, x / sqrt(mean(x^2) + eps), in
                                fp32 and without a gain */
  float norm_eps;            /* eps of that norm; 0 selects 1e-6 */
  int32_t v_head_dim;        /* dv, the width of V, O, dO and dV rows: 0 selects
                                head_dim; else 64 or 128, and a value other than
                                head_dim needs ATTN_BF16 (q, k keep head_dim) */
} attn_problem;

/* Counts for throughput and roofline reporting (exact, from the plan). */
typedef struct {
  int64_t visible_pairs;     /* (query slot, key slot) pairs inside the mask, all heads */
  double fwd_flops;          /* 2 (d + dv) visible_pairs (QK^T and PV) */
  double bwd_flops;          /* 2 (3 d + 2 dv) visible_pairs (five products: S, dP,
                                dV, dQ, dK); 2.5 fwd_flops when dv = d */
  double rope_bytes;         /* read Q, K and write Q', K' once */
  double fwd_bytes;          /* read Q, K, V and write O, LSE once */
  double bwd_bytes;          /* read Q, K, V, O, dO, LSE and write dQ, dK, dV once */
  int64_t fwd_items;         /* work items (attention head x sequence x query tile) */
  int64_t bwd_items;         /* key-tile work items of the backward */
  int64_t slots;             /* N' */
  int32_t attn_heads;        /* H' */
  int32_t max_positions;     /* positions the rotary table covers (longest
                                sequence, doubled when paired) */
  int32_t kv_heads;          /* K/V heads: Hkv, or H' when not grouped */
  int32_t v_head_dim;        /* dv */
  int32_t fwd_split_items;   /* forward query tiles whose key range is cut into
                                parts run by separate workgroups (merged in the
                                same launch) */
} attn_plan_info;

/*
 * The problem statement follows the varlen attention call of "Paired Head
 * Attention", section "Source 3" (packed tokens, cu_seqlens, causal, a left
 * window, softmax scale), with the rotary and pairing arguments of its
 * sections "Zero-copy RoPE" and "Source 4", and the textbook module's
 * num_kv_heads ("Upgrading a textbook decoder", section 4).
 * Validate a problem and build its host plan: paired slot boundaries
 * (2 * cu when paired), the per-token rotary positions, the fp64-computed
 * cos/sin table rounded to fp32 (two levels: angles lo * theta and
 * 64 hi * theta, combined by angle addition in the kernels for position
 * 64 hi + lo, so the table stays cache resident), and the tile work lists
 * (fully masked causal and window tiles are never listed; longest items
 * first; a forward query tile whose key range is long next to the mean load
 * of a workgroup slot may be cut into parts that separate workgroups run and
 * the last of them merges).  A window of at least the longest sequence's
 * slot count hides nothing and is treated as no window.  Host only: makes
 * no HIP call.  On success *out owns a plan to free with attn_plan_destroy.
 * Errors: ATTN_E_INVALID (bad field), ATTN_E_UNSUPPORTED (head_dim or
 * v_head_dim not 64 or 128; v_head_dim != head_dim with fp32; grouped K/V
 * heads with pairing; num_heads * max(head_dim, v_head_dim) above 2^20,
 * which keeps the byte offsets inside a 256-slot tile in 31 bits),
 * ATTN_E_NOMEM.
 */
attn_status attn_plan_create(const attn_problem *problem, attn_plan **out);

/* Device workspace the plan needs, in bytes (0 for a NULL plan). */
size_t attn_plan_workspace_bytes(const attn_plan *plan);

/*
 * Copy the plan's tables and work lists into d_workspace (device memory of at
 * least attn_plan_workspace_bytes, 256-byte aligned) on `stream`.  The caller
 * keeps the workspace alive and unchanged while launches use it.  Rebinding
 * the same plan to another workspace is allowed.
 */
attn_status attn_plan_bind(attn_plan *plan, void *d_workspace, size_t bytes, void *stream);

/* Fill *info with the plan's exact counts.  Host only. */
attn_status attn_plan_stats(const attn_plan *plan, attn_plan_info *info);

/*
 * Introspection of the tile work lists (host only), for testing and
 * scheduling analysis.  which = 0: forward items (256 query slots each for
 * bf16; 128 for fp32, for windows of at most 512 slots, when no sequence is
 * longer than 2048 slots and at head widths d = dv = 64); which = 1:
 * backward key-tile items (128 key slots); which = 2: backward dQ items (128
 * query slots).  The backward lists are empty for fp32 problems.  The head
 * of every item is a query (attention) head; with grouped K/V heads the key
 * tiles of a group's query heads add into the same dK/dV rows.
 * Each item is 8 int32: {attention head, r0, r1, s0, s1, x, y, z}.
 * Backward lists: x = stream, the index of the (attention head, sequence)
 * pair, y = z = 0.  Forward list: x = merge group (-1 when the query tile is
 * whole, else the index of the cut query tile), y = the part's
 * partial-result slot (consecutive for the parts of one group), z = part
 * index << 16 | number of parts (1 when whole).  The list order is the
 * launch order: item i runs as workgroup i, on XCD i mod 8; items of one
 * stream and nearby tiles share an XCD (and its L2), longest first within it.
 * Forward and dQ: query slots [r0, r1) of one sequence and the key slots
 * [s0, s1) any of them may see (for a part of a cut forward tile: its share
 * of them, the parts tiling the tile's range in part order).  Backward: key slots [r0, r1) and the query slots
 * [s0, s1) that may see them.  Copies min(count, capacity) items into out
 * (out may be NULL when capacity is 0) and stores the total count in *count.
 */
attn_status attn_plan_work_items(const attn_plan *plan, int32_t which, int32_t *out,
                                 int64_t capacity, int64_t *count);

/*
 * Rotary embedding of Q and K ("Upgrading a textbook decoder", section 2;
 * "Paired Head Attention", "Zero-copy RoPE" and "Staggered rotary"):
 * token t of its sequence, head h, is rotated by angle p * base^(-2i/d) on
 * pair i, p = t (unpaired) or 2t + (h mod 2) (paired):
 *     (a, b) -> (a cos - b sin, b cos + a sin).
 * q: [N, H, d], k: [N, Hkv, d] with token strides q_tok_stride >= H*d,
 * k_tok_stride >= Hkv*d (elements; e.g. 3*H*d for a packed [N, 3, H, d]
 * QKV).  q_out, k_out: dense [N, H, d] and [N, Hkv, d]; q_out == q (in place)
 * is allowed when q_tok_stride == H*d, same for k.  Written dense, the outputs
 * already are the paired interleaved layout.
 * v / v_out: when v_out is not NULL, V ([N, Hkv, dv], token stride
 * v_tok_stride >= Hkv*dv) is copied dense into v_out in the same pass; when
 * v_out is NULL, v is ignored.
 * ATTN_PAIRED_ADJACENT: the outputs are written in that layout's head order
 * (see Layouts), so v_out is required (V' feeds attn_fwd) and neither output
 * may alias its input (ATTN_E_INVALID otherwise).
 * QK norm ("Paired Head Attention", section "Source 4: Triton kernel
 * interleave indexing": the rotary kernel also applies the Q/K RMS-norm;
 * "Upgrading a textbook decoder", section 1 "RMSNorm"): when the plan sets
 * qk_norm, each head row of Q and K is divided by sqrt(mean(x^2) + eps)
 * before it is rotated, in the same pass.
 * The plan's rope mode must not be ATTN_ROPE_NONE (ATTN_E_INVALID).
 */
attn_status rope_qkv(const attn_plan *plan, const void *q, int64_t q_tok_stride, const void *k,
                     int64_t k_tok_stride, const void *v, int64_t v_tok_stride, void *q_out,
                     void *k_out, void *v_out, void *stream);

/*
 * rope_qkv with FP8 inputs, for the FP8 packed-QKV training path ("Paired
 * Head Attention" article, section 5, interplay with other mechanisms).  The
 * pages do not fix the format or scaling; this entry reads them as e4m3 codes
 * with one scale per tensor, dequantised in the rotary kernel so that no bf16
 * copy of the projection output is written first.  q, k, v hold e4m3 codes (OCP
 * FP8: sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities,
 * S.1111.111 is NaN) as bytes [N, H, d] / [N, Hkv, d] / [N, Hkv, dv] rows at
 * token strides q_tok_stride, k_tok_stride, v_tok_stride (in bytes =
 * elements); element
 * value = decoded code * scales[i] (scales: host array of 3 floats for q, k,
 * v, read before the call returns).  The dequantised rows then go through
 * exactly rope_qkv's steps (QK norm if set, rotation, adjacent permutation)
 * and are stored as bf16 q_out, k_out [N, H, d] / [N, Hkv, d]; v_out (bf16
 * [N, Hkv, dv], required) is the dequantised V in slot order.
 * bf16 plans only (ATTN_E_UNSUPPORTED otherwise).  Input pointers and strides
 * must be multiples of 8 bytes, outputs 16-byte aligned (ATTN_E_ALIGN);
 * outputs must not overlap the inputs; non-finite scales are ATTN_E_INVALID.
 */
attn_status rope_qkv_fp8(const attn_plan *plan, const void *q, int64_t q_tok_stride,
                         const void *k, int64_t k_tok_stride, const void *v,
                         int64_t v_tok_stride, const float *scales, void *q_out, void *k_out,
                         void *v_out, void *stream);

/*
 * Forward attention over the plan's sequences and mask (flash-style: the
 * N' x N' score matrix never reaches HBM; "Upgrading a textbook decoder",
 * section 4).  q: dense [N, H, d], k: [N, Hkv, d], v: [N, Hkv, dv], o:
 * [N, H, dv], in the plan's dtype (q, k already rotated); lse: float
 * [H', N'].  Every slot of o and lse
 * is written.
 */
attn_status attn_fwd(const attn_plan *plan, const void *q, const void *k, const void *v, void *o,
                     float *lse, void *stream);

/*
 * Backward of attn_fwd with respect to its inputs q, k, v (the rotated
 * values).  The pages print no correct backward: this is the chain rule
 * through the forward as defined ("mHC module" article, section 2.1:
 * softmax of the masked, scaled scores, times V) with the softmax Jacobian
 * diag(P) - P P^T; the backward printed in that article's section 4.1 is not
 * the derivative of softmax and is not followed.  Recomputing
 * P = exp(s q k^T - LSE):
 *     D_i = dO_i . O_i,  dS = P o (dO V^T - D),
 *     dV = P^T dO,  dQ = s dS K,  dK = s dS^T Q.
 * q: dense [N, H, d], k: [N, Hkv, d], v: [N, Hkv, dv], o, d_o: [N, H, dv], in
 * the plan's dtype; lse: float [H', N'] as written by attn_fwd; dq: float
 * [N, H, d], dk: float [N, Hkv, d], dv: float [N, Hkv, dv], fully overwritten.
 * With grouped K/V heads, dK and dV of a K/V head sum the contributions of
 * every query head of its group (float atomic adds, so their rounding order
 * may differ between runs; without grouping every output element is written
 * once and results are bit-reproducible).
 * bf16 only (ATTN_E_UNSUPPORTED for fp32).  Uses the workspace's scratch
 * area, so two attn_bwd calls sharing one workspace must not overlap.
 */
attn_status attn_bwd(const attn_plan *plan, const void *q, const void *k, const void *v,
                     const void *o, const float *lse, const void *d_o, float *dq, float *dk,
                     float *dv, void *stream);

/*
 * attn_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * the same computation, arguments, results (bit for bit) and errors as
 * attn_bwd, but its scratch (the D value of every attention head and slot,
 * H' x N' floats) lives in a device array of the library of 32 MiB per GPU
 * (kept until the process ends) instead of the plan's workspace.  The call
 * itself allocates nothing.  Problems with H' x N' x 4 bytes above 32 MiB
 * return ATTN_E_WORKSPACE.  Every call on one GPU shares that array (its
 * contents are rewritten by each call before use), so calls that overlap on
 * one GPU race: serialise them on one stream.  The stream's device (the
 * current device for the null stream) is where the array is looked up, once
 * per device, on its first call there.
 */
attn_status attn_bwd_noalloc(const attn_plan *plan, const void *q, const void *k, const void *v,
                             const void *o, const float *lse, const void *d_o, float *dq,
                             float *dk, float *dv, void *stream);

/*
 * Backward of rope_qkv: the gradients with respect to its inputs q, k (before
 * the norm and the rotation), given the gradients d_q, d_k of its outputs
 * Q', K' as attn_bwd writes them.  Per head row: rotation by -phi at the same
 * positions (the transpose of the rotation; same paired stagger), then, when
 * the plan sets qk_norm, the norm's gradient
 *     dx = r g - (r^3 / d) x (g . x),   r = 1 / sqrt(mean(x^2) + eps),
 * which needs the forward inputs q, k (plan dtype, token strides as in
 * rope_qkv; ignored and may be NULL without qk_norm).
 * d_q: float [N', H', d] slot layout (= [N, H, d] memory), d_k: likewise with
 * Hkv heads; dq_out, dk_out: float [N, H, d] / [N, Hkv, d] in head order.
 * d_v / dv_out (optional, both or neither; float [N, Hkv, dv]): dV copied
 * from the slot layout
 * into head order (V is not rotated; this only matters for the adjacent
 * pairing, whose slot layout permutes heads).
 * Outputs may alias d_q / d_k / d_v except with ATTN_PAIRED_ADJACENT
 * (ATTN_E_INVALID).  Floats 16-byte aligned; token strides of q, k multiples
 * of 8 (bf16) or 4 (fp32) elements.
 */
attn_status rope_qkv_bwd(const attn_plan *plan, const void *q, int64_t q_tok_stride,
                         const void *k, int64_t k_tok_stride, const float *d_q, const float *d_k,
                         const float *d_v, float *dq_out, float *dk_out, float *dv_out,
                         void *stream);

/* Static description of a status code. */
const char *attn_status_str(attn_status status);

/* Free a plan (NULL is a no-op).  Device memory is the caller's. */
void attn_plan_destroy(attn_plan *plan);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355_H */
