// plan.cpp -- host side of the library: problem validation, the plan
// (rotary table, per-token positions, tile work lists, exact counts), the
// workspace binding and the C-ABI entry points that check arguments before
// handing over to the gfx950 launchers.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <queue>

#include <hip/hip_runtime_api.h>

#include "attn_internal.h"
#include "launch.h"

using attn::WorkItem;

namespace {

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Visible (query, key) pairs of one sequence of L slots: the lower triangle
// with the diagonal, cut to a band of `window` diagonals when window > 0
// ("Paired Head Attention", section "Sequence length and window").
int64_t visible_pairs_of(int64_t L, int causal, int window) {
  if (L <= 0) return 0;
  if (!causal) return L * L;
  if (window <= 0 || L <= window) return L * (L + 1) / 2;
  const int64_t W = window;
  return W * (W + 1) / 2 + (L - W) * W;
}

// Tiles of `tile` slots of [b, e), each with the span of partner slots that
// can see it / be seen by it; appended as work items of `head`.
// forward=true:  item rows are queries, span = visible keys.
// forward=false: item rows are keys, span = queries that see them.
void cut_items(std::vector<WorkItem> &out, int head, int stream, int64_t b, int64_t e, int tile,
               int causal, int window, bool forward) {
  for (int64_t r0 = b; r0 < e; r0 += tile) {
    const int64_t r1 = std::min<int64_t>(r0 + tile, e);
    int64_t s0, s1;
    if (forward) {
      s0 = (window > 0) ? std::max<int64_t>(b, r0 - window + 1) : b;
      s1 = causal ? r1 : e;
    } else {
      s0 = causal ? r0 : b;
      s1 = (window > 0) ? std::min<int64_t>(e, r1 - 1 + window) : e;
    }
    WorkItem w{};
    w.head = head;
    w.q0 = (int32_t)r0;
    w.q1 = (int32_t)r1;
    w.k0 = (int32_t)s0;
    w.k1 = (int32_t)s1;
    w.pad0 = stream;
    out.push_back(w);
  }
}

int64_t steps_of(const WorkItem &w, int step) { return (w.k1 - w.k0 + step - 1) / step; }

// A work item with its scheduling bookkeeping.  `stream` numbers the
// (attention head, sequence) pairs; a query tile whose key range was cut into
// `parts` pieces keeps its index `item` on every piece.
struct Piece {
  WorkItem w;
  int64_t steps = 0;
  int32_t stream = 0, item = 0, part = 0, parts = 1;
};

// The items as pieces; items of more than `limit` steps (of `step` partner
// slots) are cut along their partner range at step boundaries:
// mode 0 into ceil(n / limit) parts of (nearly) equal length, mode 1 into
// parts of `limit` steps and a shorter last one.  Order is kept, the parts of
// an item adjacent.
std::vector<Piece> split_items(const std::vector<WorkItem> &v, int step, int64_t limit,
                               int mode) {
  std::vector<Piece> out;
  out.reserve(v.size());
  for (size_t i = 0; i < v.size(); ++i) {
    const int64_t n = steps_of(v[i], step);
    std::vector<int64_t> len;
    if (n <= limit) {
      len.push_back(n);
    } else if (mode == 0) {
      const int64_t parts = (n + limit - 1) / limit;
      for (int64_t p = 0; p < parts; ++p) len.push_back(n / parts + (p < n % parts ? 1 : 0));
    } else {
      for (int64_t r = n; r > 0; r -= limit) len.push_back(std::min(r, limit));
    }
    int64_t at = 0;
    for (size_t p = 0; p < len.size(); ++p) {
      Piece c;
      c.w = v[i];
      c.w.k0 = (int32_t)std::min<int64_t>(v[i].k1, v[i].k0 + at * step);
      c.w.k1 = (int32_t)std::min<int64_t>(v[i].k1, v[i].k0 + (at + len[p]) * step);
      at += len[p];
      c.steps = len[p];
      c.stream = v[i].pad0;
      c.item = (int32_t)i;
      c.part = (int32_t)p;
      c.parts = (int32_t)len.size();
      out.push_back(c);
    }
  }
  return out;
}

// Order pieces for the 8 XCDs of the chip.  Workgroup i runs on XCD i mod 8,
// and each XCD has its own L2, so items that read the same keys (one head of
// one sequence, nearby tiles) should share an XCD.  Pieces arrive in
// (stream, tile) order; runs of `chunk` consecutive items of one stream form
// a chunk (the parts of an item stay in its chunk).  Chunks go to XCDs by
// longest-processing-time (largest chunk to the least loaded XCD).  Inside an
// XCD the pieces run longest first (lpt = true), or chunk by chunk (the chunk
// with the longest piece first, its pieces longest first; lpt = false), which
// keeps fewer chunks' keys in flight at once.  Position 8j + x of the result
// is the j-th piece of XCD x; an XCD that runs out takes the next piece of
// the one with the most work left.
std::vector<Piece> order_for_xcds(const std::vector<Piece> &v, int chunk, bool lpt) {
  constexpr int kXcd = 8;
  struct Chunk {
    std::vector<Piece> pieces;
    int64_t work = 0, longest = 0;
    int items = 0;
  };
  std::vector<Chunk> chunks;
  for (size_t i = 0; i < v.size(); ++i) {
    const bool same_item = i > 0 && v[i].item == v[i - 1].item;
    const bool same_run = i > 0 && v[i].stream == v[i - 1].stream;
    if (!same_item && (!same_run || chunks.back().items == chunk)) chunks.emplace_back();
    Chunk &c = chunks.back();
    if (!same_item) ++c.items;
    c.pieces.push_back(v[i]);
    c.work += v[i].steps;
    c.longest = std::max<int64_t>(c.longest, v[i].steps);
  }
  const auto longer = [](const Piece &a, const Piece &b) { return a.steps > b.steps; };
  for (Chunk &c : chunks) std::stable_sort(c.pieces.begin(), c.pieces.end(), longer);
  std::vector<size_t> order(chunks.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(),
                   [&](size_t a, size_t b) { return chunks[a].work > chunks[b].work; });
  std::vector<std::vector<size_t>> xcd_chunks(kXcd);
  int64_t load[kXcd] = {0};
  for (size_t ci : order) {
    const int x = (int)(std::min_element(load, load + kXcd) - load);
    load[x] += chunks[ci].work;
    xcd_chunks[x].push_back(ci);
  }
  std::vector<std::vector<Piece>> q(kXcd);
  for (int x = 0; x < kXcd; ++x) {
    std::stable_sort(xcd_chunks[x].begin(), xcd_chunks[x].end(),
                     [&](size_t a, size_t b) { return chunks[a].longest > chunks[b].longest; });
    for (size_t ci : xcd_chunks[x])
      q[x].insert(q[x].end(), chunks[ci].pieces.begin(), chunks[ci].pieces.end());
    if (lpt) std::stable_sort(q[x].begin(), q[x].end(), longer);
  }
  std::vector<size_t> head(kXcd, 0);
  std::vector<int64_t> left(kXcd, 0);
  for (int x = 0; x < kXcd; ++x)
    for (const Piece &c : q[x]) left[x] += c.steps;
  std::vector<Piece> out;
  out.reserve(v.size());
  while (out.size() < v.size()) {
    const int x = (int)(out.size() % kXcd);
    int src = x;
    if (head[src] == q[src].size())
      src = (int)(std::max_element(left.begin(), left.end()) - left.begin());
    const Piece &c = q[src][head[src]++];
    left[src] -= c.steps;
    out.push_back(c);
  }
  return out;
}

// Makespan, in steps, of a launch order under a simple model of the chip:
// workgroup i goes to XCD i mod 8, each XCD starts its workgroups in order on
// `slots` block slots as they free up, and a block costs its steps plus one
// (loading its queries, writing its rows), plus two more when it is one part
// of a cut item (writing and reading the partial result).
double simulated_makespan(const std::vector<Piece> &order, int slots) {
  constexpr int kXcd = 8;
  double makespan = 0.0;
  for (int x = 0; x < kXcd; ++x) {
    std::priority_queue<double, std::vector<double>, std::greater<double>> free_at;
    for (int s = 0; s < slots; ++s) free_at.push(0.0);
    for (size_t i = x; i < order.size(); i += kXcd) {
      const double t = free_at.top() + (double)order[i].steps + 1.0 + (order[i].parts > 1 ? 2.0 : 0.0);
      free_at.pop();
      free_at.push(t);
      makespan = std::max(makespan, t);
    }
  }
  return makespan;
}

// The forward work list as launched, cut or not, and ordered for the XCDs.
// Query tiles longer than a third of the mean load of a block slot (and at
// least kMinCut steps) are cut into pieces of that many steps and a shorter
// last one, so that the end of each XCD's longest-first list holds short
// pieces; a cut is kept only when the list-schedule model above predicts a
// makespan at least 3% shorter than the uncut list's.  (Measured on the long
// causal problem, T = 16384: whole tiles 488 us, pieces of 204 / 128 / 64 / 32
// steps 466 / 469 / 448 / 477 us; on 8 x 1024 tokens, cutting its 16-step
// tiles into 2- to 8-step pieces was 3-85% slower: the merge of a part costs
// about a step, and a block alone on a CU runs faster than the model's
// equal-speed slots, so the model overstates the tail.)
// Returns the pieces; *groups receives the number of cut items.
std::vector<WorkItem> schedule_forward(const std::vector<WorkItem> &items, int step, int chunk,
                                       int slots_per_xcd, bool allow_split, int32_t *groups,
                                       int32_t *part_slots) {
  constexpr int64_t kMinCut = 16;
  std::vector<Piece> best = order_for_xcds(split_items(items, step, INT64_MAX, 0), chunk, true);
  if (allow_split && !items.empty()) {
    int64_t total = 0;
    for (const WorkItem &w : items) total += steps_of(w, step);
    const double mean = (double)total / (8.0 * slots_per_xcd);
    const int64_t limit = std::max<int64_t>(kMinCut, (int64_t)(mean / 3.0));
    std::vector<Piece> c = order_for_xcds(split_items(items, step, limit, 1), chunk, true);
    if (simulated_makespan(c, slots_per_xcd) < 0.97 * simulated_makespan(best, slots_per_xcd))
      best.swap(c);
  }
  // cut items: group index (counter) and partial-result slots, numbered in
  // item order so the parts of one item have consecutive slots
  std::vector<int32_t> parts_of(items.size(), 1), group_of(items.size(), -1),
      first_slot(items.size(), -1);
  for (const Piece &c : best) parts_of[(size_t)c.item] = c.parts;
  int32_t ng = 0, ns = 0;
  for (size_t i = 0; i < items.size(); ++i)
    if (parts_of[i] > 1) {
      group_of[i] = ng++;
      first_slot[i] = ns;
      ns += parts_of[i];
    }
  std::vector<WorkItem> out;
  out.reserve(best.size());
  for (const Piece &c : best) {
    WorkItem w = c.w;
    if (c.parts > 1) {
      w.pad0 = group_of[(size_t)c.item];
      w.pad1 = first_slot[(size_t)c.item] + c.part;
      w.pad2 = (c.part << 16) | c.parts;
    } else {
      w.pad0 = -1;
      w.pad1 = 0;
      w.pad2 = 1;
    }
    out.push_back(w);
  }
  *groups = ng;
  *part_slots = ns;
  return out;
}

// The backward lists, uncut, chunk by chunk inside each XCD.
void order_uncut(std::vector<WorkItem> &v, int step, int chunk) {
  std::vector<Piece> o = order_for_xcds(split_items(v, step, INT64_MAX, 0), chunk, false);
  for (size_t i = 0; i < v.size(); ++i) v[i] = o[i].w;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

namespace attn {

attn_status check_bwd_args(const attn_plan *p, const void *q, const void *k, const void *v,
                           const void *o, const float *lse, const void *d_o, float *dq,
                           float *dk, float *dv) {
  if (!p) return ATTN_E_INVALID;
  if (p->p.dtype != ATTN_BF16) return ATTN_E_UNSUPPORTED;
  if (!p->ws) return ATTN_E_WORKSPACE;
  if (p->p.N == 0) return ATTN_OK;
  if (!q || !k || !v || !o || !lse || !d_o || !dq || !dk || !dv) return ATTN_E_INVALID;
  const void *ptrs[] = {q, k, v, o, lse, d_o, dq, dk, dv};
  for (const void *x : ptrs)
    if (!aligned16(x)) return ATTN_E_ALIGN;
  return ATTN_OK;
}

}  // namespace attn

extern "C" {

const char *attn_status_str(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_E_INVALID: return "invalid argument";
    case ATTN_E_UNSUPPORTED: return "unsupported problem";
    case ATTN_E_ALIGN: return "misaligned pointer or stride";
    case ATTN_E_WORKSPACE: return "plan not bound or workspace too small";
    case ATTN_E_HIP: return "HIP runtime error";
    case ATTN_E_NOMEM: return "host allocation failed";
  }
  return "unknown status";
}

attn_status attn_plan_create(const attn_problem *pr, attn_plan **out) {
  if (!out) return ATTN_E_INVALID;
  *out = nullptr;
  if (!pr || !pr->cu_seqlens) return ATTN_E_INVALID;
  if (pr->num_tokens < 0 || pr->num_heads < 1 || pr->num_seqs < 1) return ATTN_E_INVALID;
  if (pr->dtype != ATTN_BF16 && pr->dtype != ATTN_FP32) return ATTN_E_INVALID;
  if (pr->causal != 0 && pr->causal != 1) return ATTN_E_INVALID;
  if (pr->window > 0 && !pr->causal) return ATTN_E_INVALID;
  if (pr->rope < ATTN_ROPE_NONE || pr->rope > ATTN_ROPE_ADJACENT) return ATTN_E_INVALID;
  if (pr->rope != ATTN_ROPE_NONE && !(pr->rope_base > 0.0 && std::isfinite(pr->rope_base)))
    return ATTN_E_INVALID;
  if (pr->paired != ATTN_UNPAIRED && pr->paired != ATTN_PAIRED &&
      pr->paired != ATTN_PAIRED_ADJACENT)
    return ATTN_E_INVALID;
  if (pr->paired && (pr->num_heads % 2)) return ATTN_E_INVALID;
  if (!std::isfinite(pr->softmax_scale) || pr->softmax_scale < 0.0f) return ATTN_E_INVALID;
  if (pr->qk_norm != 0 && pr->qk_norm != 1) return ATTN_E_INVALID;
  if (pr->qk_norm && pr->rope == ATTN_ROPE_NONE) return ATTN_E_INVALID;  // applied by rope_qkv
  if (!std::isfinite(pr->norm_eps) || pr->norm_eps < 0.0f) return ATTN_E_INVALID;
  if (pr->head_dim <= 0 || (pr->head_dim % 2)) return ATTN_E_INVALID;
  const int mult = pr->paired ? 2 : 1;
  // slots are int32 inside the kernels
  if (pr->num_tokens * mult > (int64_t(1) << 30)) return ATTN_E_UNSUPPORTED;
  const int32_t *cu = pr->cu_seqlens;
  const int S = pr->num_seqs;
  if (cu[0] != 0 || (int64_t)cu[S] != pr->num_tokens) return ATTN_E_INVALID;
  int64_t max_len = 0;
  for (int i = 0; i < S; ++i) {
    if (cu[i + 1] < cu[i]) return ATTN_E_INVALID;
    max_len = std::max<int64_t>(max_len, cu[i + 1] - cu[i]);
  }
  const int Hkv = pr->num_kv_heads == 0 ? pr->num_heads : pr->num_kv_heads;
  if (Hkv < 1 || pr->num_heads % Hkv) return ATTN_E_INVALID;
  if (pr->head_dim != 64 && pr->head_dim != 128) return ATTN_E_UNSUPPORTED;
  const int dv = pr->v_head_dim == 0 ? pr->head_dim : pr->v_head_dim;
  if (dv <= 0 || (dv % 2)) return ATTN_E_INVALID;
  if (dv != 64 && dv != 128) return ATTN_E_UNSUPPORTED;
  if (dv != pr->head_dim && pr->dtype != ATTN_BF16) return ATTN_E_UNSUPPORTED;
  if (Hkv != pr->num_heads && pr->paired) return ATTN_E_UNSUPPORTED;
  // tiles of up to 256 slots are addressed by 32-bit byte offsets, with an
  // offset of 2^31 standing for "out of range"
  if ((int64_t)pr->num_heads * std::max(pr->head_dim, dv) > (int64_t(1) << 20))
    return ATTN_E_UNSUPPORTED;

  attn_plan *p = new (std::nothrow) attn_plan();
  if (!p) return ATTN_E_NOMEM;
  try {
    attn::Problem &P = p->p;
    P.N = pr->num_tokens;
    P.H = pr->num_heads;
    P.d = pr->head_dim;
    P.dv = dv;
    P.dtype = pr->dtype;
    P.causal = pr->causal;
    // A window that spans the longest sequence hides nothing: it is no
    // window, which also keeps the kernels' slot + window sums inside int32.
    P.window = pr->window > 0 && (int64_t)pr->window < max_len * mult ? pr->window : 0;
    P.scale = pr->softmax_scale == 0.0f ? (float)(1.0 / std::sqrt((double)pr->head_dim))
                                         : pr->softmax_scale;
    P.rope = pr->rope;
    P.rope_base = pr->rope_base;
    P.paired = pr->paired;
    P.Hs = pr->paired ? P.H / 2 : P.H;
    P.Hkv = Hkv;
    P.Hks = pr->paired ? P.Hs : Hkv;
    P.G = P.Hs / P.Hks;
    P.qk_norm = pr->qk_norm;
    P.norm_eps = pr->norm_eps == 0.0f ? 1e-6f : pr->norm_eps;
    P.Ns = P.N * mult;
    p->cu.assign(cu, cu + S + 1);

    // Per-token offset inside its sequence (positions restart per sequence).
    p->tok_pos.resize((size_t)P.N);
    for (int s = 0; s < S; ++s)
      for (int32_t n = cu[s]; n < cu[s + 1]; ++n) p->tok_pos[(size_t)n] = n - cu[s];

    // Rotary table: cos and sin of angles p * base^(-2i/d) ("Upgrading a
    // textbook decoder", section 2), computed in fp64 and rounded once to
    // fp32.  Paired positions reach 2t + 1, so the range doubles.  Two levels,
    // so that the table stays in every XCD's L2: rows [0, F) hold the angles
    // lo * theta_i, rows F + hi the angles hi * F * theta_i (F = kRopeFine); the
    // kernels form position p = hi * F + lo by the angle-addition formulas.
    if (P.rope != ATTN_ROPE_NONE) {
      const int half = P.d / 2;
      constexpr int F = attn::kRopeFine;
      p->max_pos = (int32_t)std::max<int64_t>(1, max_len * mult);
      const int32_t rows = F + (p->max_pos + F - 1) / F;
      p->rope_cos.resize((size_t)rows * half);
      p->rope_sin.resize((size_t)rows * half);
      std::vector<double> theta(half);
      for (int i = 0; i < half; ++i) theta[i] = std::pow(P.rope_base, -2.0 * i / (double)P.d);
      for (int32_t r = 0; r < rows; ++r) {
        const double step = r < F ? (double)r : (double)(r - F) * F;
        for (int i = 0; i < half; ++i) {
          const double phi = step * theta[i];
          p->rope_cos[(size_t)r * half + i] = (float)std::cos(phi);
          p->rope_sin[(size_t)r * half + i] = (float)std::sin(phi);
        }
      }
    }

    // Work lists and exact counts.
    int64_t pairs = 0;
    int stream = 0;
    const bool bf16 = P.dtype == ATTN_BF16;  // the backward is bf16 only
    const bool short_rows = (P.window > 0 && P.window <= attn::kFwdShortWindow) ||
                            max_len * mult <= attn::kFwdShortSeq || (P.d == 64 && P.dv == 64);
    p->fwd_bq = !bf16 ? attn::kFwdBQF32 : short_rows ? attn::kFwdBQShort : attn::kFwdBQ;
    // One stream per (K/V head, sequence).  With grouped K/V heads, the items
    // of the group's query heads are interleaved tile by tile, so the ones
    // that read the same K/V rows land in one chunk (one XCD, one L2).
    std::vector<std::vector<WorkItem>> tf(P.G), tq(P.G), tb(P.G);
    auto interleave = [](std::vector<std::vector<WorkItem>> &parts, std::vector<WorkItem> &out) {
      for (size_t i = 0;; ++i) {
        bool any = false;
        for (auto &v : parts)
          if (i < v.size()) {
            out.push_back(v[i]);
            any = true;
          }
        if (!any) break;
      }
      for (auto &v : parts) v.clear();
    };
    const int bwd_rows = 32 * attn::bwd_waves(P.d, P.dv);  // backward item rows
    for (int kh = 0; kh < P.Hks; ++kh)
      for (int s = 0; s < S; ++s) {
        const int64_t b = (int64_t)cu[s] * mult, e = (int64_t)cu[s + 1] * mult;
        if (e == b) continue;
        for (int g = 0; g < P.G; ++g) {
          const int j = kh * P.G + g;  // query attention head
          pairs += visible_pairs_of(e - b, P.causal, P.window);
          cut_items(tf[g], j, stream, b, e, p->fwd_bq, P.causal, P.window, true);
          if (bf16) {
            cut_items(tq[g], j, stream, b, e, bwd_rows, P.causal, P.window, true);
            cut_items(tb[g], j, stream, b, e, bwd_rows, P.causal, P.window, false);
          }
        }
        interleave(tf, p->fwd);
        interleave(tq, p->dq);
        interleave(tb, p->bwd);  // per query head; grouped heads add into dK/dV
        ++stream;
      }
    // forward: long query tiles are cut along their keys when that shortens
    // the launch (bf16 kernels merge the parts); the backward lists stay whole
    const int fwd_slots = attn::kCUs / 8 * attn::fwd_blocks_per_cu(P.dtype, P.d, P.dv, p->fwd_bq);
    p->fwd = schedule_forward(p->fwd, attn::kFwdBK, attn::kXcdChunk, fwd_slots, bf16,
                              &p->fwd_groups, &p->fwd_part_slots);
    order_uncut(p->bwd, attn::kBwdBQ, attn::kXcdChunk);
    order_uncut(p->dq, attn::kFwdBK, attn::kXcdChunk);

    const double elems = (double)P.N * P.H * P.d;       // Q, dQ
    const double kv_elems = (double)P.N * P.Hkv * P.d;  // K, dK
    const double o_elems = (double)P.N * P.H * P.dv;    // O, dO
    const double v_elems = (double)P.N * P.Hkv * P.dv;  // V, dV
    const double es = P.dtype == ATTN_BF16 ? 2.0 : 4.0;
    const double lse_bytes = 4.0 * (double)P.Ns * P.Hs;
    attn_plan_info &I = p->info;
    I.visible_pairs = pairs;
    I.fwd_flops = 2.0 * (P.d + P.dv) * (double)pairs;
    I.bwd_flops = 2.0 * (3.0 * P.d + 2.0 * P.dv) * (double)pairs;
    I.rope_bytes = 2.0 * (elems + kv_elems) * es;
    I.fwd_bytes = (elems + kv_elems + v_elems + o_elems) * es + lse_bytes;
    I.bwd_bytes = (elems + kv_elems + v_elems + 2.0 * o_elems) * es + lse_bytes +
                  (elems + kv_elems + v_elems) * 4.0;
    I.fwd_items = (int64_t)p->fwd.size();
    I.fwd_split_items = p->fwd_groups;
    I.bwd_items = (int64_t)p->bwd.size();
    I.slots = P.Ns;
    I.attn_heads = P.Hs;
    I.kv_heads = P.Hks;
    I.v_head_dim = P.dv;
    I.max_positions = p->max_pos;

    // Workspace layout.
    size_t off = 0;
    p->off_pos = off;
    off = align256(off + sizeof(int32_t) * p->tok_pos.size());
    p->off_cos = off;
    off = align256(off + sizeof(float) * p->rope_cos.size());
    p->off_sin = off;
    off = align256(off + sizeof(float) * p->rope_sin.size());
    p->off_fwd = off;
    off = align256(off + sizeof(WorkItem) * p->fwd.size());
    p->off_bwd = off;
    off = align256(off + sizeof(WorkItem) * p->bwd.size());
    p->off_dq = off;
    off = align256(off + sizeof(WorkItem) * p->dq.size());
    p->off_delta = off;
    off = align256(off + sizeof(float) * (size_t)P.Ns * P.Hs);
    p->zero_counters.assign((size_t)p->fwd_groups, 0);
    p->off_split_cnt = off;
    off = align256(off + sizeof(int32_t) * (size_t)p->fwd_groups);
    p->off_split_part = off;
    off = align256(off + attn::fwd_partial_bytes(P.dv, p->fwd_bq) * (size_t)p->fwd_part_slots);
    p->ws_bytes = std::max<size_t>(off, 256);
  } catch (const std::bad_alloc &) {
    delete p;
    return ATTN_E_NOMEM;
  }
  *out = p;
  return ATTN_OK;
}

size_t attn_plan_workspace_bytes(const attn_plan *p) { return p ? p->ws_bytes : 0; }

attn_status attn_plan_bind(attn_plan *p, void *ws, size_t bytes, void *stream) {
  if (!p || !ws) return ATTN_E_INVALID;
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return ATTN_E_ALIGN;
  if (bytes < p->ws_bytes) return ATTN_E_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char *base = static_cast<char *>(ws);
  struct Sec {
    size_t off;
    const void *src;
    size_t n;
  } secs[] = {
      {p->off_pos, p->tok_pos.data(), sizeof(int32_t) * p->tok_pos.size()},
      {p->off_cos, p->rope_cos.data(), sizeof(float) * p->rope_cos.size()},
      {p->off_sin, p->rope_sin.data(), sizeof(float) * p->rope_sin.size()},
      {p->off_fwd, p->fwd.data(), sizeof(WorkItem) * p->fwd.size()},
      {p->off_bwd, p->bwd.data(), sizeof(WorkItem) * p->bwd.size()},
      {p->off_dq, p->dq.data(), sizeof(WorkItem) * p->dq.size()},
      {p->off_split_cnt, p->zero_counters.data(), sizeof(int32_t) * p->zero_counters.size()},
  };
  for (const Sec &s : secs) {
    if (s.n == 0) continue;
    if (hipMemcpyAsync(base + s.off, s.src, s.n, hipMemcpyHostToDevice, st) != hipSuccess)
      return ATTN_E_HIP;
  }
  p->ws = base;
  return ATTN_OK;
}

attn_status attn_plan_stats(const attn_plan *p, attn_plan_info *info) {
  if (!p || !info) return ATTN_E_INVALID;
  *info = p->info;
  return ATTN_OK;
}

attn_status attn_plan_work_items(const attn_plan *p, int32_t which, int32_t *out,
                                 int64_t capacity, int64_t *count) {
  if (!p || !count || which < 0 || which > 2 || capacity < 0) return ATTN_E_INVALID;
  const std::vector<WorkItem> &v = which == 0 ? p->fwd : which == 1 ? p->bwd : p->dq;
  *count = (int64_t)v.size();
  const int64_t n = std::min<int64_t>(capacity, (int64_t)v.size());
  if (n > 0 && !out) return ATTN_E_INVALID;
  if (n > 0) std::memcpy(out, v.data(), sizeof(WorkItem) * (size_t)n);
  return ATTN_OK;
}

void attn_plan_destroy(attn_plan *p) { delete p; }

attn_status rope_qkv(const attn_plan *p, const void *q, int64_t qs, const void *k, int64_t ks,
                     const void *v, int64_t vs, void *q_out, void *k_out, void *v_out,
                     void *stream) {
  if (!p) return ATTN_E_INVALID;
  if (p->p.rope == ATTN_ROPE_NONE) return ATTN_E_INVALID;
  if (!p->ws) return ATTN_E_WORKSPACE;
  const int64_t row = (int64_t)p->p.H * p->p.d;
  const int64_t kv_row = (int64_t)p->p.Hkv * p->p.d;
  const int64_t v_row = (int64_t)p->p.Hkv * p->p.dv;
  if (p->p.N == 0) return ATTN_OK;
  if (!q || !k || !q_out || !k_out || (v_out && !v)) return ATTN_E_INVALID;
  if (qs < row || ks < kv_row || (v_out && vs < v_row)) return ATTN_E_INVALID;
  const int64_t vec = p->p.dtype == ATTN_BF16 ? 8 : 4;
  if (qs % vec || ks % vec || (v_out && vs % vec)) return ATTN_E_ALIGN;
  if (!aligned16(q) || !aligned16(k) || !aligned16(q_out) || !aligned16(k_out) ||
      (v_out && (!aligned16(v) || !aligned16(v_out))))
    return ATTN_E_ALIGN;
  if ((q_out == q && qs != row) || (k_out == k && ks != kv_row)) return ATTN_E_INVALID;
  // the adjacent pairing permutes heads on store: V must be copied with them,
  // and an in-place store would overwrite heads not yet read
  if (p->p.paired == ATTN_PAIRED_ADJACENT && (!v_out || q_out == q || k_out == k))
    return ATTN_E_INVALID;
  return attn::launch_rope(p, q, qs, k, ks, v_out ? v : nullptr, vs, q_out, k_out, v_out,
                           static_cast<hipStream_t>(stream));
}

attn_status rope_qkv_fp8(const attn_plan *p, const void *q, int64_t qs, const void *k,
                         int64_t ks, const void *v, int64_t vs, const float *scales, void *q_out,
                         void *k_out, void *v_out, void *stream) {
  if (!p) return ATTN_E_INVALID;
  if (p->p.rope == ATTN_ROPE_NONE) return ATTN_E_INVALID;
  if (p->p.dtype != ATTN_BF16) return ATTN_E_UNSUPPORTED;
  if (!p->ws) return ATTN_E_WORKSPACE;
  if (!scales) return ATTN_E_INVALID;
  for (int i = 0; i < 3; ++i)
    if (!std::isfinite(scales[i])) return ATTN_E_INVALID;
  if (p->p.N == 0) return ATTN_OK;
  const int64_t row = (int64_t)p->p.H * p->p.d;
  const int64_t kv_row = (int64_t)p->p.Hkv * p->p.d;
  const int64_t v_row = (int64_t)p->p.Hkv * p->p.dv;
  if (!q || !k || !v || !q_out || !k_out || !v_out) return ATTN_E_INVALID;
  if (qs < row || ks < kv_row || vs < v_row) return ATTN_E_INVALID;
  // one load covers 8 codes
  const auto a8 = [](const void *x) { return (reinterpret_cast<uintptr_t>(x) & 7) == 0; };
  if (qs % 8 || ks % 8 || vs % 8 || !a8(q) || !a8(k) || !a8(v)) return ATTN_E_ALIGN;
  if (!aligned16(q_out) || !aligned16(k_out) || !aligned16(v_out)) return ATTN_E_ALIGN;
  if (q_out == q || k_out == k || v_out == v) return ATTN_E_INVALID;
  return attn::launch_rope_fp8(p, q, qs, k, ks, v, vs, scales, q_out, k_out, v_out,
                               static_cast<hipStream_t>(stream));
}

attn_status rope_qkv_bwd(const attn_plan *p, const void *q, int64_t qs, const void *k,
                         int64_t ks, const float *d_q, const float *d_k, const float *d_v,
                         float *dq_out, float *dk_out, float *dv_out, void *stream) {
  if (!p) return ATTN_E_INVALID;
  if (p->p.rope == ATTN_ROPE_NONE) return ATTN_E_INVALID;
  if (!p->ws) return ATTN_E_WORKSPACE;
  if (p->p.N == 0) return ATTN_OK;
  if (!d_q || !d_k || !dq_out || !dk_out || (!d_v != !dv_out)) return ATTN_E_INVALID;
  const void *fl[] = {d_q, d_k, dq_out, dk_out, d_v, dv_out};
  for (const void *x : fl)
    if (x && !aligned16(x)) return ATTN_E_ALIGN;
  if (p->p.paired == ATTN_PAIRED_ADJACENT &&
      (dq_out == d_q || dk_out == d_k || (dv_out && dv_out == d_v)))
    return ATTN_E_INVALID;
  if (p->p.qk_norm) {
    const int64_t row = (int64_t)p->p.H * p->p.d, kv_row = (int64_t)p->p.Hkv * p->p.d;
    if (!q || !k) return ATTN_E_INVALID;
    if (qs < row || ks < kv_row) return ATTN_E_INVALID;
    const int64_t vec = p->p.dtype == ATTN_BF16 ? 8 : 4;
    if (qs % vec || ks % vec || !aligned16(q) || !aligned16(k)) return ATTN_E_ALIGN;
  }
  return attn::launch_rope_bwd(p, p->p.qk_norm ? q : nullptr, qs, p->p.qk_norm ? k : nullptr, ks,
                               d_q, d_k, d_v, dq_out, dk_out, dv_out,
                               static_cast<hipStream_t>(stream));
}

attn_status attn_fwd(const attn_plan *p, const void *q, const void *k, const void *v, void *o,
                     float *lse, void *stream) {
  if (!p) return ATTN_E_INVALID;
  if (!p->ws) return ATTN_E_WORKSPACE;
  if (p->p.N == 0) return ATTN_OK;
  if (!q || !k || !v || !o || !lse) return ATTN_E_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return ATTN_E_ALIGN;
  return attn::launch_fwd(p, q, k, v, o, lse, static_cast<hipStream_t>(stream));
}

attn_status attn_bwd(const attn_plan *p, const void *q, const void *k, const void *v,
                     const void *o, const float *lse, const void *d_o, float *dq, float *dk,
                     float *dv, void *stream) {
  const attn_status st = attn::check_bwd_args(p, q, k, v, o, lse, d_o, dq, dk, dv);
  if (st != ATTN_OK || p->p.N == 0) return st;
  return attn::launch_bwd(p, q, k, v, o, lse, d_o, dq, dk, dv,
                          reinterpret_cast<float *>(p->ws + p->off_delta),
                          static_cast<hipStream_t>(stream));
}

}  // extern "C"
