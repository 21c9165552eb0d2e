/*
 * oracle.c -- plain fp64 CPU oracle for rotary causal self-attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header or table with the GPU path.
 *
 * Everything is computed in double precision, one score row at a time, with
 * no tiling, no online softmax and no fusion: the obvious definition written
 * out.  Sources (page title, section):
 *
 *  - Rotation and frequencies: "Upgrading a textbook decoder (FlashAttention,
 *    GQA, RoPE, RMSNorm, SwiGLU)" (juejin.cn), section 2 "RoPE":
 *    inv_freq_i = 1 / base^(2i/d); rotate_half pairs element i with i + d/2
 *    and maps (a, b) -> (a cos - b sin, b cos + a sin).
 *  - Adjacent-pair rotation: "Paired Head Attention" record article
 *    (hncyxsy.com), section "Zero-copy RoPE: one-line rotary()": the partner of
 *    an element is the other element of its (2i, 2i+1) pair (x_flip).
 *  - Paired positions: same article, sections "Staggered rotary" and
 *    "Source 2: paired rotary table": token t of head h is rotated at position
 *    2t + (h mod 2).
 *  - Paired slots: same article, sections "Core idea" and "Source 4: Triton
 *    kernel interleave indexing": head h of token t goes to slot
 *    2t + floor(h / (H/2)) of attention head h mod (H/2); sequence boundaries
 *    double ("Sequence length and window").
 *  - Mask and softmax: "SingleHeadAttention" note (ranhao.site), forward():
 *    lower-triangular mask with -inf fill, softmax over the row;
 *    "mHC module" article (lshu.cn), section 2.2: max-subtracted softmax;
 *    section 2.1: softmax(Q K^T / sqrt(d_k)) V.
 *  - Window: "Paired Head Attention" article, section "Sequence length and
 *    window": a window of 128 key slots covers 64 positions of each paired
 *    head, i.e. key slot j is visible from query slot i iff 0 <= i - j < W.
 *  - Backward: the gradient of L = sum(O * dO) through softmax(s Q K^T) V,
 *    written from the chain rule (the softmax Jacobian is diag(P) - P P^T).
 *  - QK RMS-norm before the rotation: "Paired Head Attention" article,
 *    section "Source 4: Triton kernel interleave indexing" (the RoPE kernel
 *    also applies the Q/K RMS-norm, and its backward uses the same index map);
 *    the norm itself: "Upgrading a textbook decoder", section 1 "RMSNorm",
 *    x / sqrt(mean(x^2) + eps) with eps = 1e-6.
 *
 *  - Separate value width: "Paired Head Attention" article, section "Source 1:
 *    model configuration" (each attention module takes its own qk_dim and
 *    v_dim): q, k carry d features and v, dO, O, dV carry dv; the scores use
 *    q . k over d, the output sums P v over dv.
 *
 * Conventions: tensors are row-major [N, H, d] (token, head, feature); v and
 * the tensors shaped like it are [N, H, dv].
 * paired = 0: slot = token, attention head = h.
 * paired = 1: slot = 2 t + h / (H/2), attention head = h mod (H/2)
 *             (the article's code: view of [T, H, d] as [2T, H/2, d]).
 * paired = 2: slot = 2 t + h mod 2, attention head = h / 2
 *             (the article's prose: adjacent heads h, h^1 form a pair).
 * LSE is laid out [H', N'] (attention head, slot) and uses the natural log.
 *
 * Return values: 0 on success, -1 on an invalid argument, -2 on allocation
 * failure.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_EINVAL (-1)
#define OR_ENOMEM (-2)

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* cu_seqlens must start at 0, be non-decreasing and end at N. */
static int check_cu(const int32_t *cu, int S, int64_t N) {
  if (!cu || S < 0) return 0;
  if (cu[0] != 0) return 0;
  for (int k = 0; k < S; ++k)
    if (cu[k + 1] < cu[k]) return 0;
  return (int64_t)cu[S] == N;
}

static int check_shape(int64_t N, int H, int d, int paired) {
  if (N < 0 || H <= 0 || d <= 0) return 0;
  if (paired < 0 || paired > 2) return 0;
  if (paired && (H % 2) != 0) return 0;
  return 1;
}

/* Rotation position of (token offset t inside its sequence, head h). */
static int64_t rope_position(int64_t t, int h, int paired) {
  return paired ? 2 * t + (h % 2) : t;
}

/* Map logical (token n, head h) to (slot, attention head). */
int oracle_slot_map(int64_t n, int h, int H, int paired, int64_t *slot, int *head) {
  if (H <= 0 || h < 0 || h >= H || !slot || !head) return OR_EINVAL;
  if (paired == 0) {
    *slot = n;
    *head = h;
  } else if (paired == 1) {
    if (H % 2) return OR_EINVAL;
    *slot = 2 * n + h / (H / 2);
    *head = h % (H / 2);
  } else if (paired == 2) {
    if (H % 2) return OR_EINVAL;
    *slot = 2 * n + (h % 2);
    *head = h / 2;
  } else {
    return OR_EINVAL;
  }
  return OR_OK;
}

/*
 * y = RoPE(x) for x of shape [N, H, d].  convention 1 = half-split pairs
 * (i, i + d/2), convention 2 = adjacent pairs (2i, 2i + 1).  Positions restart
 * at 0 at every sequence start given by cu (cu has S + 1 entries).
 */
int oracle_rope(const double *x, int64_t N, int H, int d, const int32_t *cu, int S,
                int convention, double base, int paired, double *y) {
  if (!x || !y || !check_shape(N, H, d, paired) || !check_cu(cu, S, N)) return OR_EINVAL;
  if (convention != 1 && convention != 2) return OR_EINVAL;
  if (d % 2) return OR_EINVAL; /* rotation acts on pairs */
  if (!(base > 0.0)) return OR_EINVAL;
  const int half = d / 2;
  for (int k = 0; k < S; ++k) {
    const int64_t start = cu[k], end = cu[k + 1];
#pragma omp parallel for schedule(static)
    for (int64_t n = start; n < end; ++n) {
      const int64_t t = n - start;
      for (int h = 0; h < H; ++h) {
        const double *xr = x + (n * H + h) * (int64_t)d;
        double *yr = y + (n * H + h) * (int64_t)d;
        const double p = (double)rope_position(t, h, paired);
        for (int i = 0; i < half; ++i) {
          const double theta = pow(base, -2.0 * (double)i / (double)d);
          const double phi = p * theta;
          const double c = cos(phi), s = sin(phi);
          const int ia = (convention == 1) ? i : 2 * i;
          const int ib = (convention == 1) ? i + half : 2 * i + 1;
          const double a = xr[ia], b = xr[ib];
          yr[ia] = a * c - b * s;
          yr[ib] = b * c + a * s;
        }
      }
    }
  }
  return OR_OK;
}

/*
 * Transpose of oracle_rope: every pair rotated by -phi at the same positions
 * (a rotation matrix is orthogonal, its transpose is its inverse):
 * (a, b) -> (a cos + b sin, b cos - a sin).  This carries a gradient with
 * respect to the rotated values back to the values before the rotation.
 */
int oracle_rope_bwd(const double *dy, int64_t N, int H, int d, const int32_t *cu, int S,
                    int convention, double base, int paired, double *dx) {
  if (!dy || !dx || !check_shape(N, H, d, paired) || !check_cu(cu, S, N)) return OR_EINVAL;
  if (convention != 1 && convention != 2) return OR_EINVAL;
  if (d % 2) return OR_EINVAL;
  if (!(base > 0.0)) return OR_EINVAL;
  const int half = d / 2;
  for (int k = 0; k < S; ++k) {
    const int64_t start = cu[k], end = cu[k + 1];
#pragma omp parallel for schedule(static)
    for (int64_t n = start; n < end; ++n) {
      const int64_t t = n - start;
      for (int h = 0; h < H; ++h) {
        const double *yr = dy + (n * H + h) * (int64_t)d;
        double *xr = dx + (n * H + h) * (int64_t)d;
        const double p = (double)rope_position(t, h, paired);
        for (int i = 0; i < half; ++i) {
          const double phi = p * pow(base, -2.0 * (double)i / (double)d);
          const double c = cos(phi), s = sin(phi);
          const int ia = (convention == 1) ? i : 2 * i;
          const int ib = (convention == 1) ? i + half : 2 * i + 1;
          const double a = yr[ia], b = yr[ib];
          xr[ia] = a * c + b * s;
          xr[ib] = b * c - a * s;
        }
      }
    }
  }
  return OR_OK;
}

/*
 * RMS normalisation of each of `rows` rows of d values ("Upgrading a textbook
 * decoder", section 1 "RMSNorm"): y = x / sqrt(mean(x^2) + eps), without a
 * gain (a gain of ones).
 */
int oracle_rms_norm(const double *x, int64_t rows, int d, double eps, double *y) {
  if (!x || !y || rows < 0 || d <= 0 || !(eps >= 0.0)) return OR_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const double *xr = x + r * d;
    double ms = 0.0;
    for (int i = 0; i < d; ++i) ms += xr[i] * xr[i];
    ms /= d;
    const double inv = 1.0 / sqrt(ms + eps);
    for (int i = 0; i < d; ++i) y[r * d + i] = xr[i] * inv;
  }
  return OR_OK;
}

/*
 * Gradient of oracle_rms_norm.  With r = 1 / sqrt(mean(x^2) + eps), y_i = x_i r
 * and dr/dx_j = -r^3 x_j / d, so the chain rule gives
 *     dx_j = r dy_j - (r^3 / d) x_j sum_i dy_i x_i.
 */
int oracle_rms_norm_bwd(const double *x, const double *dy, int64_t rows, int d, double eps,
                        double *dx) {
  if (!x || !dy || !dx || rows < 0 || d <= 0 || !(eps >= 0.0)) return OR_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const double *xr = x + r * d, *gr = dy + r * d;
    double ms = 0.0, xg = 0.0;
    for (int i = 0; i < d; ++i) {
      ms += xr[i] * xr[i];
      xg += xr[i] * gr[i];
    }
    ms /= d;
    const double inv = 1.0 / sqrt(ms + eps);
    const double c = inv * inv * inv / d * xg;
    for (int i = 0; i < d; ++i) dx[r * d + i] = inv * gr[i] - c * xr[i];
  }
  return OR_OK;
}

/* ---------------------------------------------------------------------- */
/* Attention over slots.                                                   */

typedef struct {
  int64_t N, Ns;     /* tokens, slots */
  int H, Hs, d, dv;  /* heads given, attention heads, q/k head dim, v head dim */
  int paired, causal, window;
  double scale;
  int S;
  int64_t *cus;      /* slot boundaries, S + 1 entries */
  double *q, *k;     /* gathered [Hs][Ns][d] */
  double *v, *g;     /* gathered [Hs][Ns][dv]; g = dO (may be NULL) */
} problem;

static void problem_free(problem *p) {
  free(p->cus);
  free(p->q);
  free(p->k);
  free(p->v);
  free(p->g);
}

/* Gather a logical [N, H, w] tensor into [Hs][Ns][w] slot order. */
static void gather(const double *src, const problem *p, int w, double *dst) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < p->N; ++n)
    for (int h = 0; h < p->H; ++h) {
      int64_t s;
      int j;
      oracle_slot_map(n, h, p->H, p->paired, &s, &j);
      memcpy(dst + ((int64_t)j * p->Ns + s) * w, src + (n * p->H + h) * (int64_t)w,
             sizeof(double) * (size_t)w);
    }
}

/* Scatter [Hs][Ns][w] slot order back to a logical [N, H, w] tensor. */
static void scatter(const double *src, const problem *p, int w, double *dst) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < p->N; ++n)
    for (int h = 0; h < p->H; ++h) {
      int64_t s;
      int j;
      oracle_slot_map(n, h, p->H, p->paired, &s, &j);
      memcpy(dst + (n * p->H + h) * (int64_t)w, src + ((int64_t)j * p->Ns + s) * w,
             sizeof(double) * (size_t)w);
    }
}

static int problem_init(problem *p, const double *q, const double *k, const double *v,
                        const double *dout, int64_t N, int H, int d, int dv, const int32_t *cu,
                        int S, int paired, int causal, int window, double scale) {
  memset(p, 0, sizeof(*p));
  if (!q || !k || !v || !check_shape(N, H, d, paired) || dv < 1 || !check_cu(cu, S, N))
    return OR_EINVAL;
  if (window > 0 && !causal) return OR_EINVAL;
  p->N = N;
  p->H = H;
  p->d = d;
  p->dv = dv;
  p->paired = paired;
  p->Hs = paired ? H / 2 : H;
  p->Ns = paired ? 2 * N : N;
  p->causal = causal;
  p->window = window;
  p->scale = (scale == 0.0) ? 1.0 / sqrt((double)d) : scale;
  p->S = S;
  const size_t elems = (size_t)p->Ns * (size_t)p->Hs * (size_t)d;
  const size_t velems = (size_t)p->Ns * (size_t)p->Hs * (size_t)dv;
  p->cus = (int64_t *)malloc(sizeof(int64_t) * (size_t)(S + 1));
  p->q = (double *)malloc(sizeof(double) * (elems ? elems : 1));
  p->k = (double *)malloc(sizeof(double) * (elems ? elems : 1));
  p->v = (double *)malloc(sizeof(double) * (velems ? velems : 1));
  if (dout) p->g = (double *)malloc(sizeof(double) * (velems ? velems : 1));
  if (!p->cus || !p->q || !p->k || !p->v || (dout && !p->g)) {
    problem_free(p);
    return OR_ENOMEM;
  }
  for (int i = 0; i <= S; ++i) p->cus[i] = (int64_t)cu[i] * (paired ? 2 : 1);
  gather(q, p, d, p->q);
  gather(k, p, d, p->k);
  gather(v, p, dv, p->v);
  if (dout) gather(dout, p, dv, p->g);
  return OR_OK;
}

/* Index of the sequence that holds slot i. */
static int doc_of(const problem *p, int64_t i) {
  int lo = 0, hi = p->S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (p->cus[mid] <= i) lo = mid;
    else hi = mid - 1;
  }
  while (lo < p->S && p->cus[lo + 1] <= i) ++lo; /* skip empty sequences */
  return lo;
}

/* Is key slot jj visible from query slot i (both inside sequence [b, e))? */
static int visible(const problem *p, int64_t i, int64_t jj, int64_t b, int64_t e) {
  if (jj < b || jj >= e) return 0;
  if (p->causal && jj > i) return 0;
  if (p->window > 0 && i - jj >= p->window) return 0;
  return 1;
}

static double dot(const double *a, const double *b, int d) {
  double s = 0.0;
  for (int c = 0; c < d; ++c) s += a[c] * b[c];
  return s;
}

/*
 * Score row of query slot i of head j: z[jj - b] = scale * q_i . k_jj for
 * visible keys, -inf otherwise.  Returns the row max m and the sum
 * l = sum exp(z - m).
 */
static void score_row(const problem *p, int j, int64_t i, double *z, double *m_out,
                      double *l_out) {
  const int d = p->d;
  const int doc = doc_of(p, i);
  const int64_t b = p->cus[doc], e = p->cus[doc + 1];
  const double *qi = p->q + ((int64_t)j * p->Ns + i) * d;
  double m = -INFINITY;
  for (int64_t jj = b; jj < e; ++jj) {
    if (!visible(p, i, jj, b, e)) {
      z[jj - b] = -INFINITY;
      continue;
    }
    const double zz = p->scale * dot(qi, p->k + ((int64_t)j * p->Ns + jj) * d, d);
    z[jj - b] = zz;
    if (zz > m) m = zz;
  }
  double l = 0.0;
  for (int64_t jj = b; jj < e; ++jj)
    if (z[jj - b] != -INFINITY) l += exp(z[jj - b] - m);
  *m_out = m;
  *l_out = l;
}

static int64_t max_doc_len(const problem *p) {
  int64_t mx = 1;
  for (int k = 0; k < p->S; ++k)
    if (p->cus[k + 1] - p->cus[k] > mx) mx = p->cus[k + 1] - p->cus[k];
  return mx;
}

/* Forward of one row: o (dv values) and lse. */
static void fwd_row(const problem *p, int j, int64_t i, double *z, double *o, double *lse) {
  const int dv = p->dv;
  const int doc = doc_of(p, i);
  const int64_t b = p->cus[doc], e = p->cus[doc + 1];
  double m, l;
  score_row(p, j, i, z, &m, &l);
  for (int c = 0; c < dv; ++c) o[c] = 0.0;
  for (int64_t jj = b; jj < e; ++jj) {
    if (z[jj - b] == -INFINITY) continue;
    const double pij = exp(z[jj - b] - m) / l;
    const double *vj = p->v + ((int64_t)j * p->Ns + jj) * dv;
    for (int c = 0; c < dv; ++c) o[c] += pij * vj[c];
  }
  *lse = m + log(l);
}

/*
 * Full forward.  q, k: [N, H, d] (already rotated); v, o: [N, H, dv]; lse:
 * [H', N'].  scale == 0 selects 1 / sqrt(d).
 */
int oracle_attn_fwd(const double *q, const double *k, const double *v, int64_t N, int H, int d,
                    int dv, const int32_t *cu, int S, int paired, int causal, int window,
                    double scale, double *o, double *lse) {
  problem p;
  int rc = problem_init(&p, q, k, v, NULL, N, H, d, dv, cu, S, paired, causal, window, scale);
  if (rc) return rc;
  if (!o || !lse) {
    problem_free(&p);
    return OR_EINVAL;
  }
  const size_t elems = (size_t)p.Ns * (size_t)p.Hs * (size_t)dv;
  double *os = (double *)malloc(sizeof(double) * (elems ? elems : 1));
  if (!os) {
    problem_free(&p);
    return OR_ENOMEM;
  }
  const int64_t L = max_doc_len(&p);
  int fail = 0;
#pragma omp parallel
  {
    double *z = (double *)malloc(sizeof(double) * (size_t)L);
    if (!z) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(dynamic, 16) collapse(2)
    for (int j = 0; j < p.Hs; ++j)
      for (int64_t i = 0; i < p.Ns; ++i)
        if (z) fwd_row(&p, j, i, z, os + ((int64_t)j * p.Ns + i) * dv, lse + (int64_t)j * p.Ns + i);
    free(z);
  }
  if (!fail) scatter(os, &p, dv, o);
  free(os);
  problem_free(&p);
  return fail ? OR_ENOMEM : OR_OK;
}

/*
 * Forward of selected rows only.  rows holds nrows pairs (attention head j,
 * slot i).  o_rows: [nrows, dv]; lse_rows: [nrows].
 */
int oracle_attn_fwd_rows(const double *q, const double *k, const double *v, int64_t N, int H,
                         int d, int dv, const int32_t *cu, int S, int paired, int causal,
                         int window, double scale, int64_t nrows, const int64_t *rows,
                         double *o_rows, double *lse_rows) {
  problem p;
  int rc = problem_init(&p, q, k, v, NULL, N, H, d, dv, cu, S, paired, causal, window, scale);
  if (rc) return rc;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[2 * r] < 0 || rows[2 * r] >= p.Hs || rows[2 * r + 1] < 0 || rows[2 * r + 1] >= p.Ns) {
      problem_free(&p);
      return OR_EINVAL;
    }
  const int64_t L = max_doc_len(&p);
  int fail = 0;
#pragma omp parallel
  {
    double *z = (double *)malloc(sizeof(double) * (size_t)L);
    if (!z) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r)
      if (z) fwd_row(&p, (int)rows[2 * r], rows[2 * r + 1], z, o_rows + r * dv, lse_rows + r);
    free(z);
  }
  problem_free(&p);
  return fail ? OR_ENOMEM : OR_OK;
}

/* ---------------------------------------------------------------------- */
/* Backward.                                                               */

/*
 * Row statistics needed by the backward: m_i, l_i (softmax of row i) and
 * D_i = dO_i . O_i with O_i the exact forward output.
 */
static void stats_row(const problem *p, int j, int64_t i, double *z, double *m, double *l,
                      double *D) {
  const int dv = p->dv;
  const int doc = doc_of(p, i);
  const int64_t b = p->cus[doc], e = p->cus[doc + 1];
  score_row(p, j, i, z, m, l);
  const double *gi = p->g + ((int64_t)j * p->Ns + i) * dv;
  double acc = 0.0;
  for (int64_t jj = b; jj < e; ++jj) {
    if (z[jj - b] == -INFINITY) continue;
    const double pij = exp(z[jj - b] - *m) / *l;
    acc += pij * dot(gi, p->v + ((int64_t)j * p->Ns + jj) * dv, dv);
  }
  *D = acc; /* dO_i . O_i = sum_jj P_ij (dO_i . v_jj) */
}

/* dQ_i = scale * sum_jj P_ij (dO_i . v_jj - D_i) k_jj. */
static void dq_row(const problem *p, int j, int64_t i, double *z, double *dq) {
  const int d = p->d, dv = p->dv;
  const int doc = doc_of(p, i);
  const int64_t b = p->cus[doc], e = p->cus[doc + 1];
  double m, l, D;
  stats_row(p, j, i, z, &m, &l, &D);
  const double *gi = p->g + ((int64_t)j * p->Ns + i) * dv;
  for (int c = 0; c < d; ++c) dq[c] = 0.0;
  for (int64_t jj = b; jj < e; ++jj) {
    if (z[jj - b] == -INFINITY) continue;
    const double pij = exp(z[jj - b] - m) / l;
    const double dp = dot(gi, p->v + ((int64_t)j * p->Ns + jj) * dv, dv);
    const double ds = pij * (dp - D);
    const double *kj = p->k + ((int64_t)j * p->Ns + jj) * d;
    for (int c = 0; c < d; ++c) dq[c] += p->scale * ds * kj[c];
  }
}

/*
 * dV_jj = sum_i P_ij dO_i and dK_jj = scale * sum_i P_ij (dO_i . v_jj - D_i) q_i
 * over the query slots i that see key slot jj.  m, l, D hold the row
 * statistics of attention head j, indexed by slot.
 */
static void dkv_col(const problem *p, int j, int64_t jj, const double *m, const double *l,
                    const double *D, double *dk, double *dv) {
  const int d = p->d, w = p->dv;
  const int doc = doc_of(p, jj);
  const int64_t b = p->cus[doc], e = p->cus[doc + 1];
  const double *kj = p->k + ((int64_t)j * p->Ns + jj) * d;
  const double *vj = p->v + ((int64_t)j * p->Ns + jj) * w;
  for (int c = 0; c < d; ++c) dk[c] = 0.0;
  for (int c = 0; c < w; ++c) dv[c] = 0.0;
  for (int64_t i = b; i < e; ++i) {
    if (!visible(p, i, jj, b, e)) continue;
    const double *qi = p->q + ((int64_t)j * p->Ns + i) * d;
    const double *gi = p->g + ((int64_t)j * p->Ns + i) * w;
    const double zz = p->scale * dot(qi, kj, d);
    const double pij = exp(zz - m[i]) / l[i];
    const double ds = pij * (dot(gi, vj, w) - D[i]);
    for (int c = 0; c < w; ++c) dv[c] += pij * gi[c];
    for (int c = 0; c < d; ++c) dk[c] += p->scale * ds * qi[c];
  }
}

/* Statistics for every row of every (head, slot); arrays [Hs][Ns]. */
static int all_stats(const problem *p, double *m, double *l, double *D, const unsigned char *need) {
  const int64_t L = max_doc_len(p);
  int fail = 0;
#pragma omp parallel
  {
    double *z = (double *)malloc(sizeof(double) * (size_t)L);
    if (!z) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(dynamic, 16) collapse(2)
    for (int j = 0; j < p->Hs; ++j)
      for (int64_t i = 0; i < p->Ns; ++i) {
        const int64_t r = (int64_t)j * p->Ns + i;
        if (z && (!need || need[r])) stats_row(p, j, i, z, m + r, l + r, D + r);
      }
    free(z);
  }
  return fail;
}

/*
 * Full backward.  Inputs q, k: [N, H, d] (rotated), v, dout: [N, H, dvd].
 * Outputs dq, dk: [N, H, d], dv: [N, H, dvd], gradients of sum(O * dout) with
 * respect to q, k, v.
 */
int oracle_attn_bwd(const double *q, const double *k, const double *v, const double *dout,
                    int64_t N, int H, int d, int dvd, const int32_t *cu, int S, int paired,
                    int causal, int window, double scale, double *dq, double *dk, double *dv) {
  if (!dout || !dq || !dk || !dv) return OR_EINVAL;
  problem p;
  int rc = problem_init(&p, q, k, v, dout, N, H, d, dvd, cu, S, paired, causal, window, scale);
  if (rc) return rc;
  const size_t rowsn = (size_t)p.Hs * (size_t)p.Ns;
  const size_t elems = rowsn * (size_t)d, velems = rowsn * (size_t)dvd;
  double *m = (double *)malloc(sizeof(double) * (rowsn ? rowsn : 1));
  double *l = (double *)malloc(sizeof(double) * (rowsn ? rowsn : 1));
  double *D = (double *)malloc(sizeof(double) * (rowsn ? rowsn : 1));
  double *dqs = (double *)malloc(sizeof(double) * (elems ? elems : 1));
  double *dks = (double *)malloc(sizeof(double) * (elems ? elems : 1));
  double *dvs = (double *)malloc(sizeof(double) * (velems ? velems : 1));
  int fail = !m || !l || !D || !dqs || !dks || !dvs;
  if (!fail) fail = all_stats(&p, m, l, D, NULL);
  if (!fail) {
    const int64_t L = max_doc_len(&p);
#pragma omp parallel
    {
      double *z = (double *)malloc(sizeof(double) * (size_t)L);
      if (!z) {
#pragma omp atomic write
        fail = 1;
      }
#pragma omp for schedule(dynamic, 16) collapse(2)
      for (int j = 0; j < p.Hs; ++j)
        for (int64_t i = 0; i < p.Ns; ++i)
          if (z) dq_row(&p, j, i, z, dqs + ((int64_t)j * p.Ns + i) * d);
      free(z);
    }
#pragma omp parallel for schedule(dynamic, 16) collapse(2)
    for (int j = 0; j < p.Hs; ++j)
      for (int64_t jj = 0; jj < p.Ns; ++jj) {
        const int64_t base = (int64_t)j * p.Ns;
        dkv_col(&p, j, jj, m + base, l + base, D + base, dks + (base + jj) * d,
                dvs + (base + jj) * dvd);
      }
  }
  if (!fail) {
    scatter(dqs, &p, d, dq);
    scatter(dks, &p, d, dk);
    scatter(dvs, &p, dvd, dv);
  }
  free(m);
  free(l);
  free(D);
  free(dqs);
  free(dks);
  free(dvs);
  problem_free(&p);
  return fail ? OR_ENOMEM : OR_OK;
}

/*
 * Backward at selected points.  q_rows: nq pairs (head j, slot i) -> dq_rows
 * [nq, d]; k_cols: nk pairs (head j, slot jj) -> dk_cols [nk, d], dv_cols
 * [nk, dv].  Row statistics are computed only for rows that see a requested
 * key.
 */
int oracle_attn_bwd_sampled(const double *q, const double *k, const double *v,
                            const double *dout, int64_t N, int H, int d, int dv,
                            const int32_t *cu, int S, int paired, int causal, int window,
                            double scale, int64_t nq, const int64_t *q_rows, double *dq_rows,
                            int64_t nk, const int64_t *k_cols, double *dk_cols,
                            double *dv_cols) {
  if (!dout) return OR_EINVAL;
  problem p;
  int rc = problem_init(&p, q, k, v, dout, N, H, d, dv, cu, S, paired, causal, window, scale);
  if (rc) return rc;
  for (int64_t r = 0; r < nq; ++r)
    if (q_rows[2 * r] < 0 || q_rows[2 * r] >= p.Hs || q_rows[2 * r + 1] < 0 ||
        q_rows[2 * r + 1] >= p.Ns)
      rc = OR_EINVAL;
  for (int64_t r = 0; r < nk; ++r)
    if (k_cols[2 * r] < 0 || k_cols[2 * r] >= p.Hs || k_cols[2 * r + 1] < 0 ||
        k_cols[2 * r + 1] >= p.Ns)
      rc = OR_EINVAL;
  if (rc) {
    problem_free(&p);
    return rc;
  }
  const int64_t L = max_doc_len(&p);
  int fail = 0;
#pragma omp parallel
  {
    double *z = (double *)malloc(sizeof(double) * (size_t)L);
    if (!z) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nq; ++r)
      if (z) dq_row(&p, (int)q_rows[2 * r], q_rows[2 * r + 1], z, dq_rows + r * d);
    free(z);
  }
  if (nk > 0 && !fail) {
    const size_t rowsn = (size_t)p.Hs * (size_t)p.Ns;
    unsigned char *need = (unsigned char *)calloc(rowsn ? rowsn : 1, 1);
    double *m = (double *)malloc(sizeof(double) * (rowsn ? rowsn : 1));
    double *l = (double *)malloc(sizeof(double) * (rowsn ? rowsn : 1));
    double *D = (double *)malloc(sizeof(double) * (rowsn ? rowsn : 1));
    fail = !need || !m || !l || !D;
    if (!fail) {
      for (int64_t r = 0; r < nk; ++r) {
        const int j = (int)k_cols[2 * r];
        const int64_t jj = k_cols[2 * r + 1];
        const int doc = doc_of(&p, jj);
        for (int64_t i = p.cus[doc]; i < p.cus[doc + 1]; ++i)
          if (visible(&p, i, jj, p.cus[doc], p.cus[doc + 1])) need[(int64_t)j * p.Ns + i] = 1;
      }
      fail = all_stats(&p, m, l, D, need);
    }
    if (!fail) {
#pragma omp parallel for schedule(dynamic, 1)
      for (int64_t r = 0; r < nk; ++r) {
        const int j = (int)k_cols[2 * r];
        const int64_t base = (int64_t)j * p.Ns;
        dkv_col(&p, j, k_cols[2 * r + 1], m + base, l + base, D + base, dk_cols + r * d,
                dv_cols + r * dv);
      }
    }
    free(need);
    free(m);
    free(l);
    free(D);
  }
  problem_free(&p);
  return fail ? OR_ENOMEM : OR_OK;
}
