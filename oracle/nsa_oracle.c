/*
 * fp64 CPU oracle for the VideoNSA attention layer, forward pass.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. It shares no code, header, table or
 * helper with the GPU library; both only read the same seeded inputs.
 *
 * What it computes follows the VideoNSA pages:
 *   - paper summary page, "Method": tokens are split into vision and text sets
 *     by position; vision tokens go through three NSA branches (compression
 *     of 64-token blocks into block keys/values through a learned map,
 *     selection of the top blocks by importance score, a sliding window over
 *     the most recent tokens), mixed by per-head sigmoid gates; text tokens use
 *     standard GQA; outputs go back to their original positions.
 *   - model card, "Model Architecture": the compression branch averages frame
 *     KV blocks; learnable per-head gates weight the branches.
 *   - paper summary, "Key claims" §2.2: token classification by position id.
 * Every step below is written in its plainest form, in double precision, from
 * the exact input values (inputs arrive as float32 arrays; bf16 data is exact
 * in float32). Where the pages leave a step open, the reading taken is stated
 * at the step:
 *   R1  vision queries attend to vision keys only; text queries attend to all
 *       earlier positions (vision and text).
 *   R2  a compressed block becomes visible to vision query t once it is
 *       complete: (b+1)*B <= t+1.
 *   R3  a trailing partial vision block has no compressed token.
 *   R4  the learned map is one d x d linear (no bias) applied to the block mean,
 *       separate maps for keys and values, shared across KV heads.
 *   R5  query head h reads KV head h / G, G = Hq / Hkv.
 *   R6  importance score of a block for KV group g = sum over the group's G
 *       query heads of the normalised compression-attention probability.
 *   R7  top-k ties go to the lower block index.
 *   R8  a query with no visible compressed block gets o_cmp = 0, lse = -inf.
 *   R9  softmax scale 1/sqrt(d) unless the caller gives another.
 *   R10 the window holds exactly w keys, the query included.
 *   R11 gates are independent sigmoids in branch order (cmp, sel, swa).
 *   R12 the query's own block is always selected and counts toward k.
 *   R14 blocks count from the first vision token.
 * The decode entry evaluates the same steps for a query that is the last
 * token of its cache: the L/B complete blocks are its compressed keys, and
 * its own block is the last, partial when B does not divide L.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  int64_t n_tokens;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t block;
  int32_t top_k;
  int32_t window;
  double scale; /* <= 0: 1/sqrt(head_dim) */
} ora_desc;

typedef struct {
  int32_t batch;
  int32_t cache_len;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t block;
  int32_t top_k;
  int32_t window;
  double scale;
} ora_decode_desc;

enum { ORA_OK = 0, ORA_EINVAL = -1, ORA_ENOMEM = -2 };

/* ---------------------------------------------------------------- helpers */

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

static double dot_df(const double *a, const float *b, int n) {
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += a[i] * (double)b[i];
  return s;
}

static double dot_dd(const double *a, const double *b, int n) {
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += a[i] * b[i];
  return s;
}

/* Plain softmax attention of one query over n keys.
 * Keys/values are rows of float arrays: key j is at kv + rows[j]*stride.
 * Writes o[d] and returns log-sum-exp of the scaled logits (-inf if n == 0). */
static double attend_f(const double *qv, int d, double scale, int64_t n,
                       const int64_t *rows, const float *kb, const float *vb,
                       int64_t stride, double *s, double *o) {
  for (int i = 0; i < d; ++i) o[i] = 0.0;
  if (n == 0) return -INFINITY;
  double m = -INFINITY;
  for (int64_t j = 0; j < n; ++j) {
    s[j] = scale * dot_df(qv, kb + rows[j] * stride, d);
    if (s[j] > m) m = s[j];
  }
  double l = 0.0;
  for (int64_t j = 0; j < n; ++j) l += exp(s[j] - m);
  double lse = m + log(l);
  for (int64_t j = 0; j < n; ++j) {
    double p = exp(s[j] - lse);
    const float *vr = vb + rows[j] * stride;
    for (int i = 0; i < d; ++i) o[i] += p * (double)vr[i];
  }
  return lse;
}

/* ------------------------------------------------------ O2: block pooling */

/* Compressed token of each complete block (R3): mean of the block's B rows,
 * then y = W x (R4). x holds n rows of [Hkv, d]; out is [n/B, Hkv, d]. */
static void pool_blocks(int64_t n, int hkv, int d, int B, const float *x,
                        const int64_t *idx, const float *w, double *out) {
  int64_t n_blk = n / B;
#pragma omp parallel for schedule(static)
  for (int64_t bg = 0; bg < n_blk * hkv; ++bg) {
    int64_t b = bg / hkv;
    int g = (int)(bg % hkv);
    double *mean = (double *)calloc((size_t)d, sizeof(double));
    for (int j = 0; j < B; ++j) {
      int64_t r = b * B + j;
      if (idx) r = idx[r];
      const float *xr = x + (r * hkv + g) * (int64_t)d;
      for (int i = 0; i < d; ++i) mean[i] += (double)xr[i];
    }
    for (int i = 0; i < d; ++i) mean[i] /= (double)B;
    double *y = out + (b * hkv + g) * (int64_t)d;
    for (int r = 0; r < d; ++r) {
      double acc = 0.0;
      for (int i = 0; i < d; ++i) acc += (double)w[(int64_t)r * d + i] * mean[i];
      y[r] = acc;
    }
    free(mean);
  }
}

/* ------------------------------------------------ one vision query (O3-O8) */

typedef struct {
  int hq, hkv, G, d, B, k, w;
  double scale;
  const float *kx, *vx; /* key/value rows; vision-local key j lives at row vrow(j) */
  const int64_t *vidx;  /* vision-local index -> row, NULL = identity */
  int64_t kv_stride;    /* floats between consecutive rows of one head: hkv*d */
  const double *kc, *vc; /* compressed keys/values [n_blk, hkv, d] */
  int64_t n_blk;
} vis_ctx;

typedef struct {
  double *s;      /* logits, length >= max keys */
  double *p;      /* per-head compression probabilities [hq, n_blk] */
  double *qv;     /* query vector */
  int64_t *rows;  /* key row list */
  int64_t *cand;  /* candidate blocks */
  double *score;  /* group score of the current group */
  double *o3;     /* per-branch outputs of one head [3, d] */
} scratch_t;

static int64_t vrow(const vis_ctx *c, int64_t j) { return c->vidx ? c->vidx[j] : j; }

/* ranking order of R7: higher score first, then lower block index */
typedef struct { double score; int64_t blk; } ranked_t;
static int ranked_cmp(const void *pa, const void *pb) {
  const ranked_t *a = (const ranked_t *)pa, *b = (const ranked_t *)pb;
  if (a->score > b->score) return -1;
  if (a->score < b->score) return 1;
  return (a->blk < b->blk) ? -1 : (a->blk > b->blk);
}
static int i32_cmp(const void *pa, const void *pb) {
  int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
  return (a > b) - (a < b);
}

/* Evaluates vision query t (vision-local). q is [hq, d] of that token;
 * gates [hq, 3] (may be NULL: outputs without gating are still written).
 * inject: NULL or [hkv, k] block lists replacing the selection step.
 * Outputs (each may be NULL): out [hq,d], lse [hq], sel [hkv,k],
 * ocmp/osel/oswa [hq,d], counts [3], scores [hkv, n_blk]. */
static int vision_query(const vis_ctx *c, scratch_t *w, int64_t t, const float *q,
                        const float *gates, const int32_t *inject, double *out,
                        double *lse, int32_t *sel, double *ocmp, double *osel,
                        double *oswa, int64_t *counts, double *scores) {
  const int d = c->d, B = c->B;
  const int64_t nc = (t + 1) / B; /* R2: complete blocks visible */
  const int64_t cur = t / B;
  int32_t S[1024];
  if (c->k > 1024) return ORA_EINVAL;

  /* O3: compression attention, per head */
  for (int h = 0; h < c->hq; ++h) {
    const int g = h / c->G; /* R5 */
    for (int i = 0; i < d; ++i) w->qv[i] = (double)q[(int64_t)h * d + i];
    double *o = ocmp ? ocmp + (int64_t)h * d : w->o3;
    double *ph = w->p + (int64_t)h * c->n_blk;
    for (int i = 0; i < d; ++i) o[i] = 0.0;
    double l_h = -INFINITY; /* R8 */
    if (nc > 0) {
      double m = -INFINITY;
      for (int64_t b = 0; b < nc; ++b) {
        w->s[b] = c->scale * dot_dd(w->qv, c->kc + (b * c->hkv + g) * (int64_t)d, d);
        if (w->s[b] > m) m = w->s[b];
      }
      double l = 0.0;
      for (int64_t b = 0; b < nc; ++b) l += exp(w->s[b] - m);
      l_h = m + log(l);
      for (int64_t b = 0; b < nc; ++b) {
        ph[b] = exp(w->s[b] - l_h);
        const double *vr = c->vc + (b * c->hkv + g) * (int64_t)d;
        for (int i = 0; i < d; ++i) o[i] += ph[b] * vr[i];
      }
    }
    if (lse) lse[h] = l_h;
    if (out && gates) {
      double gc = sigmoid((double)gates[h * 3 + 0]);
      for (int i = 0; i < d; ++i) out[(int64_t)h * d + i] = gc * o[i];
    }
  }

  /* O4 + O5: group importance score and top-k selection, per KV group */
  int64_t cnt_sel = 0;
  for (int g = 0; g < c->hkv; ++g) {
    for (int64_t b = 0; b < nc; ++b) {
      double sc = 0.0;
      for (int hh = 0; hh < c->G; ++hh) sc += w->p[(int64_t)(g * c->G + hh) * c->n_blk + b];
      w->score[b] = sc; /* R6 */
    }
    if (scores) {
      double *sr = scores + (int64_t)g * c->n_blk;
      for (int64_t b = 0; b < c->n_blk; ++b) sr[b] = (b < nc) ? w->score[b] : -1.0;
    }
    int ns = 0;
    if (inject) {
      for (int i = 0; i < c->k; ++i) {
        int32_t b = inject[g * c->k + i];
        if (b < -1 || b > cur) return ORA_EINVAL;
        if (b >= 0) S[ns++] = b;
      }
    } else {
      /* candidates: visible blocks other than the query's own (R12) */
      ranked_t *rk = (ranked_t *)w->cand;
      int64_t n_cand = 0;
      for (int64_t b = 0; b < nc; ++b)
        if (b != cur) { rk[n_cand].score = w->score[b]; rk[n_cand].blk = b; ++n_cand; }
      qsort(rk, (size_t)n_cand, sizeof(ranked_t), ranked_cmp); /* R7 */
      S[ns++] = (int32_t)cur;
      for (int64_t i = 0; i < n_cand && ns < c->k; ++i) S[ns++] = (int32_t)rk[i].blk;
    }
    qsort(S, (size_t)ns, sizeof(int32_t), i32_cmp);
    if (sel) {
      for (int i = 0; i < c->k; ++i) sel[g * c->k + i] = (i < ns) ? S[i] : -1;
    }

    /* O6 + O7 + O8 for the G query heads of this group */
    int64_t n_rows = 0;
    for (int i = 0; i < ns; ++i) {
      int64_t b0 = (int64_t)S[i] * B;
      int64_t b1 = b0 + B - 1;
      if (b1 > t) b1 = t; /* causal inside the current block */
      for (int64_t j = b0; j <= b1; ++j) w->rows[n_rows++] = vrow(c, j);
    }
    if (g == 0) cnt_sel = n_rows;
    /* with no output requested (a selection-only call) the attention of
     * O6-O8 is skipped; every quantity of O2-O5 above is unchanged */
    if (!out && !osel && !oswa) continue;
    for (int hh = 0; hh < c->G; ++hh) {
      const int h = g * c->G + hh;
      for (int i = 0; i < d; ++i) w->qv[i] = (double)q[(int64_t)h * d + i];
      double *os = osel ? osel + (int64_t)h * d : w->o3 + d;
      attend_f(w->qv, d, c->scale, n_rows, w->rows, c->kx + g * (int64_t)d,
               c->vx + g * (int64_t)d, c->kv_stride, w->s, os);
      if (out && gates) {
        double gs = sigmoid((double)gates[h * 3 + 1]);
        for (int i = 0; i < d; ++i) out[(int64_t)h * d + i] += gs * os[i];
      }
    }
  }

  /* O7: sliding window of exactly w keys ending at the query (R10) */
  int64_t j0 = t - c->w + 1;
  if (j0 < 0) j0 = 0;
  int64_t n_swa = 0;
  for (int64_t j = j0; j <= t; ++j) w->rows[n_swa++] = vrow(c, j);
  for (int h = 0; h < c->hq && (out || oswa); ++h) {
    const int g = h / c->G;
    for (int i = 0; i < d; ++i) w->qv[i] = (double)q[(int64_t)h * d + i];
    double *ow = oswa ? oswa + (int64_t)h * d : w->o3 + 2 * d;
    attend_f(w->qv, d, c->scale, n_swa, w->rows, c->kx + g * (int64_t)d,
             c->vx + g * (int64_t)d, c->kv_stride, w->s, ow);
    if (out && gates) {
      double gw = sigmoid((double)gates[h * 3 + 2]); /* R11 */
      for (int i = 0; i < d; ++i) out[(int64_t)h * d + i] += gw * ow[i];
    }
  }
  if (counts) { counts[0] = nc; counts[1] = cnt_sel; counts[2] = n_swa; }
  return ORA_OK;
}

static int scratch_alloc(scratch_t *w, int64_t max_keys, int hq, int64_t n_blk, int d) {
  int64_t nb = n_blk > 0 ? n_blk : 1;
  w->s = (double *)malloc(sizeof(double) * (size_t)(max_keys + nb + 1));
  w->p = (double *)malloc(sizeof(double) * (size_t)(hq * nb));
  w->qv = (double *)malloc(sizeof(double) * (size_t)d);
  w->rows = (int64_t *)malloc(sizeof(int64_t) * (size_t)(max_keys + 1));
  w->cand = (int64_t *)malloc(sizeof(ranked_t) * (size_t)nb);
  w->score = (double *)malloc(sizeof(double) * (size_t)nb);
  w->o3 = (double *)malloc(sizeof(double) * (size_t)(3 * d));
  return (w->s && w->p && w->qv && w->rows && w->cand && w->score && w->o3) ? ORA_OK : ORA_ENOMEM;
}

static void scratch_free(scratch_t *w) {
  free(w->s); free(w->p); free(w->qv); free(w->rows); free(w->cand); free(w->score); free(w->o3);
}

static int check_heads(int hq, int hkv, int d, int B, int k, int w) {
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0 || d <= 0 || B <= 0 || k < 1 || w < 1) return 0;
  return 1;
}

/* ------------------------------------------------------------ prefill API */

/* Pools complete blocks of n rows x[n, hkv, d] (R3, R4); out [n/B, hkv, d]. */
int ora_cmp_pool(int64_t n, int32_t hkv, int32_t d, int32_t B, const float *x,
                 const float *w, double *out) {
  if (n < 0 || hkv <= 0 || d <= 0 || B <= 0 || !x || !w || !out) return ORA_EINVAL;
  pool_blocks(n, hkv, d, B, x, NULL, w, out);
  return ORA_OK;
}

/* Evaluates the layer at the requested global positions `rows`.
 * Inputs: q [N,hq,d], k/v [N,hkv,d], is_vision [N], wk/wv [d,d] (y = W x),
 * gates [N,hq,3]. inject_sel: NULL or [n_rows,hkv,k] (vision rows only).
 * Outputs (NULL to skip): out [n_rows,hq,d]; lse [n_rows,hq] (text rows NaN);
 * sel [n_rows,hkv,k] (text rows -2); ocmp/osel/oswa [n_rows,hq,d];
 * counts [n_rows,3] (text rows: 0,0,number of keys); scores [n_rows,hkv,n_blk];
 * kcmp/vcmp [n_blk,hkv,d]. */
int ora_prefill(const ora_desc *ds, const float *q, const float *k, const float *v,
                const uint8_t *is_vision, const float *wk, const float *wv,
                const float *gates, const int64_t *rows, int64_t n_rows,
                const int32_t *inject_sel, double *out, double *lse, int32_t *sel,
                double *ocmp, double *osel, double *oswa, int64_t *counts,
                double *scores, double *kcmp, double *vcmp) {
  if (!ds || !q || !k || !v || !is_vision || !wk || !wv || !gates) return ORA_EINVAL;
  const int64_t N = ds->n_tokens;
  const int hq = ds->n_q_heads, hkv = ds->n_kv_heads, d = ds->head_dim, B = ds->block;
  if (N < 0 || !check_heads(hq, hkv, d, B, ds->top_k, ds->window)) return ORA_EINVAL;
  if (n_rows > 0 && !rows) return ORA_EINVAL;
  const double scale = ds->scale > 0 ? ds->scale : 1.0 / sqrt((double)d); /* R9 */

  /* O1: partition by position into vision (V) and text (T) sets */
  int64_t nv = 0;
  for (int64_t i = 0; i < N; ++i) nv += is_vision[i] ? 1 : 0;
  int64_t *vidx = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nv + 1));
  int64_t *vloc = (int64_t *)malloc(sizeof(int64_t) * (size_t)(N + 1));
  if (!vidx || !vloc) { free(vidx); free(vloc); return ORA_ENOMEM; }
  for (int64_t i = 0, t = 0; i < N; ++i) {
    vloc[i] = is_vision[i] ? t : -1;
    if (is_vision[i]) vidx[t++] = i;
  }
  for (int64_t r = 0; r < n_rows; ++r) {
    if (rows[r] < 0 || rows[r] >= N || (inject_sel && vloc[rows[r]] < 0)) {
      free(vidx); free(vloc); return ORA_EINVAL;
    }
  }

  /* O2: compressed keys and values of every complete vision block */
  const int64_t n_blk = nv / B;
  double *kc = (double *)malloc(sizeof(double) * (size_t)(n_blk * hkv * d + 1));
  double *vc = (double *)malloc(sizeof(double) * (size_t)(n_blk * hkv * d + 1));
  if (!kc || !vc) { free(vidx); free(vloc); free(kc); free(vc); return ORA_ENOMEM; }
  pool_blocks(nv, hkv, d, B, k, vidx, wk, kc);
  pool_blocks(nv, hkv, d, B, v, vidx, wv, vc);
  if (kcmp) memcpy(kcmp, kc, sizeof(double) * (size_t)(n_blk * hkv * d));
  if (vcmp) memcpy(vcmp, vc, sizeof(double) * (size_t)(n_blk * hkv * d));

  vis_ctx c = {hq, hkv, hq / hkv, d, B, ds->top_k, ds->window, scale, k, v, vidx,
               (int64_t)hkv * d, kc, vc, n_blk};
  int status = ORA_OK;
  const int64_t max_keys = N + (int64_t)ds->top_k * B + ds->window + 1;

#pragma omp parallel
  {
    scratch_t w;
    int ok = scratch_alloc(&w, max_keys, hq, n_blk, d) == ORA_OK;
    if (!ok) {
#pragma omp atomic write
      status = ORA_ENOMEM;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
      if (!ok) continue;
      const int64_t pos = rows[r];
      const float *qr = q + pos * hq * (int64_t)d;
      const float *gr = gates + pos * hq * 3;
      double *o_r = out ? out + r * hq * (int64_t)d : NULL;
      if (vloc[pos] >= 0) {
        int rc = vision_query(&c, &w, vloc[pos], qr, gr,
                              inject_sel ? inject_sel + r * hkv * (int64_t)ds->top_k : NULL,
                              o_r, lse ? lse + r * hq : NULL,
                              sel ? sel + r * hkv * (int64_t)ds->top_k : NULL,
                              ocmp ? ocmp + r * hq * (int64_t)d : NULL,
                              osel ? osel + r * hq * (int64_t)d : NULL,
                              oswa ? oswa + r * hq * (int64_t)d : NULL,
                              counts ? counts + r * 3 : NULL,
                              scores ? scores + r * hkv * n_blk : NULL);
        if (rc != ORA_OK) {
#pragma omp atomic write
          status = rc;
        }
      } else {
        /* O9: text query, dense causal GQA over every earlier position (R1) */
        int64_t nk = pos + 1;
        for (int64_t j = 0; j < nk; ++j) w.rows[j] = j;
        for (int h = 0; h < hq && o_r; ++h) {
          const int g = h / (hq / hkv);
          for (int i = 0; i < d; ++i) w.qv[i] = (double)qr[(int64_t)h * d + i];
          double tmp_lse = attend_f(w.qv, d, scale, nk, w.rows, k + g * (int64_t)d,
                                    v + g * (int64_t)d, (int64_t)hkv * d, w.s,
                                    o_r ? o_r + (int64_t)h * d : w.o3);
          (void)tmp_lse;
        }
        for (int h = 0; h < hq; ++h) {
          if (lse) lse[r * hq + h] = NAN;
          if (ocmp) for (int i = 0; i < d; ++i) ocmp[(r * hq + h) * (int64_t)d + i] = NAN;
          if (osel) for (int i = 0; i < d; ++i) osel[(r * hq + h) * (int64_t)d + i] = NAN;
          if (oswa) for (int i = 0; i < d; ++i) oswa[(r * hq + h) * (int64_t)d + i] = NAN;
        }
        if (sel) for (int i = 0; i < hkv * ds->top_k; ++i) sel[r * hkv * (int64_t)ds->top_k + i] = -2;
        if (counts) { counts[r * 3 + 0] = 0; counts[r * 3 + 1] = 0; counts[r * 3 + 2] = nk; }
        if (scores) for (int64_t i = 0; i < hkv * n_blk; ++i) scores[r * hkv * n_blk + i] = -1.0;
      }
    }
    if (ok) scratch_free(&w);
  }
  free(vidx); free(vloc); free(kc); free(vc);
  return status;
}

/* ------------------------------------------------------------- decode API */

/* One query per sequence: the last token (position L-1) of a vision cache
 * whose own key/value already sit in slot L-1, so every one of the floor(L/B)
 * complete blocks has a compressed key and is visible (R2), and block
 * (L-1)/B is the query's own (R12): the last complete block when B divides
 * L, else the partial block after them (R3), exactly as for prefill's row
 * L-1. q [Bt,hq,d]; k_cache/v_cache [Bt,L,hkv,d]; k_cmp/v_cmp
 * [Bt,floor(L/B),hkv,d] (given, float32-exact); gates [Bt,hq,3]; inject_sel
 * NULL or [Bt,hkv,k].
 * Outputs: out [Bt,hq,d]; sel, lse, scores, counts may be NULL. */
int ora_decode(const ora_decode_desc *ds, const float *q, const float *k_cache,
               const float *v_cache, const float *k_cmp, const float *v_cmp,
               const float *gates, const int32_t *inject_sel, double *out,
               int32_t *sel, double *lse, double *ocmp, double *osel, double *oswa,
               int64_t *counts, double *scores) {
  if (!ds || !q || !k_cache || !v_cache || !k_cmp || !v_cmp || !gates || !out) return ORA_EINVAL;
  const int hq = ds->n_q_heads, hkv = ds->n_kv_heads, d = ds->head_dim, B = ds->block;
  const int64_t L = ds->cache_len;
  if (ds->batch < 0 || L < 1 || !check_heads(hq, hkv, d, B, ds->top_k, ds->window)) return ORA_EINVAL;
  const double scale = ds->scale > 0 ? ds->scale : 1.0 / sqrt((double)d);
  const int64_t n_blk = L / B;
  int status = ORA_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int bi = 0; bi < ds->batch; ++bi) {
    scratch_t w;
    double *kc = (double *)malloc(sizeof(double) * (size_t)(n_blk * hkv * d));
    double *vc = (double *)malloc(sizeof(double) * (size_t)(n_blk * hkv * d));
    if (!kc || !vc || scratch_alloc(&w, L + (int64_t)ds->top_k * B + ds->window + 1, hq, n_blk, d) != ORA_OK) {
#pragma omp atomic write
      status = ORA_ENOMEM;
      free(kc); free(vc);
      continue;
    }
    const float *kcs = k_cmp + (int64_t)bi * n_blk * hkv * d;
    const float *vcs = v_cmp + (int64_t)bi * n_blk * hkv * d;
    for (int64_t i = 0; i < n_blk * hkv * d; ++i) { kc[i] = (double)kcs[i]; vc[i] = (double)vcs[i]; }
    vis_ctx c = {hq, hkv, hq / hkv, d, B, ds->top_k, ds->window, scale,
                 k_cache + (int64_t)bi * L * hkv * d, v_cache + (int64_t)bi * L * hkv * d,
                 NULL, (int64_t)hkv * d, kc, vc, n_blk};
    int rc = vision_query(&c, &w, L - 1, q + (int64_t)bi * hq * d, gates + (int64_t)bi * hq * 3,
                          inject_sel ? inject_sel + (int64_t)bi * hkv * ds->top_k : NULL,
                          out + (int64_t)bi * hq * d, lse ? lse + (int64_t)bi * hq : NULL,
                          sel ? sel + (int64_t)bi * hkv * ds->top_k : NULL,
                          ocmp ? ocmp + (int64_t)bi * hq * d : NULL,
                          osel ? osel + (int64_t)bi * hq * d : NULL,
                          oswa ? oswa + (int64_t)bi * hq * d : NULL,
                          counts ? counts + (int64_t)bi * 3 : NULL,
                          scores ? scores + (int64_t)bi * hkv * n_blk : NULL);
    if (rc != ORA_OK) {
#pragma omp atomic write
      status = rc;
    }
    scratch_free(&w);
    free(kc); free(vc);
  }
  return status;
}

int ora_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
