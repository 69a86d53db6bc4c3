/*
 * CPU oracle for the CSA sparse-attention decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no source, header, table or helper
 * with the HIP library; the two meet only in the seeded inputs.
 *
 * Plain loops in float64, one query token at a time, written to be checked by
 * eye against the pages:
 *   - "Perf: skip redundant CSA scoring and fuse gather unpack" (description,
 *     changes table): a ratio-4 compressed cache scored by the indexer, a causal
 *     Top-K, and a bypass that emits bounded indices when the visible cache fits
 *     within IDX_TOPK;
 *   - "Fix: port the DeepSeek-V4 MoE, hc_pre and prefill fixes to DSpark"
 *     (description): Top-K over a score prefix must hold past width 256, and the
 *     attended row bound is WIN + min(max_visible_cmp, IDX_TOPK);
 *   - "Perf: fuse HCA merge, inverse RoPE, and packing" (description, changes
 *     table): raw-window and compressed softmax streams merged, inverse RoPE on
 *     the output, heads packed into output groups.
 * Where the pages leave a step open, the reading taken is stated at the step.
 *
 * Threads split the token loop only; each token is computed the same way
 * whatever the thread count, so results do not depend on it.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ODT_F32 0
#define ODT_BF16 1

typedef struct {
  int32_t batch, q_per_req, ratio, n_cap, topk, win, w_cap, heads, head_dim,
      rope_dim, idx_heads, idx_dim, out_groups, max_len, dtype;
} oracle_shape_t;

/* Value of element i of an input tensor stored as fp32 or as bf16 bits. */
static double in_val(const void *base, size_t i, int dtype) {
  if (dtype == ODT_F32) return (double)((const float *)base)[i];
  uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Round a double to the nearest bf16 value (ties to even), returned as float.
 * Done directly from the double so there is a single rounding. */
static float round_bf16(double x) {
  if (x == 0.0 || !isfinite(x)) return (float)x;
  int e;
  double f = frexp(x, &e); /* x = f * 2^e, 0.5 <= |f| < 1 */
  double r = nearbyint(ldexp(f, 8)); /* 8 significant bits, ties to even */
  return (float)ldexp(r, e - 8);
}

/* Value of an OCP FP8 E4M3 code (the "e4m3fn" encoding): sign bit, 4
 * exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
 * subnormals m/8 * 2^-6; S.1111.111 is NaN and there are no infinities, so
 * the largest finite value is 1.75 * 2^8 = 448.  Written from that definition,
 * in float64, where every such value is exact. */
static double e4m3_val(uint8_t code) {
  const int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  const double mag = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* Element c of indexer key row j of request b.  With an FP8 key cache
 * (k_idx8 non-NULL) the row is stored as E4M3 codes plus one fp32 scale per
 * row, and its value is scale * decode(code) (the pages pass an indexer key
 * cache together with its scale, "Fix: complete DeepSeek V4 TP CSA decode",
 * description; the encoding and the per-row granularity are a reading of
 * that passage, which names neither).  Otherwise the row is read in the
 * input dtype. */
static double key_val(const oracle_shape_t *sh, const void *k_idx, const uint8_t *k_idx8,
                      const float *k_scale, int32_t b, int32_t j, int32_t c) {
  const size_t row = (size_t)b * sh->n_cap + (size_t)j;
  if (k_idx8) return (double)k_scale[row] * e4m3_val(k_idx8[row * (size_t)sh->idx_dim + c]);
  return in_val(k_idx, row * (size_t)sh->idx_dim + c, sh->dtype);
}

/* Causal visibility: compressed row j summarises raw tokens R*j .. R*j+R-1
 * and is visible to a query at position p once the whole block is at or before
 * p.  Hence the count of visible rows is floor((p+1)/R).  (The pages name only
 * "causal visibility" and max_visible_cmp; this is the plainest reading.) */
int32_t oracle_n_vis(int32_t p, int32_t ratio) {
  if (p < 0) return 0;
  return (p + 1) / ratio;
}

/* ---------------------------------------------------------------- Top-K -- */

typedef struct {
  float score;
  int32_t idx;
} cand_t;

/* Order for selection: higher score first; equal scores (as IEEE values, so
 * -0 == +0) are ordered by lower index first. */
static int cand_cmp(const void *a, const void *b) {
  const cand_t *x = (const cand_t *)a, *y = (const cand_t *)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->idx < y->idx) ? -1 : (x->idx > y->idx);
}

static int int_cmp(const void *a, const void *b) {
  int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
  return (x > y) - (x < y);
}

/* Select among candidates 0..n-1 the k best by (score desc, index asc) using a
 * full sort, then emit the chosen indices in ascending order, padded with -1
 * up to k.  The output order is a reading: the pages speak only of "bounded
 * Top-K indices"; ascending order makes the bypass and the general path agree
 * whenever every visible row fits. */
int32_t oracle_select_row(const float *scores, int32_t n, int32_t k,
                          int32_t *out) {
  if (n < 0 || k < 0) return 1;
  cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)(n > 0 ? n : 1));
  if (!c) return 2;
  for (int32_t j = 0; j < n; ++j) {
    c[j].score = scores[j];
    c[j].idx = j;
  }
  qsort(c, (size_t)n, sizeof(cand_t), cand_cmp);
  int32_t m = n < k ? n : k;
  for (int32_t i = 0; i < m; ++i) out[i] = c[i].idx;
  qsort(out, (size_t)m, sizeof(int32_t), int_cmp);
  for (int32_t i = m; i < k; ++i) out[i] = -1;
  free(c);
  return 0;
}

/* ------------------------------------------------------- per-token steps -- */

/* Indexer score of one token (b,s) against its visible rows:
 *   score[j] = sum_h w[h] * relu(q_idx[h] . k_idx[j])
 * (the sum_h w_h * relu(q_h . k) indexer), all in float64 and rounded once to
 * fp32.  Tokens that bypass (n_vis <= K) are not scored at all. */
static void score_token(const oracle_shape_t *sh, int32_t b, int32_t s,
                        const void *q_idx, const float *w, const void *k_idx,
                        const uint8_t *k_idx8, const float *k_scale,
                        const int32_t *start_pos, float *scores) {
  const int32_t S = sh->q_per_req, Hi = sh->idx_heads, Di = sh->idx_dim;
  const int32_t p = start_pos[b] + s;
  const int32_t n = oracle_n_vis(p, sh->ratio);
  if (n <= sh->topk) return; /* bypass: nothing scored */
  const size_t tok = (size_t)b * S + s;
  float *row = scores + tok * (size_t)sh->n_cap;
  for (int32_t j = 0; j < n; ++j) {
    double acc = 0.0;
    for (int32_t h = 0; h < Hi; ++h) {
      double dot = 0.0;
      const size_t qo = (tok * Hi + h) * (size_t)Di;
      for (int32_t c = 0; c < Di; ++c)
        dot += in_val(q_idx, qo + c, sh->dtype) * key_val(sh, k_idx, k_idx8, k_scale, b, j, c);
      double r = dot > 0.0 ? dot : 0.0;
      acc += (double)w[tok * Hi + h] * r;
    }
    row[j] = (float)acc;
  }
}

/* Top-K of one token: the bypass when every visible row fits (indices
 * 0..n_vis-1 then -1), otherwise the full-sort selection above. */
static void topk_token(const oracle_shape_t *sh, int32_t b, int32_t s,
                       const float *scores, const int32_t *start_pos,
                       int32_t *topk_idx) {
  const int32_t S = sh->q_per_req, K = sh->topk;
  const int32_t p = start_pos[b] + s;
  const int32_t n = oracle_n_vis(p, sh->ratio);
  const size_t tok = (size_t)b * S + s;
  int32_t *out = topk_idx + tok * (size_t)K;
  if (n <= K) {
    for (int32_t i = 0; i < K; ++i) out[i] = i < n ? i : -1;
    return;
  }
  oracle_select_row(scores + tok * (size_t)sh->n_cap, n, K, out);
}

/* One softmax stream over a list of rows: max logit m, sum of exp l and the
 * unnormalised value sum o (length D). An empty list gives l = 0, o = 0. */
typedef struct {
  double m, l;
} stream_t;

static void attend_stream(const oracle_shape_t *sh, const double *qv,
                          const void *kbuf, const void *vbuf,
                          const size_t *rows, int32_t nrows, double scale,
                          double *logit, stream_t *st, double *o) {
  const int32_t D = sh->head_dim;
  for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
  st->m = -INFINITY;
  st->l = 0.0;
  if (nrows == 0) return;
  for (int32_t r = 0; r < nrows; ++r) {
    double dot = 0.0;
    for (int32_t d = 0; d < D; ++d)
      dot += qv[d] * in_val(kbuf, rows[r] * (size_t)D + d, sh->dtype);
    logit[r] = scale * dot;
    if (logit[r] > st->m) st->m = logit[r];
  }
  for (int32_t r = 0; r < nrows; ++r) {
    double e = exp(logit[r] - st->m);
    st->l += e;
    for (int32_t d = 0; d < D; ++d)
      o[d] += e * in_val(vbuf, rows[r] * (size_t)D + d, sh->dtype);
  }
}

/* Two-stream attention of one token, all heads:
 *   window stream: raw positions max(0, p-WIN+1) .. p (the token's own KV is
 *     already written), stored in a ring at slot pos mod W_cap;
 *   compressed stream: every entry of the token's Top-K list in [0, N_cap)
 *     (other entries are padding);
 * then the two softmaxes are merged by their maxima and sums, the RoPE part of
 * the output is turned back by the query position's angle, the value is
 * rounded once to the output type and head h lands in group h / (H/G). */
static void attn_token(const oracle_shape_t *sh, int32_t b, int32_t s,
                       const void *q, const void *k_win, const void *v_win,
                       const void *k_cmp, const void *v_cmp,
                       const int32_t *topk_idx, const int32_t *start_pos,
                       const float *rope_cos, const float *rope_sin,
                       double scale, float *out, size_t *rows_w,
                       size_t *rows_c, double *logit, double *buf) {
  const int32_t S = sh->q_per_req, H = sh->heads, D = sh->head_dim;
  const int32_t K = sh->topk, Dr = sh->rope_dim, G = sh->out_groups;
  const int32_t Hg = H / G;
  const int32_t p = start_pos[b] + s;
  const size_t tok = (size_t)b * S + s;
  const size_t T = (size_t)sh->batch * S;

  int32_t lo = p - sh->win + 1;
  if (lo < 0) lo = 0;
  int32_t nw = 0;
  for (int32_t t = lo; t <= p; ++t)
    rows_w[nw++] = (size_t)b * sh->w_cap + (size_t)(t % sh->w_cap);
  int32_t nc = 0;
  for (int32_t e = 0; e < K; ++e) {
    int32_t j = topk_idx[tok * K + e];
    if (j >= 0 && j < sh->n_cap) rows_c[nc++] = (size_t)b * sh->n_cap + (size_t)j;
  }

  double *qv = buf, *ow = buf + D, *oc = buf + 2 * D, *o = buf + 3 * D;
  for (int32_t h = 0; h < H; ++h) {
    for (int32_t d = 0; d < D; ++d)
      qv[d] = in_val(q, (tok * H + h) * (size_t)D + d, sh->dtype);
    stream_t sw, sc;
    attend_stream(sh, qv, k_win, v_win, rows_w, nw, scale, logit, &sw, ow);
    attend_stream(sh, qv, k_cmp, v_cmp, rows_c, nc, scale, logit, &sc, oc);
    /* merge: an empty stream (l == 0) carries no weight */
    double m = sw.m > sc.m ? sw.m : sc.m;
    double aw = sw.l > 0.0 ? exp(sw.m - m) : 0.0;
    double ac = sc.l > 0.0 ? exp(sc.m - m) : 0.0;
    double l = aw * sw.l + ac * sc.l;
    for (int32_t d = 0; d < D; ++d) o[d] = (aw * ow[d] + ac * oc[d]) / l;
    /* inverse RoPE on the last Dr dims, pairs (2i, 2i+1) of that block:
     * rotate by -theta_i(p), using the caller's fp32 table row p */
    const int32_t r0 = D - Dr;
    for (int32_t i = 0; i < Dr / 2; ++i) {
      double c = rope_cos[(size_t)p * (Dr / 2) + i];
      double sn = rope_sin[(size_t)p * (Dr / 2) + i];
      double x = o[r0 + 2 * i], y = o[r0 + 2 * i + 1];
      o[r0 + 2 * i] = x * c + y * sn;
      o[r0 + 2 * i + 1] = -x * sn + y * c;
    }
    /* round once and pack: out[g][token][(h mod Hg)*D + d] */
    const int32_t g = h / Hg, hl = h % Hg;
    float *dst = out + ((size_t)g * T + tok) * (size_t)Hg * D + (size_t)hl * D;
    for (int32_t d = 0; d < D; ++d)
      dst[d] = sh->dtype == ODT_BF16 ? round_bf16(o[d]) : (float)o[d];
  }
}

/* ------------------------------------------------------------ threading -- */

enum { JOB_SCORE = 1, JOB_TOPK = 2, JOB_ATTN = 4 };

typedef struct {
  const oracle_shape_t *sh;
  int jobs;
  const void *q_idx, *k_idx, *q, *k_win, *v_win, *k_cmp, *v_cmp;
  const uint8_t *k_idx8;
  const float *k_scale;
  const float *w, *rope_cos, *rope_sin;
  const int32_t *start_pos;
  float *scores;
  int32_t *topk_idx;
  float *out;
  double scale;
  int32_t tok_begin, tok_end, nthreads, tid;
  int status;
} job_t;

static void *run_job(void *arg) {
  job_t *jb = (job_t *)arg;
  const oracle_shape_t *sh = jb->sh;
  const int32_t S = sh->q_per_req, D = sh->head_dim;
  const int32_t nrow_max = sh->win + sh->topk;
  size_t *rows_w = (size_t *)malloc(sizeof(size_t) * (size_t)(sh->win + 1));
  size_t *rows_c = (size_t *)malloc(sizeof(size_t) * (size_t)(sh->topk + 1));
  double *logit = (double *)malloc(sizeof(double) * (size_t)(nrow_max + 1));
  double *buf = (double *)malloc(sizeof(double) * (size_t)(4 * D + 4));
  if (!rows_w || !rows_c || !logit || !buf) {
    jb->status = 2;
  } else {
    for (int32_t t = jb->tok_begin + jb->tid; t < jb->tok_end; t += jb->nthreads) {
      int32_t b = t / S, s = t % S;
      if (jb->jobs & JOB_SCORE)
        score_token(sh, b, s, jb->q_idx, jb->w, jb->k_idx, jb->k_idx8, jb->k_scale,
                    jb->start_pos, jb->scores);
      if (jb->jobs & JOB_TOPK)
        topk_token(sh, b, s, jb->scores, jb->start_pos, jb->topk_idx);
      if (jb->jobs & JOB_ATTN)
        attn_token(sh, b, s, jb->q, jb->k_win, jb->v_win, jb->k_cmp, jb->v_cmp,
                   jb->topk_idx, jb->start_pos, jb->rope_cos, jb->rope_sin,
                   jb->scale, jb->out, rows_w, rows_c, logit, buf);
    }
  }
  free(rows_w);
  free(rows_c);
  free(logit);
  free(buf);
  return NULL;
}

static int check_shape(const oracle_shape_t *sh, const int32_t *start_pos,
                       int needs_rows) {
  if (sh->batch < 0 || sh->q_per_req < 0 || sh->ratio < 1 || sh->n_cap < 1 ||
      sh->topk < 1 || sh->win < 1 || sh->heads < 1 || sh->head_dim < 1 ||
      sh->rope_dim < 0 || sh->rope_dim > sh->head_dim || (sh->rope_dim & 1) ||
      sh->out_groups < 1 || sh->heads % sh->out_groups || sh->idx_heads < 1 ||
      sh->idx_dim < 1)
    return 10;
  if (sh->w_cap < sh->win + sh->q_per_req - 1) return 11;
  for (int32_t b = 0; b < sh->batch; ++b) {
    if (start_pos[b] < 0 || start_pos[b] + sh->q_per_req > sh->max_len) return 12;
    if (needs_rows &&
        oracle_n_vis(start_pos[b] + sh->q_per_req - 1, sh->ratio) > sh->n_cap)
      return 13;
  }
  return 0;
}

/* Run any subset of the three steps over tokens [tok_begin, tok_end) with
 * nthreads threads.  With k_idx8 and k_scale non-NULL the indexer keys come
 * from the FP8 cache (key_val above) and k_idx is not read.  Returns 0 on
 * success. */
int32_t oracle_run(const oracle_shape_t *sh, int32_t jobs, int32_t tok_begin,
                   int32_t tok_end, int32_t nthreads, const void *q_idx,
                   const float *w, const void *k_idx, const int32_t *start_pos,
                   float *scores, int32_t *topk_idx, const void *q,
                   const void *k_win, const void *v_win, const void *k_cmp,
                   const void *v_cmp, const float *rope_cos,
                   const float *rope_sin, int32_t rope_rows,
                   float softmax_scale, float *out, const uint8_t *k_idx8,
                   const float *k_scale) {
  int st = check_shape(sh, start_pos, (jobs & (JOB_SCORE | JOB_TOPK)) != 0);
  if (st) return st;
  if ((jobs & JOB_ATTN) && rope_rows < sh->max_len) return 14;
  if (nthreads < 1) nthreads = 1;
  job_t *jb = (job_t *)calloc((size_t)nthreads, sizeof(job_t));
  pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
  if (!jb || !th) {
    free(jb);
    free(th);
    return 2;
  }
  for (int32_t i = 0; i < nthreads; ++i) {
    jb[i] = (job_t){.sh = sh, .jobs = jobs, .q_idx = q_idx, .k_idx = k_idx,
                    .k_idx8 = k_idx8, .k_scale = k_scale,
                    .q = q, .k_win = k_win, .v_win = v_win, .k_cmp = k_cmp,
                    .v_cmp = v_cmp, .w = w, .rope_cos = rope_cos,
                    .rope_sin = rope_sin, .start_pos = start_pos,
                    .scores = scores, .topk_idx = topk_idx, .out = out,
                    .scale = (double)softmax_scale, .tok_begin = tok_begin,
                    .tok_end = tok_end, .nthreads = nthreads, .tid = i};
  }
  int32_t launched = 0;
  for (int32_t i = 1; i < nthreads; ++i) {
    if (pthread_create(&th[i], NULL, run_job, &jb[i]) != 0) break;
    launched = i;
  }
  run_job(&jb[0]);
  for (int32_t i = 1; i <= launched; ++i) pthread_join(th[i], NULL);
  /* a thread that failed to start leaves its tokens undone: run them here */
  for (int32_t i = launched + 1; i < nthreads; ++i) run_job(&jb[i]);
  int32_t rc = 0;
  for (int32_t i = 0; i < nthreads; ++i)
    if (jb[i].status) rc = jb[i].status;
  free(jb);
  free(th);
  return rc;
}

/* ------------------------------------------------ window-cache writeback -- */

/* Writeback of the step's new window entries: the K and V rows of each new
 * token t (rows of k_new / v_new, elem_bytes per element, D elements) are
 * copied to row slot[t] of k_cache / v_cache.  Every entry of the slot mapping
 * is committed whatever the token count ("Perf: parallelize the DSpark TP-4
 * SWA decode hot tasks", description, writeback item, and the review on the
 * same page: a partial last tile must not be dropped).  A slot outside
 * [0, n_slots) marks padding and is skipped.  Rows are copied bit for bit. */
void oracle_swa_writeback(int32_t n_tokens, int32_t D, int32_t elem_bytes, const void *k_new,
                          const void *v_new, const int32_t *slot, void *k_cache,
                          void *v_cache, int64_t n_slots) {
  const size_t row = (size_t)D * (size_t)elem_bytes;
  for (int32_t t = 0; t < n_tokens; ++t) {
    const int64_t dst = slot[t];
    if (dst < 0 || dst >= n_slots) continue;
    memcpy((char *)k_cache + (size_t)dst * row, (const char *)k_new + (size_t)t * row, row);
    memcpy((char *)v_cache + (size_t)dst * row, (const char *)v_new + (size_t)t * row, row);
  }
}

/* Helper for tests: round a double to bf16 exactly as the output step does. */
float oracle_round_bf16(double x) { return round_bf16(x); }

/* Helper for tests: the value of one E4M3 code. */
double oracle_e4m3_value(int32_t code) { return e4m3_val((uint8_t)code); }
