/*
 * apex_oracle.c -- plain, slow, fp64 CPU oracle for rotary position embedding
 * followed by scaled dot-product attention with grouped-query KV sharing,
 * causal masking and sliding-window masking.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load this library. It shares no code, header or table with
 * the GPU library, and the GPU library never calls it.
 *
 * What it computes, and where that is defined (APEX-1 Mathematical Reference):
 *   - RoPE frequencies: theta_i = b^(-2i/d_h), i = 0 .. d_h/2-1
 *     (Part 1, §4.3 "Frequency Formula").
 *   - YaRN (Part 1, §5.3-5.5), scale factor s >= 1 (1 = off): each frequency
 *     is kept, divided by s, or divided by t s + (1 - t) by the regime of its
 *     wavelength, and the attention scores are multiplied by
 *     0.1 ln(s) + 1. beta_fast = 32, beta_slow = 1 (the pages' defaults).
 *   - RoPE rotation: the pair (x_2i, x_2i+1) is rotated by the angle m*theta_i,
 *     x'_2i = x_2i cos - x_2i+1 sin,  x'_2i+1 = x_2i sin + x_2i+1 cos
 *     (Part 1, §4.2 "Core Idea"; the sign and the adjacent pairing are fixed by
 *     the rotate-half definition of §4.4 and the worked example of §4.6).
 *   - Attention(Q,K,V) = softmax(Q K^T / sqrt(d_h)) V  (Part 2, §6.2).
 *   - GQA: G = H_q/H_kv, query head h reads KV head floor(h/G)  (Part 2, §8.2).
 *   - Window mask: key j is visible to query i iff 0 <= i-j < W and j <= i
 *     (Part 2, §10.2). W = 0 means no window. Non-causal: every key visible.
 *   - MLA attention with decoupled RoPE (Part 2, §9.3): q and k rows are
 *     [content (d_h) | rope (d_r)], RoPE rotates only the rope part with the
 *     frequencies of a d_r-dimensional head, v rows have d_h values, and the
 *     scores are scaled by 1 / sqrt(d_h + d_r), the width of the dot product.
 *   - RMSNorm (Part 1, §3.2): y = x / sqrt(mean(x^2) + eps) * gamma over each
 *     row of d features.
 *   - Prefix-bidirectional regime (Part 2, §11.1, picture in §11.3): with a
 *     prefix of P positions, a query i < P sees exactly the keys j < P; the
 *     other queries keep the causal (and window) mask. P = 0: no prefix.
 *
 * Readings taken where the pages leave a step open:
 *   - Prefill row s of Q and K sits at position m0 + s; the mask uses i - j only.
 *   - Decode: the query sits at position m; cache slot j holds position j and
 *     is stored already rotated; when a new key/value is given it occupies
 *     slot m (the new key is rotated at m here, the new value used as is).
 *   - The max subtraction inside the softmax is only for range; it does not
 *     change the mathematical result.
 *   - Inputs are read exactly as the device sees them (fp32, or bf16 bits
 *     widened exactly) and every intermediate is fp64 with no rounding.
 *
 * Build: gcc -O2 -shared -fPIC -pthread apex_oracle.c -lm
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

/* Exact widening of one stored element to double. */
static double load_elem(const void* base, int dtype, int64_t idx) {
  if (dtype == ORACLE_F32) return (double)((const float*)base)[idx];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* YaRN frequency (Part 1, §5.3 regimes, §5.4 interpolation) of one RoPE
 * frequency at scale factor s, with beta_fast = 32 and beta_slow = 1. The
 * regimes are taken in the table's order by the wavelength lambda = 2 pi /
 * theta: lambda < beta_fast keeps theta; lambda > beta_slow * s divides it
 * by s; otherwise theta / (t s + 1 - t) with t = (lambda / beta_slow - 1) /
 * (s - 1) clamped to [0, 1] (the worked example of §5.6 clamps t). */
#define ORACLE_TWO_PI 6.283185307179586476925286766559
double apex_oracle_yarn_theta(double theta, double s) {
  const double beta_fast = 32.0, beta_slow = 1.0;
  if (s == 1.0) return theta;
  const double lambda = ORACLE_TWO_PI / theta;
  if (lambda < beta_fast) return theta;
  if (lambda > beta_slow * s) return theta / s;
  double t = (lambda / beta_slow - 1.0) / (s - 1.0);
  if (t < 0.0) t = 0.0;
  if (t > 1.0) t = 1.0;
  return theta / (t * s + (1.0 - t));
}

/* The YaRN attention temperature: scores are multiplied by 0.1 ln(s) + 1
 * (Part 1, §5.5). */
double apex_oracle_yarn_attn_factor(double s) { return 0.1 * log(s) + 1.0; }

/* theta_i = b^(-2i/d_h)  (Part 1, §4.3), then YaRN at scale s (s = 1: none). */
int apex_oracle_theta(int d_h, double base, double yarn_s, double* theta) {
  if (d_h < 2 || (d_h & 1) || !(base > 0.0) || !(yarn_s >= 1.0) || !theta) return -1;
  for (int i = 0; i < d_h / 2; i++)
    theta[i] = apex_oracle_yarn_theta(pow(base, -2.0 * i / d_h), yarn_s);
  return 0;
}

/* Rotate one row x[0..d_h) at position pos into y (y may equal x)  (Part 1, §4.2). */
void apex_oracle_rope_row(const double* x, double* y, int d_h, int64_t pos, double base,
                          double yarn_s) {
  for (int i = 0; i < d_h / 2; i++) {
    double theta = apex_oracle_yarn_theta(pow(base, -2.0 * i / d_h), yarn_s);
    double angle = (double)pos * theta;
    double c = cos(angle), s = sin(angle);
    double a = x[2 * i], b = x[2 * i + 1];
    y[2 * i] = a * c - b * s;
    y[2 * i + 1] = a * s + b * c;
  }
}

/* Visibility of key j to query i  (Part 2, §10.2; causal = j <= i). */
int apex_oracle_visible(int64_t i, int64_t j, int causal, int64_t W, int64_t P) {
  if (!causal) return 1;
  if (i < P) return j < P;
  if (j > i) return 0;
  if (W > 0 && !(i - j < W)) return 0;
  return 1;
}

/* softmax(q.k_j * scale) over the n listed keys, then the weighted sum of v_j.
 * keys[j], vals[j] point at rows of length d. probs (optional) receives the
 * n weights.  (Part 2, §6.2) */
static void attend(const double* q, const double* const* keys, const double* const* vals,
                   int64_t n, int d, int dv, double scale, double* scores, double* out,
                   double* probs) {
  double mx = -INFINITY;
  for (int64_t j = 0; j < n; j++) {
    double dot = 0.0;
    for (int t = 0; t < d; t++) dot += q[t] * keys[j][t];
    scores[j] = dot * scale;
    if (scores[j] > mx) mx = scores[j];
  }
  double sum = 0.0;
  for (int64_t j = 0; j < n; j++) {
    scores[j] = exp(scores[j] - mx);
    sum += scores[j];
  }
  for (int t = 0; t < dv; t++) out[t] = 0.0;
  for (int64_t j = 0; j < n; j++) {
    double w = scores[j] / sum;
    if (probs) probs[j] = w;
    for (int t = 0; t < dv; t++) out[t] += w * vals[j][t];
  }
}

/* ---- a minimal parallel-for over [0, n) ---- */
typedef void (*range_fn)(void* ctx, int64_t lo, int64_t hi);
typedef struct { range_fn fn; void* ctx; int64_t lo, hi; } range_job;
static void* range_thread(void* p) {
  range_job* j = (range_job*)p;
  j->fn(j->ctx, j->lo, j->hi);
  return NULL;
}
static void parallel_for(int64_t n, int nthreads, range_fn fn, void* ctx) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > n) nthreads = (int)(n > 0 ? n : 1);
  if (nthreads == 1) { fn(ctx, 0, n); return; }
  pthread_t th[256];
  range_job jobs[256];
  for (int t = 0; t < nthreads; t++) {
    jobs[t].fn = fn; jobs[t].ctx = ctx;
    jobs[t].lo = n * t / nthreads; jobs[t].hi = n * (t + 1) / nthreads;
    pthread_create(&th[t], NULL, range_thread, &jobs[t]);
  }
  for (int t = 0; t < nthreads; t++) pthread_join(th[t], NULL);
}

/* ---------------------------- prefill ---------------------------- */
typedef struct {
  const void *q, *k, *v;
  int dtype, S, Hq, Hkv, d, dv, r_off, d_rope, causal, W, apply_rope;
  int64_t P, m0;
  double base, yarn_s;
  int b, kvh;
  double *krot, *vd;          /* [S, d] rotated keys and widened values of the group */
  const int64_t* rows;        /* requested flat rows of this group */
  const int64_t* row_slot;    /* where each requested row goes in out */
  double* out;
  double* probs;              /* optional [nrows, S] */
} prefill_ctx;

static void prefill_prepare_keys(void* p, int64_t lo, int64_t hi) {
  prefill_ctx* c = (prefill_ctx*)p;
  int64_t kv_off = ((int64_t)c->b * c->Hkv + c->kvh) * c->S;
  for (int64_t j = lo; j < hi; j++) {
    double* kr = c->krot + j * c->d;
    double* vr = c->vd + j * c->dv;
    for (int t = 0; t < c->d; t++) kr[t] = load_elem(c->k, c->dtype, (kv_off + j) * c->d + t);
    for (int t = 0; t < c->dv; t++) vr[t] = load_elem(c->v, c->dtype, (kv_off + j) * c->dv + t);
    if (c->apply_rope)
      apex_oracle_rope_row(kr + c->r_off, kr + c->r_off, c->d_rope, c->m0 + j, c->base, c->yarn_s);
  }
}

static void prefill_rows(void* p, int64_t lo, int64_t hi) {
  prefill_ctx* c = (prefill_ctx*)p;
  double* q = (double*)malloc(sizeof(double) * c->d);
  double* scores = (double*)malloc(sizeof(double) * c->S);
  const double** keys = (const double**)malloc(sizeof(double*) * c->S);
  const double** vals = (const double**)malloc(sizeof(double*) * c->S);
  int64_t* idx = (int64_t*)malloc(sizeof(int64_t) * c->S);
  double* pr = (double*)malloc(sizeof(double) * c->S);
  double scale = apex_oracle_yarn_attn_factor(c->yarn_s) / sqrt((double)c->d);
  for (int64_t r = lo; r < hi; r++) {
    int64_t flat = c->rows[r];                 /* (b*Hq + h)*S + i */
    int64_t i = flat % c->S;
    for (int t = 0; t < c->d; t++) q[t] = load_elem(c->q, c->dtype, flat * c->d + t);
    if (c->apply_rope)
      apex_oracle_rope_row(q + c->r_off, q + c->r_off, c->d_rope, c->m0 + i, c->base, c->yarn_s);
    int64_t n = 0;
    for (int64_t j = 0; j < c->S; j++) {
      if (!apex_oracle_visible(i, j, c->causal, c->W, c->P)) continue;
      keys[n] = c->krot + j * c->d;
      vals[n] = c->vd + j * c->dv;
      idx[n] = j;
      n++;
    }
    double* o = c->out + c->row_slot[r] * c->dv;
    attend(q, keys, vals, n, c->d, c->dv, scale, scores, o, c->probs ? pr : NULL);
    if (c->probs) {
      double* prow = c->probs + c->row_slot[r] * c->S;
      for (int64_t j = 0; j < c->S; j++) prow[j] = 0.0;
      for (int64_t t = 0; t < n; t++) prow[idx[t]] = pr[t];
    }
  }
  free(q); free(scores); free(keys); free(vals); free(idx); free(pr);
}

/* Attention output rows of a prefill, general form: q [B,Hq,S,dqk], k
 * [B,Hkv,S,dqk], v [B,Hkv,S,dv] (row-major, fp32 or bf16 bits); RoPE rotates
 * dims [r_off, r_off + d_rope) of q and k with the frequencies of a
 * d_rope-dimensional head; scores scaled by attn_factor(yarn_s) / sqrt(dqk).
 * rows: flat indices (b*Hq+h)*S+i of the rows to compute, or NULL for all
 * rows in order. out: [nrows, dv] doubles. P: prefix length (0: none; needs
 * causal). probs: optional [nrows, S] softmax weights (0 for masked keys).
 * Returns 0, or -1 on invalid arguments. */
static int prefill_general(const void* q, const void* k, const void* v, int dtype,
                           int B, int S, int Hq, int Hkv, int dqk, int dv, int r_off, int d_rope,
                           int causal, int W, int64_t P, int64_t m0, double base, double yarn_s,
                           int apply_rope, int64_t nrows, const int64_t* rows, double* out,
                           double* probs, int nthreads) {
  if (!q || !k || !v || !out || B < 1 || S < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv ||
      dqk < 1 || dv < 1 || d_rope < 2 || (d_rope & 1) || r_off < 0 || r_off + d_rope > dqk ||
      W < 0 || (W > 0 && !causal) || P < 0 || (P > 0 && !causal) ||
      (dtype != 0 && dtype != 1) || (apply_rope && !(base > 0.0)) || !(yarn_s >= 1.0))
    return -1;
  int64_t total = (int64_t)B * Hq * S;
  if (!rows) nrows = total;
  int G = Hq / Hkv;
  int64_t* all = (int64_t*)malloc(sizeof(int64_t) * (nrows > 0 ? nrows : 1));
  int64_t* slot = (int64_t*)malloc(sizeof(int64_t) * (nrows > 0 ? nrows : 1));
  double* krot = (double*)malloc(sizeof(double) * (size_t)S * dqk);
  double* vd = (double*)malloc(sizeof(double) * (size_t)S * dv);
  for (int64_t r = 0; r < nrows; r++) {
    int64_t f = rows ? rows[r] : r;
    if (f < 0 || f >= total) { free(all); free(slot); free(krot); free(vd); return -1; }
  }
  for (int b = 0; b < B; b++) {
    for (int kvh = 0; kvh < Hkv; kvh++) {
      int64_t n = 0;
      for (int64_t r = 0; r < nrows; r++) {
        int64_t f = rows ? rows[r] : r;
        int64_t bh = f / S;
        if (bh / Hq == b && (bh % Hq) / G == kvh) { all[n] = f; slot[n] = r; n++; }
      }
      if (n == 0) continue;
      prefill_ctx c = {q, k, v, dtype, S, Hq, Hkv, dqk, dv, r_off, d_rope, causal, W, apply_rope,
                       P, m0, base, yarn_s, b, kvh, krot, vd, all, slot, out, probs};
      parallel_for(S, nthreads, prefill_prepare_keys, &c);
      parallel_for(n, nthreads, prefill_rows, &c);
    }
  }
  free(all); free(slot); free(krot); free(vd);
  return 0;
}

/* Prefill with q, k, v, out rows of d values and RoPE over the whole row. */
int apex_oracle_prefill(const void* q, const void* k, const void* v, int dtype,
                        int B, int S, int Hq, int Hkv, int d, int causal, int W,
                        int64_t P, int64_t m0, double base, double yarn_s, int apply_rope,
                        int64_t nrows, const int64_t* rows, double* out, double* probs,
                        int nthreads) {
  if (d < 2 || (d & 1)) return -1;
  return prefill_general(q, k, v, dtype, B, S, Hq, Hkv, d, d, 0, d, causal, W, P, m0, base,
                         yarn_s, apply_rope, nrows, rows, out, probs, nthreads);
}

/* MLA prefill with decoupled RoPE (Part 2, §9.3): q and k rows of
 * d_h + d_r values, [content | rope], RoPE on the last d_r; v and out rows of
 * d_h values; scale 1 / sqrt(d_h + d_r). */
int apex_oracle_prefill_mla(const void* q, const void* k, const void* v, int dtype,
                            int B, int S, int Hq, int Hkv, int d_h, int d_r, int causal, int W,
                            int64_t P, int64_t m0, double base, double yarn_s, int apply_rope,
                            int64_t nrows, const int64_t* rows, double* out, double* probs,
                            int nthreads) {
  if (d_h < 1) return -1;
  return prefill_general(q, k, v, dtype, B, S, Hq, Hkv, d_h + d_r, d_h, d_h, d_r, causal, W, P,
                         m0, base, yarn_s, apply_rope, nrows, rows, out, probs, nthreads);
}

/* ----------------------------- decode ----------------------------- */
typedef struct {
  const void *q, *kc, *vc, *kn, *vn;
  int dtype, Sk, Hq, Hkv, d, dv, r_off, d_rope, W, apply_rope;
  int64_t m;
  double base, yarn_s;
  const int64_t* rows;  /* flat b*Hq + h */
  double* out;
} decode_ctx;

static void decode_rows(void* p, int64_t lo, int64_t hi) {
  decode_ctx* c = (decode_ctx*)p;
  int d = c->d, dv = c->dv, G = c->Hq / c->Hkv;
  int64_t n_max = c->m + 1;
  double* q = (double*)malloc(sizeof(double) * d);
  double* kd = (double*)malloc(sizeof(double) * (size_t)n_max * d);
  double* vd = (double*)malloc(sizeof(double) * (size_t)n_max * dv);
  double* scores = (double*)malloc(sizeof(double) * n_max);
  const double** keys = (const double**)malloc(sizeof(double*) * n_max);
  const double** vals = (const double**)malloc(sizeof(double*) * n_max);
  double scale = apex_oracle_yarn_attn_factor(c->yarn_s) / sqrt((double)d);
  for (int64_t r = lo; r < hi; r++) {
    int64_t bh = c->rows ? c->rows[r] : r;
    int64_t b = bh / c->Hq, h = bh % c->Hq, kvh = h / G;
    for (int t = 0; t < d; t++) q[t] = load_elem(c->q, c->dtype, bh * d + t);
    if (c->apply_rope)
      apex_oracle_rope_row(q + c->r_off, q + c->r_off, c->d_rope, c->m, c->base, c->yarn_s);
    int64_t kv_row0 = (b * c->Hkv + kvh) * (int64_t)c->Sk;
    int64_t n = 0;
    for (int64_t j = 0; j <= c->m; j++) {
      if (!apex_oracle_visible(c->m, j, 1, c->W, 0)) continue;
      double* kr = kd + n * d;
      double* vr = vd + n * dv;
      if (j == c->m && c->kn) {
        for (int t = 0; t < d; t++) kr[t] = load_elem(c->kn, c->dtype, (b * c->Hkv + kvh) * d + t);
        if (c->apply_rope)
          apex_oracle_rope_row(kr + c->r_off, kr + c->r_off, c->d_rope, c->m, c->base, c->yarn_s);
      } else {
        for (int t = 0; t < d; t++) kr[t] = load_elem(c->kc, c->dtype, (kv_row0 + j) * d + t);
      }
      if (j == c->m && c->vn) {
        for (int t = 0; t < dv; t++)
          vr[t] = load_elem(c->vn, c->dtype, (b * c->Hkv + kvh) * dv + t);
      } else {
        for (int t = 0; t < dv; t++) vr[t] = load_elem(c->vc, c->dtype, (kv_row0 + j) * dv + t);
      }
      keys[n] = kr;
      vals[n] = vr;
      n++;
    }
    attend(q, keys, vals, n, d, dv, scale, scores, c->out + r * dv, NULL);
  }
  free(q); free(kd); free(vd); free(scores); free(keys); free(vals);
}

/* Decode step, general form: one query per (b, h) at position m against a
 * cache of Sk slots. q [B,Hq,1,dqk]; k_cache [B,Hkv,Sk,dqk], v_cache
 * [B,Hkv,Sk,dv] (slots stored rotated); k_new [B,Hkv,1,dqk], v_new
 * [B,Hkv,1,dv] or NULL (then slot m is read from the cache). RoPE rotates
 * dims [r_off, r_off + d_rope) of q and k_new with the frequencies of a
 * d_rope-dimensional head; scores scaled by attn_factor(yarn_s) / sqrt(dqk).
 * rows: flat b*Hq+h, or NULL for all. out [nrows, dv]. */
static int decode_general(const void* q, const void* k_cache, const void* v_cache,
                          const void* k_new, const void* v_new, int dtype, int B, int Sk, int Hq,
                          int Hkv, int dqk, int dv, int r_off, int d_rope, int W, int64_t m,
                          double base, double yarn_s, int apply_rope, int64_t nrows,
                          const int64_t* rows, double* out, int nthreads) {
  if (!q || !k_cache || !v_cache || !out || B < 1 || Sk < 1 || Hq < 1 || Hkv < 1 ||
      Hq % Hkv || dqk < 1 || dv < 1 || d_rope < 2 || (d_rope & 1) || r_off < 0 ||
      r_off + d_rope > dqk || W < 0 || m < 0 || m >= Sk || (dtype != 0 && dtype != 1) ||
      (apply_rope && !(base > 0.0)) || !(yarn_s >= 1.0))
    return -1;
  int64_t total = (int64_t)B * Hq;
  if (!rows) nrows = total;
  for (int64_t r = 0; r < nrows; r++) {
    int64_t f = rows ? rows[r] : r;
    if (f < 0 || f >= total) return -1;
  }
  decode_ctx c = {q, k_cache, v_cache, k_new, v_new, dtype, Sk, Hq, Hkv, dqk, dv, r_off, d_rope,
                  W, apply_rope, m, base, yarn_s, rows, out};
  parallel_for(nrows, nthreads, decode_rows, &c);
  return 0;
}

/* Decode with q, k and v rows of d values and RoPE over the whole row. */
int apex_oracle_decode(const void* q, const void* k_cache, const void* v_cache,
                       const void* k_new, const void* v_new, int dtype,
                       int B, int Sk, int Hq, int Hkv, int d, int W, int64_t m,
                       double base, double yarn_s, int apply_rope,
                       int64_t nrows, const int64_t* rows, double* out, int nthreads) {
  if (d < 2 || (d & 1)) return -1;
  return decode_general(q, k_cache, v_cache, k_new, v_new, dtype, B, Sk, Hq, Hkv, d, d, 0, d, W,
                        m, base, yarn_s, apply_rope, nrows, rows, out, nthreads);
}

/* MLA decode with decoupled RoPE (Part 2, §9.3): q, k_cache, k_new rows of
 * d_h + d_r values [content | rope], RoPE on the last d_r; v rows and out of
 * d_h values; scale 1 / sqrt(d_h + d_r). */
int apex_oracle_decode_mla(const void* q, const void* k_cache, const void* v_cache,
                           const void* k_new, const void* v_new, int dtype,
                           int B, int Sk, int Hq, int Hkv, int d_h, int d_r, int W, int64_t m,
                           double base, double yarn_s, int apply_rope,
                           int64_t nrows, const int64_t* rows, double* out, int nthreads) {
  if (d_h < 1) return -1;
  return decode_general(q, k_cache, v_cache, k_new, v_new, dtype, B, Sk, Hq, Hkv, d_h + d_r, d_h,
                        d_h, d_r, W, m, base, yarn_s, apply_rope, nrows, rows, out, nthreads);
}

/* ----------------------------- RMSNorm ----------------------------- */
typedef struct {
  const void *x, *gamma;
  int dtype, d;
  double eps;
  double* out;
} rmsnorm_ctx;

static void rmsnorm_rows(void* p, int64_t lo, int64_t hi) {
  rmsnorm_ctx* c = (rmsnorm_ctx*)p;
  for (int64_t r = lo; r < hi; r++) {
    double msq = 0.0;
    for (int t = 0; t < c->d; t++) {
      double v = load_elem(c->x, c->dtype, r * c->d + t);
      msq += v * v;
    }
    msq /= c->d;
    double rms = sqrt(msq + c->eps);
    for (int t = 0; t < c->d; t++)
      c->out[r * c->d + t] =
          load_elem(c->x, c->dtype, r * c->d + t) / rms * load_elem(c->gamma, c->dtype, t);
  }
}

/* RMSNorm of `rows` rows of d features: x [rows, d], gamma [d] (fp32 or bf16
 * bits), out [rows, d] doubles. Returns 0, or -1 on invalid arguments. */
int apex_oracle_rmsnorm(const void* x, const void* gamma, int dtype, int64_t rows, int d,
                        double eps, double* out, int nthreads) {
  if (!x || !gamma || !out || rows < 1 || d < 1 || !(eps >= 0.0) || (dtype != 0 && dtype != 1))
    return -1;
  rmsnorm_ctx c = {x, gamma, dtype, d, eps, out};
  parallel_for(rows, nthreads, rmsnorm_rows, &c);
  return 0;
}
