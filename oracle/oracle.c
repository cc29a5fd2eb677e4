/*
 * oracle.c -- plain, slow, fp32 CPU reference of the greedy speculative
 * decoding verify transaction.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library.  The product path
 * (libspecv) shares no source, header, table or helper with it.
 *
 * What it computes, and where the pages define it (citations name the page
 * and the part of it; the pages have no numbered sections):
 *   - A dense decoder trunk: RMSNorm, RoPE, GQA causal attention, SwiGLU MLP
 *     and an LM head.  The pegainfer page (DFlash speculative decoding for
 *     Qwen3-4B, performance and graph sections) lists these as the trunk's
 *     dense ops.  Conventions the pages leave open (epsilon, RoPE base and
 *     layout, untied embeddings) come from the model description passed in.
 *   - The verify forward: one forward over the span [last, d1..dK] giving the
 *     trunk argmax at every row (pegainfer page, transaction section, the
 *     verify step).
 *   - accept_greedy: the longest prefix of drafts each equal to the argmax of
 *     the row before it, plus the trunk's own token at the first mismatch, so
 *     a step commits between 1 and K+1 tokens (same section, the accept step).
 *   - The cache advance: with m drafts accepted, rows [last, d1..dm] are the
 *     cached ones, so the cache grows by m+1 (pegainfer page, draft-seed
 *     alignment paragraph).  Rejected rows stay in memory past the length and
 *     are never read (coreai-model-zoo dense n-gram note, the paragraph on
 *     KV-only bundles: rollback is simply not advancing the position).
 *   - The n-gram prompt-lookup proposer (TensorSharp speculative decoding
 *     page, n-gram section; coreai note, adaptive-K section, which drafts only
 *     off a match of two or more tokens), written as a brute-force search.
 *   - Adaptive K: start at 1, add 2 after a fully accepted round, subtract 1
 *     after any rejection, clamp to [1, cap] (coreai note, adaptive-K section).
 *   - Sliding-window layers (TensorSharp page, sliding-window section): a
 *     layer marked local attends, from the row at position t, only the keys
 *     at positions [t - W + 1, t]; the cache stays a plain linear one here,
 *     so rewinding it is exact by definition.
 *   - Recurrent layers (TensorSharp page, recurrent-trunk section: a layer
 *     whose state a dropped tail cannot roll back): a delta rule per kv head
 *     with the state S [d_v][d_k], updated row by row with the normalised key
 *     and value of the row, S <- S + beta (v - S k) k^T, and read by each
 *     normalised query of the head's group, o = S q (no positional rotation).
 *     A verify that rejects drafts restores the state from before the verify
 *     and runs the accepted rows through again -- the slow, plain way the
 *     page describes before per-row snapshots.
 *   - Sampled verification: each row draws its token (Gumbel-max over the
 *     logits divided by the temperature, with Philox4x32-10 noise keyed by the
 *     seed, the sequence and the row's position) and drafts are accepted while
 *     the drawn token matches (TensorSharp page, protocol section).
 *
 * Row invariance: every dot product below is summed in one fixed sequential
 * order over its reduction index, whatever other rows share the call, so a
 * multi-row forward is bit-identical to the same rows decoded one at a time
 * (the rows gate of the coreai note, section on gating the bundle).
 *
 * Build: gcc -O3 -fopenmp -ffp-contract=off (no -ffast-math: no reassociation).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORC_PLANT
#define ORC_PLANT 0 /* >0 plants one deliberate mistake; used only to show the pins have teeth */
#endif

#define ORC_API __attribute__((visibility("default")))

enum { ORC_OK = 0, ORC_EINVAL = -1, ORC_ECAPACITY = -2, ORC_ESTATE = -3, ORC_ENAN = -4, ORC_ENOMEM = -5 };
enum { ORC_FMT_BF16 = 0, ORC_FMT_INT4G128 = 1 };
enum { ORC_WQ = 0, ORC_WK, ORC_WV, ORC_WO, ORC_WG, ORC_WU, ORC_WD, ORC_NW };
enum { ORC_MAT_EMB = 100, ORC_MAT_LM = 101 };
enum { ORC_NORM_ATTN = 0, ORC_NORM_FFN = 1, ORC_NORM_FINAL = 2 };

typedef struct {
  int32_t n_layers, hidden, n_q, n_kv, head_dim, ffn, vocab;
  float eps;
  double rope_theta;
  int32_t swa_window;  /* > 0: the layers in swa_layers attend only the last swa_window positions */
  uint64_t swa_layers; /* bit l: layer l is a sliding-window layer */
  uint64_t rec_layers; /* bit l: layer l is a recurrent (delta-rule) layer instead of attention */
  float rec_beta;      /* the delta rule's write strength */
} orc_shape;

typedef struct {
  int fmt, rows, cols;
  const uint16_t* bf16;   /* [rows][cols] bf16 bit patterns           */
  const uint8_t* q4;      /* [rows][cols/2]: low nibble = even column */
  const uint16_t* scales; /* [rows][cols/128] bf16 bit patterns        */
} orc_mat;

typedef struct orc_model {
  orc_shape s;
  int max_ctx, n_seq;
  orc_mat* lay;           /* [n_layers][ORC_NW] */
  const float** g_attn;   /* [n_layers] -> [hidden] */
  const float** g_ffn;
  const float* g_final;
  orc_mat emb, lm;
  float* kc;              /* [n_seq][n_layers][max_ctx][n_kv*head_dim] */
  float* vc;
  int* len;               /* cache length per sequence */
  float* rs;              /* recurrent states [n_seq][n_layers][n_kv][head_dim (v)][head_dim (k)], or NULL */
} orc_model;

/* ---------------------------------------------------------------- scalars */

static inline float bf16_to_f32(uint16_t b) {
  union { uint32_t u; float f; } v;
  v.u = (uint32_t)b << 16;
  return v.f;
}

/* Weight element W[n][k] as an exact fp32 value.  int4: w = s * q with
 * q in [-8, 7] two's complement and s the bf16 scale of the 128-column group;
 * the product is exact in fp32 (bf16 mantissa times a 4-bit integer). */
static inline float mat_at(const orc_mat* m, int n, int k) {
  if (m->fmt == ORC_FMT_BF16) return bf16_to_f32(m->bf16[(size_t)n * m->cols + k]);
  uint8_t byte = m->q4[(size_t)n * (m->cols / 2) + k / 2];
  int nib = (k & 1) ? (byte >> 4) : (byte & 15);
  int q = nib >= 8 ? nib - 16 : nib;
  float s = bf16_to_f32(m->scales[(size_t)n * (m->cols / 128) + k / 128]);
  return s * (float)q;
}

/* Y[r][n] = sum_k W[n][k] * X[r][k], each sum sequential over k in fp32.
 * X is passed transposed (Xt[k][r]) so the per-k update over r vectorises
 * without changing any single sum's order. */
static void matmul(const orc_mat* W, const float* Xt, int R, float* Y) {
  const int N = W->rows, K = W->cols;
#pragma omp parallel
  {
    float* w = (float*)malloc(sizeof(float) * (size_t)K);
    float* acc = (float*)malloc(sizeof(float) * (size_t)R);
#pragma omp for schedule(static)
    for (int n = 0; n < N; ++n) {
      for (int k = 0; k < K; ++k) w[k] = mat_at(W, n, k);
      for (int r = 0; r < R; ++r) acc[r] = 0.0f;
      for (int k = 0; k < K; ++k) {
        const float wk = w[k];
        const float* xk = Xt + (size_t)k * R;
        for (int r = 0; r < R; ++r) acc[r] = acc[r] + wk * xk[r];
      }
      for (int r = 0; r < R; ++r) Y[(size_t)r * N + n] = acc[r];
    }
    free(w);
    free(acc);
  }
}

static void transpose(const float* X, int R, int C, float* Xt) {
  for (int r = 0; r < R; ++r)
    for (int c = 0; c < C; ++c) Xt[(size_t)c * R + r] = X[(size_t)r * C + c];
}

/* Y[r][n] = sum_k W[n][k] X[r][k] for one matrix in either storage format,
 * X row-major [R][cols]; the same product the forward uses. */
ORC_API int orc_matvec(int fmt, int rows, int cols, const void* data, const void* scales,
                       const float* X, int R, float* Y) {
  if (!data || !X || !Y || rows <= 0 || cols <= 0 || R <= 0) return ORC_EINVAL;
  if (fmt == ORC_FMT_INT4G128 && (cols % 128 || !scales)) return ORC_EINVAL;
  orc_mat w = {fmt, rows, cols, NULL, NULL, NULL};
  if (fmt == ORC_FMT_BF16) w.bf16 = (const uint16_t*)data;
  else if (fmt == ORC_FMT_INT4G128) { w.q4 = (const uint8_t*)data; w.scales = (const uint16_t*)scales; }
  else return ORC_EINVAL;
  float* Xt = (float*)malloc(sizeof(float) * (size_t)R * cols);
  if (!Xt) return ORC_ENOMEM;
  transpose(X, R, cols, Xt);
  matmul(&w, Xt, R, Y);
  free(Xt);
  return ORC_OK;
}

/* RMSNorm: y = x / sqrt(mean(x^2) + eps) * g. */
ORC_API void orc_rmsnorm(const float* x, const float* g, int H, float eps, float* y) {
  float ss = 0.0f;
  for (int i = 0; i < H; ++i) ss = ss + x[i] * x[i];
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
  for (int i = 0; i < H; ++i) {
#if ORC_PLANT == 6
    y[i] = x[i] * r;
#else
    y[i] = (x[i] * r) * g[i];
#endif
  }
}

/* Rotary embedding, rotate-half (NeoX) pairing: element i rotates with
 * element i + d/2 by angle pos * theta^(-2i/d).  cos and sin are evaluated in
 * fp64 and rounded to fp32. */
ORC_API void orc_rope(float* v, int hd, int pos, double theta) {
  const int half = hd / 2;
  for (int i = 0; i < half; ++i) {
    const double inv = pow(theta, -2.0 * (double)i / (double)hd);
    const double ang = (double)pos * inv;
    const float c = (float)cos(ang);
#if ORC_PLANT == 1
    const float s = -(float)sin(ang);
#else
    const float s = (float)sin(ang);
#endif
    const float a = v[i], b = v[i + half];
    v[i] = a * c - b * s;
    v[i + half] = a * s + b * c;
  }
}

/* Causal softmax attention of one query head over cached keys 0..t:
 * s_j = (q . k_j) / sqrt(d), p = softmax(s), o = sum_j p_j v_j.
 * K and V rows are `stride` floats apart (the cache row layout). */
ORC_API void orc_attend(const float* q, const float* K, const float* V, int t, int stride, int hd,
                        float* o, float* scratch /* t+1 floats */) {
#if ORC_PLANT == 3
  const float scale = 1.0f;
#else
  const float scale = (float)(1.0 / sqrt((double)hd));
#endif
  float mx = -INFINITY;
  for (int j = 0; j <= t; ++j) {
    float d = 0.0f;
    const float* kj = K + (size_t)j * stride;
    for (int e = 0; e < hd; ++e) d = d + q[e] * kj[e];
    scratch[j] = d * scale;
    if (scratch[j] > mx) mx = scratch[j];
  }
  float l = 0.0f;
  for (int j = 0; j <= t; ++j) {
    scratch[j] = expf(scratch[j] - mx);
    l = l + scratch[j];
  }
  for (int e = 0; e < hd; ++e) o[e] = 0.0f;
  for (int j = 0; j <= t; ++j) {
    const float* vj = V + (size_t)j * stride;
    for (int e = 0; e < hd; ++e) o[e] = o[e] + scratch[j] * vj[e];
  }
  for (int e = 0; e < hd; ++e) o[e] = o[e] / l;
}

ORC_API float orc_silu(float g) { return g / (1.0f + expf(-g)); }

/* One delta-rule write into the state S [hd (v)][hd (k)]: with k^ = k / |k|,
 * u = S k^ and S <- S + beta (v - u) k^^T; a later read with key k^ then
 * returns u + beta (v - u) (exactly v for beta = 1). */
ORC_API void orc_delta_write(float* S, int hd, const float* k, const float* v, float beta) {
  float kk = 0.0f;
  for (int d = 0; d < hd; ++d) kk = kk + k[d] * k[d];
  const float nrm = sqrtf(kk);
  float kh[512];
#if ORC_PLANT == 16
  for (int d = 0; d < hd; ++d) kh[d] = k[d];
#else
  for (int d = 0; d < hd; ++d) kh[d] = k[d] / nrm;
#endif
  for (int i = 0; i < hd; ++i) {
    float u = 0.0f;
    for (int d = 0; d < hd; ++d) u = u + S[(size_t)i * hd + d] * kh[d];
    const float c = beta * (v[i] - u);
    for (int d = 0; d < hd; ++d) S[(size_t)i * hd + d] = S[(size_t)i * hd + d] + c * kh[d];
  }
}

/* A read of S with the normalised query: o = S (q / |q|). */
ORC_API void orc_delta_read(const float* S, int hd, const float* q, float* o) {
  float qq = 0.0f;
  for (int d = 0; d < hd; ++d) qq = qq + q[d] * q[d];
  const float nrm = sqrtf(qq);
  for (int i = 0; i < hd; ++i) {
    float a = 0.0f;
    for (int d = 0; d < hd; ++d) a = a + S[(size_t)i * hd + d] * (q[d] / nrm);
    o[i] = a;
  }
}

/* Largest value, lowest index on ties; NaN is an error (returns -1). */
ORC_API int orc_argmax(const float* v, int n, float* margin) {
  int best = -1;
  float b1 = -INFINITY, b2 = -INFINITY;
  for (int i = 0; i < n; ++i) {
    const float x = v[i];
    if (x != x) return -1;
#if ORC_PLANT == 10
    if (best < 0 || x >= b1) {
#else
    if (best < 0 || x > b1) {
#endif
      if (best >= 0) b2 = b1;
      b1 = x;
      best = i;
    } else if (x > b2) {
      b2 = x;
    }
  }
  if (margin) *margin = (n > 1) ? b1 - b2 : INFINITY;
  return best;
}

/* ------------------------------------------------------------------ model */

ORC_API orc_model* orc_new(const orc_shape* s, int max_ctx, int n_seq) {
  if (!s || max_ctx <= 0 || n_seq <= 0) return NULL;
  if (s->head_dim % 2 || s->n_q % s->n_kv || s->swa_window < 0) return NULL;
  if (s->rec_layers && (s->head_dim > 512 || !(s->rec_beta > 0.0f))) return NULL;
  orc_model* m = (orc_model*)calloc(1, sizeof(orc_model));
  if (!m) return NULL;
  m->s = *s;
  m->max_ctx = max_ctx;
  m->n_seq = n_seq;
  m->lay = (orc_mat*)calloc((size_t)s->n_layers * ORC_NW, sizeof(orc_mat));
  m->g_attn = (const float**)calloc((size_t)s->n_layers, sizeof(float*));
  m->g_ffn = (const float**)calloc((size_t)s->n_layers, sizeof(float*));
  const size_t kv = (size_t)n_seq * s->n_layers * max_ctx * s->n_kv * s->head_dim;
  m->kc = (float*)calloc(kv, sizeof(float));
  m->vc = (float*)calloc(kv, sizeof(float));
  m->len = (int*)calloc((size_t)n_seq, sizeof(int));
  if (s->rec_layers)
    m->rs = (float*)calloc((size_t)n_seq * s->n_layers * s->n_kv * s->head_dim * s->head_dim, sizeof(float));
  if (!m->lay || !m->g_attn || !m->g_ffn || !m->kc || !m->vc || !m->len || (s->rec_layers && !m->rs)) {
    free(m->lay); free(m->g_attn); free(m->g_ffn); free(m->kc); free(m->vc); free(m->len); free(m->rs); free(m);
    return NULL;
  }
  return m;
}

ORC_API void orc_free(orc_model* m) {
  if (!m) return;
  free(m->lay); free(m->g_attn); free(m->g_ffn); free(m->kc); free(m->vc); free(m->len); free(m->rs);
  free(m);
}

/* Borrow one weight matrix (the caller keeps the arrays alive).  which is
 * ORC_WQ..ORC_WD for a layer matrix, ORC_MAT_EMB or ORC_MAT_LM otherwise. */
ORC_API int orc_set_matrix(orc_model* m, int layer, int which, int fmt, int rows, int cols,
                           const void* data, const void* scales) {
  if (!m || !data) return ORC_EINVAL;
  if (fmt == ORC_FMT_INT4G128 && (cols % 128 || !scales)) return ORC_EINVAL;
  orc_mat w = {fmt, rows, cols, NULL, NULL, NULL};
  if (fmt == ORC_FMT_BF16) w.bf16 = (const uint16_t*)data;
  else if (fmt == ORC_FMT_INT4G128) { w.q4 = (const uint8_t*)data; w.scales = (const uint16_t*)scales; }
  else return ORC_EINVAL;
  if (which == ORC_MAT_EMB) { m->emb = w; return ORC_OK; }
  if (which == ORC_MAT_LM) { m->lm = w; return ORC_OK; }
  if (layer < 0 || layer >= m->s.n_layers || which < 0 || which >= ORC_NW) return ORC_EINVAL;
  m->lay[(size_t)layer * ORC_NW + which] = w;
  return ORC_OK;
}

ORC_API int orc_set_norm(orc_model* m, int layer, int which, const float* g) {
  if (!m || !g) return ORC_EINVAL;
  if (which == ORC_NORM_FINAL) { m->g_final = g; return ORC_OK; }
  if (layer < 0 || layer >= m->s.n_layers) return ORC_EINVAL;
  if (which == ORC_NORM_ATTN) m->g_attn[layer] = g;
  else if (which == ORC_NORM_FFN) m->g_ffn[layer] = g;
  else return ORC_EINVAL;
  return ORC_OK;
}

ORC_API int orc_cache_len(const orc_model* m, int seq) {
  if (!m || seq < 0 || seq >= m->n_seq) return ORC_EINVAL;
  return m->len[seq];
}

/* Rewind only: the cache can be shortened, never lengthened.  A model with
 * recurrent layers keeps no state for earlier lengths: only its current
 * length or 0 (which empties the sequence) is accepted. */
static size_t rec_floats(const orc_model* m) {
  return (size_t)m->s.n_layers * m->s.n_kv * m->s.head_dim * m->s.head_dim;
}

ORC_API int orc_rewind(orc_model* m, int seq, int len) {
  if (!m || seq < 0 || seq >= m->n_seq) return ORC_EINVAL;
  if (len < 0 || len > m->len[seq]) return ORC_ESTATE;
  if (m->rs && len != m->len[seq]) {
    if (len != 0) return ORC_ESTATE;
    memset(m->rs + (size_t)seq * rec_floats(m), 0, sizeof(float) * rec_floats(m));
  }
  m->len[seq] = len;
  return ORC_OK;
}

static float* kv_row(const orc_model* m, float* base, int seq, int layer, int t) {
  const size_t w = (size_t)m->s.n_kv * m->s.head_dim;
  return base + (((size_t)seq * m->s.n_layers + layer) * m->max_ctx + t) * w;
}

/* Forward n rows of sequence `seq` at positions len..len+n-1, writing their
 * K/V rows and advancing the cache length by n.  Logits are produced for rows
 * lm_from..n-1 only (prefill needs only its last row).  argmax/margin/logits
 * outputs are indexed from lm_from. */
ORC_API int orc_forward(orc_model* m, int seq, const int32_t* toks, int n, int lm_from,
                        float* logits_out, int32_t* argmax_out, float* margin_out) {
  if (!m || !toks || n <= 0 || seq < 0 || seq >= m->n_seq) return ORC_EINVAL;
  if (lm_from < 0 || lm_from > n) return ORC_EINVAL;
  const orc_shape* s = &m->s;
  const int H = s->hidden, hd = s->head_dim, nq = s->n_q, nkv = s->n_kv, F = s->ffn, V = s->vocab;
  const int G = nq / nkv, DQ = nq * hd, DK = nkv * hd;
  const int p = m->len[seq];
  if (p + n > m->max_ctx) return ORC_ECAPACITY;
  for (int r = 0; r < n; ++r)
    if (toks[r] < 0 || toks[r] >= V) return ORC_EINVAL;
  float* rs0 = NULL;  /* a failed forward leaves the recurrent state as it was */
  if (m->rs) {
    rs0 = (float*)malloc(sizeof(float) * rec_floats(m));
    if (!rs0) return ORC_ENOMEM;
    memcpy(rs0, m->rs + (size_t)seq * rec_floats(m), sizeof(float) * rec_floats(m));
  }

  const size_t big = (size_t)n * (size_t)(F > DQ ? (F > H ? F : H) : (DQ > H ? DQ : H));
  float* X = (float*)malloc(sizeof(float) * (size_t)n * H);
  float* U = (float*)malloc(sizeof(float) * big);
  float* Ut = (float*)malloc(sizeof(float) * big);
  float* Q = (float*)malloc(sizeof(float) * (size_t)n * DQ);
  float* Kn = (float*)malloc(sizeof(float) * (size_t)n * DK);
  float* Vn = (float*)malloc(sizeof(float) * (size_t)n * DK);
  float* O = (float*)malloc(sizeof(float) * (size_t)n * DQ);
  float* Y = (float*)malloc(sizeof(float) * (size_t)n * H);
  float* Gt = (float*)malloc(sizeof(float) * (size_t)n * F);
  float* Up = (float*)malloc(sizeof(float) * (size_t)n * F);
  if (!X || !U || !Ut || !Q || !Kn || !Vn || !O || !Y || !Gt || !Up) {
    free(X); free(U); free(Ut); free(Q); free(Kn); free(Vn); free(O); free(Y); free(Gt); free(Up);
    return ORC_ENOMEM;
  }
  int rc = ORC_OK;

  for (int r = 0; r < n; ++r)
    for (int i = 0; i < H; ++i) X[(size_t)r * H + i] = mat_at(&m->emb, toks[r], i);

  for (int l = 0; l < s->n_layers; ++l) {
    const orc_mat* W = m->lay + (size_t)l * ORC_NW;
    const int local = s->swa_window > 0 && l < 64 && ((s->swa_layers >> l) & 1u);
    for (int r = 0; r < n; ++r) orc_rmsnorm(X + (size_t)r * H, m->g_attn[l], H, s->eps, U + (size_t)r * H);
    transpose(U, n, H, Ut);
    matmul(&W[ORC_WQ], Ut, n, Q);
    matmul(&W[ORC_WK], Ut, n, Kn);
    matmul(&W[ORC_WV], Ut, n, Vn);
    const int rec = l < 64 && ((s->rec_layers >> l) & 1u);
    if (rec) {
      /* the rows in order through the state of each kv head; no cache rows */
      for (int r = 0; r < n; ++r)
        for (int g = 0; g < nkv; ++g) {
          float* S = m->rs + (((size_t)seq * s->n_layers + l) * nkv + g) * hd * hd;
          orc_delta_write(S, hd, Kn + (size_t)r * DK + g * hd, Vn + (size_t)r * DK + g * hd, s->rec_beta);
          for (int j = 0; j < G; ++j)
            orc_delta_read(S, hd, Q + (size_t)r * DQ + (g * G + j) * hd, O + (size_t)r * DQ + (g * G + j) * hd);
        }
    }
    for (int r = 0; !rec && r < n; ++r) {
#if ORC_PLANT == 11
      const int pos = r;
#else
      const int pos = p + r;
#endif
      for (int h = 0; h < nq; ++h) orc_rope(Q + (size_t)r * DQ + h * hd, hd, pos, s->rope_theta);
      for (int h = 0; h < nkv; ++h) orc_rope(Kn + (size_t)r * DK + h * hd, hd, pos, s->rope_theta);
#if ORC_PLANT == 12
      memcpy(kv_row(m, m->kc, seq, l, p), Kn + (size_t)r * DK, sizeof(float) * DK);
#else
      memcpy(kv_row(m, m->kc, seq, l, p + r), Kn + (size_t)r * DK, sizeof(float) * DK);
#endif
      memcpy(kv_row(m, m->vc, seq, l, p + r), Vn + (size_t)r * DK, sizeof(float) * DK);
    }
    if (!rec)
#pragma omp parallel
    {
      float* scratch = (float*)malloc(sizeof(float) * (size_t)(p + n));
#pragma omp for schedule(static) collapse(2)
      for (int r = 0; r < n; ++r)
        for (int h = 0; h < nq; ++h) {
#if ORC_PLANT == 2
          const int g = h % nkv;
#else
          const int g = h / G;
#endif
          /* keys [lo, p + r]: all earlier positions, or the last W of a
           * sliding-window layer */
          int lo = 0;
          if (local) {
#if ORC_PLANT == 15
            lo = p + r - s->swa_window;
#else
            lo = p + r - s->swa_window + 1;
#endif
            if (lo < 0) lo = 0;
          }
          orc_attend(Q + (size_t)r * DQ + h * hd, kv_row(m, m->kc, seq, l, lo) + g * hd,
                     kv_row(m, m->vc, seq, l, lo) + g * hd, p + r - lo, DK, hd, O + (size_t)r * DQ + h * hd,
                     scratch);
        }
      free(scratch);
    }
    transpose(O, n, DQ, Ut);
    matmul(&W[ORC_WO], Ut, n, Y);
    for (size_t i = 0; i < (size_t)n * H; ++i) {
#if ORC_PLANT == 4
      X[i] = Y[i];
#else
      X[i] = X[i] + Y[i];
#endif
    }
    for (int r = 0; r < n; ++r) orc_rmsnorm(X + (size_t)r * H, m->g_ffn[l], H, s->eps, U + (size_t)r * H);
    transpose(U, n, H, Ut);
    matmul(&W[ORC_WG], Ut, n, Gt);
    matmul(&W[ORC_WU], Ut, n, Up);
    for (size_t i = 0; i < (size_t)n * F; ++i) {
#if ORC_PLANT == 5
      U[i] = orc_silu(Up[i]) * Gt[i];
#else
      U[i] = orc_silu(Gt[i]) * Up[i];
#endif
    }
    transpose(U, n, F, Ut);
    matmul(&W[ORC_WD], Ut, n, Y);
    for (size_t i = 0; i < (size_t)n * H; ++i) X[i] = X[i] + Y[i];
  }

  const int nl = n - lm_from;
  if (nl > 0) {
    for (int r = 0; r < nl; ++r)
      orc_rmsnorm(X + (size_t)(lm_from + r) * H, m->g_final, H, s->eps, U + (size_t)r * H);
    transpose(U, nl, H, Ut);
    float* L = logits_out ? logits_out : (float*)malloc(sizeof(float) * (size_t)nl * V);
    if (!L) rc = ORC_ENOMEM;
    else {
      matmul(&m->lm, Ut, nl, L);
      for (int r = 0; r < nl; ++r) {
        float mg;
        const int a = orc_argmax(L + (size_t)r * V, V, &mg);
        if (a < 0) rc = ORC_ENAN;
        if (argmax_out) argmax_out[r] = a;
        if (margin_out) margin_out[r] = mg;
      }
      if (!logits_out) free(L);
    }
  }
  if (rc == ORC_OK) m->len[seq] = p + n;
  else if (rs0) memcpy(m->rs + (size_t)seq * rec_floats(m), rs0, sizeof(float) * rec_floats(m));
  free(rs0);
  free(X); free(U); free(Ut); free(Q); free(Kn); free(Vn); free(O); free(Y); free(Gt); free(Up);
  return rc;
}

/* After a verify of K+1 rows from length p accepted m drafts: a model with
 * recurrent layers goes back to the state before the verify (rs0) and runs
 * rows 0..m again, so its state is the one after row m; the cache rows they
 * rewrite are the same.  Leaves the length at p + m + 1. */
static int commit_accepted(orc_model* m, int seq, const int32_t* span, int K, int p, int mm, const float* rs0) {
#if ORC_PLANT == 17
  (void)span; (void)K; (void)rs0;
#else
  if (m->rs && mm < K) {
    memcpy(m->rs + (size_t)seq * rec_floats(m), rs0, sizeof(float) * rec_floats(m));
    m->len[seq] = p;
    const int rc = orc_forward(m, seq, span, mm + 1, mm + 1, NULL, NULL, NULL);
    if (rc != ORC_OK) return rc;
  }
#endif
#if ORC_PLANT == 8
  m->len[seq] = p + mm;
#else
  m->len[seq] = p + mm + 1;
#endif
  return ORC_OK;
}

static float* rec_copy(const orc_model* m, int seq) {
  if (!m->rs) return NULL;
  float* c = (float*)malloc(sizeof(float) * rec_floats(m));
  if (c) memcpy(c, m->rs + (size_t)seq * rec_floats(m), sizeof(float) * rec_floats(m));
  return c;
}

/* Prefill: reset the sequence, forward the prompt, return g0 = argmax of the
 * last prompt row.  g0 itself is not cached: it becomes span[0] of the first
 * verify (pegainfer page, draft-seed alignment paragraph). */
ORC_API int orc_prefill(orc_model* m, int seq, const int32_t* toks, int n, int32_t* g0, float* margin) {
  if (!m || seq < 0 || seq >= m->n_seq || n <= 0) return ORC_EINVAL;
  orc_rewind(m, seq, 0);
  return orc_forward(m, seq, toks, n, n - 1, NULL, g0, margin);
}

/* accept_greedy over argmax rows a[0..K] for drafts span[1..K]: the number of
 * leading drafts with span[i] == a[i-1]. */
ORC_API int orc_accept_greedy(const int32_t* span, const int32_t* a, int K) {
  int mm = 0;
#if ORC_PLANT == 7
  while (mm < K && span[mm] == a[mm]) ++mm;
#else
  while (mm < K && span[mm + 1] == a[mm]) ++mm;
#endif
  return mm;
}

/* Verify span = [last, d1..dK] at p = cache length: forward K+1 rows, take
 * the per-row argmax, accept, and leave the cache at p + m + 1. */
ORC_API int orc_verify(orc_model* m, int seq, const int32_t* span, int K, int32_t* argmax_out,
                       int32_t* accept_out, float* logits_out, float* margin_out) {
  if (!m || !span || !argmax_out || !accept_out || K < 0 || seq < 0 || seq >= m->n_seq) return ORC_EINVAL;
  const int p = m->len[seq];
  float* rs0 = rec_copy(m, seq);
  if (m->rs && !rs0) return ORC_ENOMEM;
  int rc = orc_forward(m, seq, span, K + 1, 0, logits_out, argmax_out, margin_out);
  if (rc == ORC_OK) {
    const int mm = orc_accept_greedy(span, argmax_out, K);
    *accept_out = mm;
    rc = commit_accepted(m, seq, span, K, p, mm, rs0);
  }
  free(rs0);
  return rc;
}

/* ------------------------------------------------------- sampled verify */

/* Sampled verification (TensorSharp speculative decoding page, protocol
 * section, the verify step: the sampler draws a token from every row and
 * drafts are accepted while the drawn token matches; the draw of the first
 * mismatching row is the corrected token).  A row draws from softmax(logit/T)
 * by the Gumbel-max rule: the token is argmax_v (logit_v / T + g_v) with
 * g_v = -log(-log u_v) and u_v uniform in (0, 1).  The uniforms come from
 * the counter-based generator Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
 * "Parallel random numbers: as easy as 1, 2, 3", SC 2011) keyed by the seed,
 * with the counter (v / 4, t, seq, 0) for the row at absolute position t of
 * sequence seq and output word v % 4: a position's draw depends on the seed,
 * the sequence and the position only, so a draft-free decode of the same
 * prefix draws exactly the same token. */

/* One Philox4x32-10 block: ten rounds of the two 32x32->64-bit products with
 * multipliers 0xD2511F53 and 0xCD9E8D57, the key bumped by the Weyl
 * constants 0x9E3779B9 and 0xBB67AE85 between rounds. */
ORC_API void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
#if ORC_PLANT == 13
    c0 = hi1 ^ c1 ^ k1;
#else
    c0 = hi1 ^ c1 ^ k0;
#endif
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* A 32-bit word as a uniform in (0, 1): the top 23 bits plus one half, times
 * 2^-23 (exact in fp32, never 0 or 1). */
ORC_API float orc_uniform01(uint32_t x) { return ((float)(x >> 9) + 0.5f) * (1.0f / 8388608.0f); }

/* g = -log(-log u). */
ORC_API float orc_gumbel(float u) { return -logf(-logf(u)); }

ORC_API float orc_gumbel_noise(uint64_t seed, int seq, int t, int v) {
  const uint32_t ctr[4] = {(uint32_t)v >> 2, (uint32_t)t, (uint32_t)seq, 0u};
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  orc_philox4x32_10(ctr, key, out);
  return orc_gumbel(orc_uniform01(out[v & 3]));
}

/* The token drawn from one row of logits at temperature temp > 0 for the
 * row at position t of sequence seq: the largest logit_v / temp + g_v,
 * lowest index on ties; margin = the two largest scores' difference.  -1 on
 * a NaN logit. */
ORC_API int orc_sample_row(const float* logits, int V, float temp, uint64_t seed, int seq, int t, float* margin) {
  int best = -1;
  float b1 = -INFINITY, b2 = -INFINITY;
  for (int v = 0; v < V; ++v) {
    if (logits[v] != logits[v]) return -1;
#if ORC_PLANT == 14
    const float sc = logits[v] * temp + orc_gumbel_noise(seed, seq, t, v);
#else
    const float sc = logits[v] / temp + orc_gumbel_noise(seed, seq, t, v);
#endif
    if (best < 0 || sc > b1) {
      if (best >= 0) b2 = b1;
      b1 = sc;
      best = v;
    } else if (sc > b2) {
      b2 = sc;
    }
  }
  if (margin) *margin = V > 1 ? b1 - b2 : INFINITY;
  return best;
}

/* Sampled verify of span = [last, d1..dK] at p = cache length: forward K+1
 * rows, draw s_i from row i (position p + i), accept while d(i+1) == s_i,
 * leave the cache at p + m + 1.  The committed tokens are s_0..s_m.
 * temp > 0; tokens_out [K+1], margin_out [K+1] (score margins), logits_out
 * [K+1][V] or NULL. */
ORC_API int orc_verify_sampled(orc_model* m, int seq, const int32_t* span, int K, float temp, uint64_t seed,
                               int32_t* tokens_out, int32_t* accept_out, float* logits_out, float* margin_out) {
  if (!m || !span || !tokens_out || !accept_out || K < 0 || seq < 0 || seq >= m->n_seq || !(temp > 0.0f))
    return ORC_EINVAL;
  const int p = m->len[seq], V = m->s.vocab;
  float* L = logits_out ? logits_out : (float*)malloc(sizeof(float) * (size_t)(K + 1) * V);
  if (!L) return ORC_ENOMEM;
  float* rs0 = rec_copy(m, seq);
  int rc = (m->rs && !rs0) ? ORC_ENOMEM : orc_forward(m, seq, span, K + 1, 0, L, NULL, NULL);
  for (int i = 0; rc == ORC_OK && i <= K; ++i) {
    float mg = 0.0f;
    tokens_out[i] = orc_sample_row(L + (size_t)i * V, V, temp, seed, seq, p + i, &mg);
    if (tokens_out[i] < 0) rc = ORC_ENAN;
    if (margin_out) margin_out[i] = mg;
  }
  if (!logits_out) free(L);
  if (rc != ORC_OK) {
    if (rs0 && m->len[seq] != p) memcpy(m->rs + (size_t)seq * rec_floats(m), rs0, sizeof(float) * rec_floats(m));
    m->len[seq] = p;
    free(rs0);
    return rc;
  }
  const int mm = orc_accept_greedy(span, tokens_out, K);  /* the same prefix rule on the drawn tokens */
  *accept_out = mm;
  rc = commit_accepted(m, seq, span, K, p, mm, rs0);
  free(rs0);
  return rc;
}

/* Sampled prefill: the prompt's rows, then g0 drawn from the last row (its
 * position n - 1) at temperature temp. */
ORC_API int orc_prefill_sampled(orc_model* m, int seq, const int32_t* toks, int n, float temp, uint64_t seed,
                                int32_t* g0, float* margin) {
  if (!m || !toks || !g0 || seq < 0 || seq >= m->n_seq || n <= 0 || !(temp > 0.0f)) return ORC_EINVAL;
  float* L = (float*)malloc(sizeof(float) * (size_t)m->s.vocab);
  if (!L) return ORC_ENOMEM;
  orc_rewind(m, seq, 0);
  int rc = orc_forward(m, seq, toks, n, n - 1, L, NULL, NULL);
  if (rc == ORC_OK) {
    *g0 = orc_sample_row(L, m->s.vocab, temp, seed, seq, n - 1, margin);
    if (*g0 < 0) rc = ORC_ENAN;
  }
  free(L);
  return rc;
}

/* ---------------------------------------------------------------- proposer */

/* Brute-force n-gram prompt lookup over history h[0..L-1].  For n from n_max
 * down to n_min, find the latest earlier occurrence of the last n tokens
 * (an occurrence ending at e <= L-2) and propose the tokens that followed it,
 * at most K and only tokens that already exist (up to h[L-1]).  Returns the
 * number of drafts (0 when no order matches). */
ORC_API int orc_ngram_propose(const int32_t* h, int L, int n_min, int n_max, int K, int32_t* drafts) {
  if (!h || L < 0 || n_min < 1 || n_max < n_min || K < 0) return ORC_EINVAL;
  if (K == 0) return 0;
  for (int n = n_max; n >= n_min; --n) {
    if (L < n + 1) continue;
#if ORC_PLANT == 9
    for (int e = L - 1; e >= n - 1; --e) {
#else
    for (int e = L - 2; e >= n - 1; --e) {
#endif
      int ok = 1;
      for (int j = 0; j < n; ++j)
        if (h[e - n + 1 + j] != h[L - n + j]) { ok = 0; break; }
      if (!ok) continue;
      int c = 0;
      for (int i = e + 1; i <= L - 1 && c < K; ++i) drafts[c++] = h[i];
      return c;
    }
  }
  return 0;
}

/* Adaptive draft length after a round with `drafted` drafts of which
 * `accepted` were accepted: full accept -> k+2, any rejection -> k-1,
 * clamped to [1, cap]; a round with no drafts leaves k unchanged. */
ORC_API int orc_adapt_k(int k, int drafted, int accepted, int cap) {
  if (drafted <= 0) return k;
  int next = (accepted >= drafted) ? k + 2 : k - 1;
  if (next < 1) next = 1;
  if (next > cap) next = cap;
  return next;
}

ORC_API int orc_plant(void) { return ORC_PLANT; }
