/*
 * CommVQ decode-step attention: plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call this file or the
 * library built from it; only the tests, the smoke check and the benchmark's CPU-baseline leg do.
 * It shares no code, header, table or constant with the HIP library.
 *
 * Sources (the pages this follows; cited by title and section/field):
 *   [ABS]  "1-bit quantization" tag page (aitopics.org): the CommVQ abstract. Additive quantization
 *          of the KV cache, decoded by a plain matrix product with the codebook; RoPE-commutative codebook.
 *   [SUM]  "CommVQ: Commutative Vector Quantization for KV Cache Compression" (atlas.scime.ai
 *          summary), section "Approach": each key/value vector is quantized as a whole with
 *          additive quantization; the key codebook commutes with RoPE so query-codebook products
 *          are precomputed and reused across tokens.
 *   [VER]  pith.science verdict for arXiv 2506.18879, fields pith_extraction.key_machinery
 *          (2x2 blocks [[x,y],[-y,x]] per 2-D subspace commute with the block-diagonal RoPE
 *          rotation; consecutive sub-vectors share one index; R residual rounds),
 *          pith_extraction.forward_implications (softmax weights multiply the value codes before
 *          the codebook multiply), referee_report.minor_comments (paper Sec. 4.1/4.2, Eq. 18).
 *
 * Every function is the plain definition, in fp64, with straight loops. Readings of points the
 * pages leave open (all listed in the design notes):
 *   - layout: head_dim D, G groups of W = D/G dims; a group holds W/2 RoPE pairs; pair j covers
 *     dims (2j, 2j+1); codes are bytes laid out [Hkv][R][T][G] (one plane of 16-byte token records per residual
 *     codebook); a codebook is [Hkv][G][R][N][W].
 *   - a key codeword stores per pair the two numbers (a, b) of the block [[a,-b],[b,a]]; the
 *     decoded sub-vector is that block applied to e1, i.e. (a, b). [[x,y],[-y,x]] on [VER] is the
 *     same family with b = -y.
 *   - RoPE pairs adjacent dims, theta_j = base^(-2j/D), key at 0-based position t is rotated by
 *     t*theta_j; q is given already rotated; q head h reads kv head h / (Hq/Hkv).
 *   - softmax runs over exactly the L_b cached tokens of sequence b, no mask.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int32_t batch, n_q_heads, n_kv_heads, head_dim;
  int32_t n_groups, n_residuals, n_codes;
  double rope_base, softmax_scale;
} oracle_dims;

/* index of code byte (kv, token, residual, group) in a [Hkv][R][T][G] byte array */
static inline int64_t code_off(const oracle_dims* d, int64_t total_tokens, int kv, int64_t t, int r, int g) {
  return (((int64_t)kv * d->n_residuals + r) * total_tokens + t) * d->n_groups + g;
}

/* offset of codeword (kv, g, r, l) in a [Hkv][G][R][N][W] codebook */
static inline int64_t cw_off(const oracle_dims* d, int kv, int g, int r, int l) {
  int W = d->head_dim / d->n_groups;
  return ((((int64_t)kv * d->n_groups + g) * d->n_residuals + r) * d->n_codes + l) * W;
}

/* Unpack: one byte per index (N = 256, 8 bits per index). out is int32 [Hkv][R][T][G]. */
void oracle_unpack(const oracle_dims* d, const uint8_t* codes, int64_t total_tokens, int32_t* out) {
  for (int kv = 0; kv < d->n_kv_heads; ++kv)
    for (int64_t t = 0; t < total_tokens; ++t)
      for (int r = 0; r < d->n_residuals; ++r)
        for (int g = 0; g < d->n_groups; ++g) {
          int64_t o = code_off(d, total_tokens, kv, t, r, g);
          out[o] = (int32_t)codes[o];
        }
}

/* Additive decode [ABS], [SUM] Approach: x_hat = sum over residual codebooks r of the selected
 * codeword, group by group. codebook [Hkv][G][R][N][W]; out [Hkv][T][D]. */
void oracle_decode(const oracle_dims* d, const double* codebook, const uint8_t* codes, int64_t total_tokens,
                   double* out) {
  int D = d->head_dim, W = D / d->n_groups;
  for (int kv = 0; kv < d->n_kv_heads; ++kv)
    for (int64_t t = 0; t < total_tokens; ++t) {
      double* x = out + ((int64_t)kv * total_tokens + t) * D;
      for (int i = 0; i < D; ++i) x[i] = 0.0;
      for (int g = 0; g < d->n_groups; ++g)
        for (int r = 0; r < d->n_residuals; ++r) {
          int l = codes[code_off(d, total_tokens, kv, t, r, g)];
          const double* c = codebook + cw_off(d, kv, g, r, l);
          for (int w = 0; w < W; ++w) x[g * W + w] += c[w];
        }
    }
}

/* RoPE frequency of pair j: theta_j = base^(-2j/D). */
static double rope_theta(const oracle_dims* d, int j) {
  return pow(d->rope_base, -2.0 * (double)j / (double)d->head_dim);
}

/* RoPE [VER] key_machinery: block-diagonal rotation of each 2-D sub-vector (2j, 2j+1) by angle
 * pos * theta_j. x and out are [n][D]; pos[i] is the 0-based position of row i. */
void oracle_rope(const oracle_dims* d, const double* x, const int64_t* pos, int64_t n, double* out) {
  int D = d->head_dim;
  for (int64_t i = 0; i < n; ++i)
    for (int j = 0; j < D / 2; ++j) {
      double phi = (double)pos[i] * rope_theta(d, j);
      double c = cos(phi), s = sin(phi);
      double x0 = x[i * D + 2 * j], x1 = x[i * D + 2 * j + 1];
      out[i * D + 2 * j] = x0 * c - x1 * s;
      out[i * D + 2 * j + 1] = x0 * s + x1 * c;
    }
}

/* The 2x2 matrix form of a key codeword pair (a, b): [[a, -b], [b, a]] (row-major, 4 doubles), and
 * the RoPE rotation by angle phi: [[cos, -sin], [sin, cos]]. Exposed so the commutation identity
 * R C == C R of [VER] key_machinery can be checked on the oracle's own representation. */
void oracle_key_block(double a, double b, double* m4) {
  m4[0] = a; m4[1] = -b; m4[2] = b; m4[3] = a;
}
void oracle_rotation(double phi, double* m4) {
  m4[0] = cos(phi); m4[1] = -sin(phi); m4[2] = sin(phi); m4[3] = cos(phi);
}

/* ---------------------------------------------------------------------------------------------
 * Full decode-step attention, the plain definition: for every cached token decode the key, rotate
 * it to its position, dot with q, softmax over the L_b tokens, then sum the decoded values weighted
 * by the softmax. q [B][Hq][D] (post-RoPE), out [B][Hq][D]. scores_out / p_out, when non-NULL, are
 * [B][Hq][max_len] and receive the scaled scores and the softmax weights (zero past L_b).
 * ------------------------------------------------------------------------------------------- */
typedef struct {
  const oracle_dims* d;
  const double *q, *k_cb, *v_cb;
  const uint8_t *k_codes, *v_codes;
  const int64_t* seq_start;
  const int32_t* seq_len;
  int64_t total_tokens;
  int32_t max_len;
  double *out, *scores_out, *p_out;
  int next_item;
  pthread_mutex_t lock;
} attn_job;

static void attn_item(attn_job* J, int b, int kv) {
  const oracle_dims* d = J->d;
  int D = d->head_dim, W = D / d->n_groups, P = D / 2;
  int gq = d->n_q_heads / d->n_kv_heads;
  int64_t L = J->seq_len[b], t0 = J->seq_start[b];
  double* kh = (double*)malloc(sizeof(double) * D);
  double* kr = (double*)malloc(sizeof(double) * D);
  double* vh = (double*)malloc(sizeof(double) * D);
  double* s = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1) * gq);
  double* theta = (double*)malloc(sizeof(double) * P);
  for (int j = 0; j < P; ++j) theta[j] = rope_theta(d, j);
  for (int64_t t = 0; t < L; ++t) {
    /* decode key: sum of R codewords per group */
    for (int i = 0; i < D; ++i) kh[i] = 0.0;
    for (int g = 0; g < d->n_groups; ++g)
      for (int r = 0; r < d->n_residuals; ++r) {
        int l = J->k_codes[code_off(d, J->total_tokens, kv, t0 + t, r, g)];
        const double* c = J->k_cb + cw_off(d, kv, g, r, l);
        for (int w = 0; w < W; ++w) kh[g * W + w] += c[w];
      }
    /* rotate pair j by t * theta_j */
    for (int j = 0; j < P; ++j) {
      double phi = (double)t * theta[j], c = cos(phi), sn = sin(phi);
      kr[2 * j] = kh[2 * j] * c - kh[2 * j + 1] * sn;
      kr[2 * j + 1] = kh[2 * j] * sn + kh[2 * j + 1] * c;
    }
    for (int hh = 0; hh < gq; ++hh) {
      const double* qv = J->q + ((int64_t)b * d->n_q_heads + kv * gq + hh) * D;
      double acc = 0.0;
      for (int i = 0; i < D; ++i) acc += qv[i] * kr[i];
      s[hh * L + t] = acc * d->softmax_scale;
    }
  }
  for (int hh = 0; hh < gq; ++hh) {
    int h = kv * gq + hh;
    double* o = J->out + ((int64_t)b * d->n_q_heads + h) * D;
    for (int i = 0; i < D; ++i) o[i] = 0.0;
    double* sp = s + (int64_t)hh * L;
    if (J->scores_out) {
      double* so = J->scores_out + ((int64_t)b * d->n_q_heads + h) * J->max_len;
      for (int64_t t = 0; t < J->max_len; ++t) so[t] = t < L ? sp[t] : 0.0;
    }
    if (L == 0) {
      if (J->p_out) memset(J->p_out + ((int64_t)b * d->n_q_heads + h) * J->max_len, 0, sizeof(double) * J->max_len);
      continue;
    }
    double m = sp[0];
    for (int64_t t = 1; t < L; ++t) if (sp[t] > m) m = sp[t];
    double z = 0.0;
    for (int64_t t = 0; t < L; ++t) { sp[t] = exp(sp[t] - m); z += sp[t]; }
    for (int64_t t = 0; t < L; ++t) sp[t] /= z;
    if (J->p_out) {
      double* po = J->p_out + ((int64_t)b * d->n_q_heads + h) * J->max_len;
      for (int64_t t = 0; t < J->max_len; ++t) po[t] = t < L ? sp[t] : 0.0;
    }
  }
  /* values: o_h = sum_t p_{h,t} * v_hat_t with v_hat_t decoded explicitly */
  for (int64_t t = 0; t < L; ++t) {
    for (int i = 0; i < D; ++i) vh[i] = 0.0;
    for (int g = 0; g < d->n_groups; ++g)
      for (int r = 0; r < d->n_residuals; ++r) {
        int l = J->v_codes[code_off(d, J->total_tokens, kv, t0 + t, r, g)];
        const double* c = J->v_cb + cw_off(d, kv, g, r, l);
        for (int w = 0; w < W; ++w) vh[g * W + w] += c[w];
      }
    for (int hh = 0; hh < gq; ++hh) {
      double* o = J->out + ((int64_t)b * d->n_q_heads + kv * gq + hh) * D;
      double pt = s[hh * L + t];
      for (int i = 0; i < D; ++i) o[i] += pt * vh[i];
    }
  }
  free(kh); free(kr); free(vh); free(s); free(theta);
}

static void* attn_worker(void* arg) {
  attn_job* J = (attn_job*)arg;
  int n_items = J->d->batch * J->d->n_kv_heads;
  for (;;) {
    pthread_mutex_lock(&J->lock);
    int it = J->next_item++;
    pthread_mutex_unlock(&J->lock);
    if (it >= n_items) break;
    attn_item(J, it / J->d->n_kv_heads, it % J->d->n_kv_heads);
  }
  return NULL;
}

/* k_codes/v_codes [Hkv][R][total_tokens][G]; k_cb/v_cb [Hkv][G][R][N][W]; sequence b occupies token
 * rows seq_start[b] .. seq_start[b]+seq_len[b]-1 of every kv head. Runs (b, kv) items on n_threads
 * threads. */
void oracle_attn_decode(const oracle_dims* d, const double* q, const uint8_t* k_codes, const uint8_t* v_codes,
                        const double* k_cb, const double* v_cb, const int64_t* seq_start, const int32_t* seq_len,
                        int64_t total_tokens, int32_t max_len, double* out, double* scores_out, double* p_out,
                        int n_threads) {
  attn_job J;
  J.d = d; J.q = q; J.k_cb = k_cb; J.v_cb = v_cb; J.k_codes = k_codes; J.v_codes = v_codes;
  J.seq_start = seq_start; J.seq_len = seq_len; J.total_tokens = total_tokens; J.max_len = max_len;
  J.out = out; J.scores_out = scores_out; J.p_out = p_out; J.next_item = 0;
  pthread_mutex_init(&J.lock, NULL);
  if (n_threads < 1) n_threads = 1;
  if (n_threads == 1) {
    attn_worker(&J);
  } else {
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * n_threads);
    for (int i = 0; i < n_threads; ++i) pthread_create(&th[i], NULL, attn_worker, &J);
    for (int i = 0; i < n_threads; ++i) pthread_join(th[i], NULL);
    free(th);
  }
  pthread_mutex_destroy(&J.lock);
}

/* Query x codebook table [SUM] Approach, [VER] key_machinery ("computed once and reused across all
 * cached positions"): for q head h (kv = h/(Hq/Hkv)), group g, residual r, code l and pair u of the
 * group (global pair j = g*W/2 + u), T = conj(q_j) * c with q_j = q[2j] + i q[2j+1] and
 * c = a + i b the codeword pair:  T.re = q[2j] a + q[2j+1] b,  T.im = q[2j] b - q[2j+1] a.
 * out [B][Hq][G][R][N][W] with (re, im) interleaved per pair. */
void oracle_table(const oracle_dims* d, const double* q, const double* k_cb, double* out) {
  int D = d->head_dim, W = D / d->n_groups, gq = d->n_q_heads / d->n_kv_heads;
  for (int b = 0; b < d->batch; ++b)
    for (int h = 0; h < d->n_q_heads; ++h) {
      const double* qv = q + ((int64_t)b * d->n_q_heads + h) * D;
      int kv = h / gq;
      for (int g = 0; g < d->n_groups; ++g)
        for (int r = 0; r < d->n_residuals; ++r)
          for (int l = 0; l < d->n_codes; ++l) {
            const double* c = k_cb + cw_off(d, kv, g, r, l);
            double* t = out + (((((int64_t)b * d->n_q_heads + h) * d->n_groups + g) * d->n_residuals + r) *
                                   d->n_codes + l) * W;
            for (int u = 0; u < W / 2; ++u) {
              int j = g * (W / 2) + u;
              double q0 = qv[2 * j], q1 = qv[2 * j + 1], a = c[2 * u], bb = c[2 * u + 1];
              t[2 * u] = q0 * a + q1 * bb;
              t[2 * u + 1] = q0 * bb - q1 * a;
            }
          }
    }
}

/* Scores through the table (the reordered form of [VER] key_machinery): for token t of sequence b
 * and q head h,  s = scale * sum_j Re( (sum_r T[g][r][i_{t,g,r}][u]) * e^{i t theta_j} ).
 * table from oracle_table; scores_out [B][Hq][max_len] (zero past L_b). */
void oracle_scores_via_table(const oracle_dims* d, const double* table, const uint8_t* k_codes,
                             const int64_t* seq_start, const int32_t* seq_len, int64_t total_tokens,
                             int32_t max_len, double* scores_out) {
  int D = d->head_dim, W = D / d->n_groups, gq = d->n_q_heads / d->n_kv_heads;
  for (int b = 0; b < d->batch; ++b)
    for (int h = 0; h < d->n_q_heads; ++h) {
      int kv = h / gq;
      double* so = scores_out + ((int64_t)b * d->n_q_heads + h) * max_len;
      for (int64_t t = 0; t < max_len; ++t) {
        if (t >= seq_len[b]) { so[t] = 0.0; continue; }
        double acc = 0.0;
        for (int g = 0; g < d->n_groups; ++g)
          for (int u = 0; u < W / 2; ++u) {
            double xr = 0.0, xi = 0.0;
            for (int r = 0; r < d->n_residuals; ++r) {
              int l = k_codes[code_off(d, total_tokens, kv, seq_start[b] + t, r, g)];
              const double* tt = table + (((((int64_t)b * d->n_q_heads + h) * d->n_groups + g) * d->n_residuals + r) *
                                              d->n_codes + l) * W;
              xr += tt[2 * u];
              xi += tt[2 * u + 1];
            }
            int j = g * (W / 2) + u;
            double phi = (double)t * rope_theta(d, j);
            acc += xr * cos(phi) - xi * sin(phi);
          }
        so[t] = acc * d->softmax_scale;
      }
    }
}

/* Value reduce through bins ([VER] forward_implications: the softmax weights multiply the value
 * codes before the codebook multiply): for every (b, h), bins[g][r][l] = sum_t p[t] [i_{t,g,r} = l],
 * then out[g*W + w] = sum_r sum_l bins[g][r][l] * CV[kv][g][r][l][w]. p [B][Hq][max_len] is used as
 * given (no renormalisation); out [B][Hq][D]. */
void oracle_value_reduce(const oracle_dims* d, const double* p, const uint8_t* v_codes, const double* v_cb,
                         const int64_t* seq_start, const int32_t* seq_len, int64_t total_tokens, int32_t max_len,
                         double* out) {
  int D = d->head_dim, W = D / d->n_groups, gq = d->n_q_heads / d->n_kv_heads;
  int G = d->n_groups, R = d->n_residuals, N = d->n_codes;
  double* bins = (double*)malloc(sizeof(double) * (size_t)G * R * N);
  for (int b = 0; b < d->batch; ++b)
    for (int h = 0; h < d->n_q_heads; ++h) {
      int kv = h / gq;
      const double* pp = p + ((int64_t)b * d->n_q_heads + h) * max_len;
      for (int64_t i = 0; i < (int64_t)G * R * N; ++i) bins[i] = 0.0;
      for (int64_t t = 0; t < seq_len[b]; ++t)
        for (int g = 0; g < G; ++g)
          for (int r = 0; r < R; ++r) {
            int l = v_codes[code_off(d, total_tokens, kv, seq_start[b] + t, r, g)];
            bins[((int64_t)g * R + r) * N + l] += pp[t];
          }
      double* o = out + ((int64_t)b * d->n_q_heads + h) * D;
      for (int g = 0; g < G; ++g)
        for (int w = 0; w < W; ++w) {
          double acc = 0.0;
          for (int r = 0; r < R; ++r)
            for (int l = 0; l < N; ++l) acc += bins[((int64_t)g * R + r) * N + l] * v_cb[cw_off(d, kv, g, r, l) + w];
          o[g * W + w] = acc;
        }
    }
  free(bins);
}

/* Greedy residual encoder, a stand-in for the pages' learned encoder ([ABS]: "lightweight encoder"):
 * for each (kv, token, group), residual rounds r = 0..R-1 pick l* = argmin_l ||res - C[g][r][l]||^2
 * (ties to the lowest l) and subtract the chosen codeword ([VER] key_machinery: R residual rounds
 * refine the reconstruction). x [Hkv][T][D] (in the codebook's own frame, i.e. before RoPE);
 * codes_out [Hkv][R][T][G]; dist_out (optional) [Hkv][R][T][G] holds the minimum squared distance
 * of each round. */
void oracle_encode_greedy(const oracle_dims* d, const double* x, const double* codebook, int64_t n_tokens,
                          uint8_t* codes_out, double* dist_out) {
  int D = d->head_dim, G = d->n_groups, W = D / G, R = d->n_residuals, N = d->n_codes;
  double* res = (double*)malloc(sizeof(double) * W);
  for (int kv = 0; kv < d->n_kv_heads; ++kv)
    for (int64_t t = 0; t < n_tokens; ++t)
      for (int g = 0; g < G; ++g) {
        const double* xv = x + ((int64_t)kv * n_tokens + t) * D + g * W;
        for (int w = 0; w < W; ++w) res[w] = xv[w];
        for (int r = 0; r < R; ++r) {
          int best = 0;
          double bestd = INFINITY;
          for (int l = 0; l < N; ++l) {
            const double* c = codebook + cw_off(d, kv, g, r, l);
            double dd = 0.0;
            for (int w = 0; w < W; ++w) { double e = res[w] - c[w]; dd += e * e; }
            if (dd < bestd) { bestd = dd; best = l; }
          }
          const double* c = codebook + cw_off(d, kv, g, r, best);
          for (int w = 0; w < W; ++w) res[w] -= c[w];
          int64_t o = code_off(d, n_tokens, kv, t, r, g);
          codes_out[o] = (uint8_t)best;
          if (dist_out) dist_out[o] = bestd;
        }
      }
  free(res);
}

/* Evaluation of given codes under the greedy residual rule, for checking an encoder whose distances are
 * computed in another precision: for each (kv, token, group) the residual rounds are replayed with the
 * GIVEN indices; round r reports the squared distance of the given codeword to the current residual
 * (chosen_out), the minimum over all codewords (best_out) and the second smallest (second_out). A given
 * code is a valid greedy choice when chosen == best; when best and second are far apart the argmin is
 * unique. codes [Hkv][R][T][G]; the three outputs [Hkv][R][T][G]. */
void oracle_encode_eval(const oracle_dims* d, const double* x, const double* codebook, int64_t n_tokens,
                        const uint8_t* codes, double* chosen_out, double* best_out, double* second_out) {
  int D = d->head_dim, G = d->n_groups, W = D / G, R = d->n_residuals, N = d->n_codes;
  double* res = (double*)malloc(sizeof(double) * W);
  for (int kv = 0; kv < d->n_kv_heads; ++kv)
    for (int64_t t = 0; t < n_tokens; ++t)
      for (int g = 0; g < G; ++g) {
        const double* xv = x + ((int64_t)kv * n_tokens + t) * D + g * W;
        for (int w = 0; w < W; ++w) res[w] = xv[w];
        for (int r = 0; r < R; ++r) {
          int64_t o = code_off(d, n_tokens, kv, t, r, g);
          int given = codes[o];
          double b1 = INFINITY, b2 = INFINITY, dg = 0.0;
          for (int l = 0; l < N; ++l) {
            const double* c = codebook + cw_off(d, kv, g, r, l);
            double dd = 0.0;
            for (int w = 0; w < W; ++w) { double e = res[w] - c[w]; dd += e * e; }
            if (l == given) dg = dd;
            if (dd < b1) { b2 = b1; b1 = dd; } else if (dd < b2) { b2 = dd; }
          }
          chosen_out[o] = dg;
          best_out[o] = b1;
          second_out[o] = b2;
          const double* c = codebook + cw_off(d, kv, g, r, given);
          for (int w = 0; w < W; ++w) res[w] -= c[w];
        }
      }
  free(res);
}

/* One M-step of the residual codebook fit ([VER] key_machinery: "the codebook is fit by an EM-style
 * clustering algorithm", R residual rounds refine the reconstruction; [ABS]: EM training). Given the
 * assignment codes [Hkv][R][T][G] (the E-step, e.g. oracle_encode_greedy), the new codeword
 * (kv, g, r, l) is the mean, over the tokens whose round-r index is l, of their round-r residual
 *     x_g(t) - sum_{r' < r} C_in[g][r'][idx_{r'}(t)],
 * which minimizes the round's squared error for that assignment. All rounds use the input codebook for
 * the residuals (a simultaneous update). A codeword no token selects keeps its input value. x [Hkv][T][D]
 * (before RoPE); codebook_in / codebook_out [Hkv][G][R][N][W]; counts_out (optional) [Hkv][G][R][N]. */
void oracle_codebook_update(const oracle_dims* d, const double* x, const double* codebook_in, const uint8_t* codes,
                            int64_t n_tokens, double* codebook_out, int64_t* counts_out) {
  int D = d->head_dim, G = d->n_groups, W = D / G, R = d->n_residuals, N = d->n_codes;
  double* sum = (double*)calloc((size_t)N * W, sizeof(double));
  int64_t* cnt = (int64_t*)calloc((size_t)N, sizeof(int64_t));
  double* res = (double*)malloc(sizeof(double) * W);
  for (int kv = 0; kv < d->n_kv_heads; ++kv)
    for (int g = 0; g < G; ++g)
      for (int r = 0; r < R; ++r) {
        memset(sum, 0, sizeof(double) * (size_t)N * W);
        memset(cnt, 0, sizeof(int64_t) * (size_t)N);
        for (int64_t t = 0; t < n_tokens; ++t) {
          const double* xv = x + ((int64_t)kv * n_tokens + t) * D + g * W;
          for (int w = 0; w < W; ++w) res[w] = xv[w];
          for (int rp = 0; rp < r; ++rp) {
            const double* c = codebook_in + cw_off(d, kv, g, rp, codes[code_off(d, n_tokens, kv, t, rp, g)]);
            for (int w = 0; w < W; ++w) res[w] -= c[w];
          }
          int l = codes[code_off(d, n_tokens, kv, t, r, g)];
          for (int w = 0; w < W; ++w) sum[(int64_t)l * W + w] += res[w];
          cnt[l] += 1;
        }
        for (int l = 0; l < N; ++l) {
          const double* cin = codebook_in + cw_off(d, kv, g, r, l);
          double* cout = codebook_out + cw_off(d, kv, g, r, l);
          for (int w = 0; w < W; ++w) cout[w] = cnt[l] > 0 ? sum[(int64_t)l * W + w] / (double)cnt[l] : cin[w];
          if (counts_out) counts_out[(((int64_t)kv * G + g) * R + r) * N + l] = cnt[l];
        }
      }
  free(res);
  free(cnt);
  free(sum);
}

/* Bit-packed indices for codebooks of fewer than 256 entries ([VER] key_machinery and the bit-rate
 * formula R*log2(N')/g: the pages' own setting shares one index across 64 dims (g = 64) with N' = 64
 * codewords, 6 bits per index, and R = 11 or 21 rounds). Reading of the layout: a token's R*G indices
 * of b = log2(N) bits form one little-endian bitstream of 32-bit words, index (round r, group g) at bit
 * offset b*(r*G + g); a token record is ceil(b*R*G/32) words, and word w of token t is stored at
 * [Hkv][w][T] (word planes). They are unpacked into the byte layout the rest of this oracle uses,
 * [Hkv][R][T][G]. */
void oracle_unpack_bits(const oracle_dims* d, const uint32_t* words, int64_t total_tokens, uint8_t* out) {
  int G = d->n_groups, R = d->n_residuals, bits = 0;
  while ((1 << bits) < d->n_codes) ++bits;
  int64_t rec = ((int64_t)bits * R * G + 31) / 32;
  for (int kv = 0; kv < d->n_kv_heads; ++kv)
    for (int64_t t = 0; t < total_tokens; ++t) {
      const uint32_t* w = words + (int64_t)kv * rec * total_tokens + t; /* word i at w[i * total_tokens] */
      for (int r = 0; r < R; ++r)
        for (int g = 0; g < G; ++g) {
          int64_t pos = (int64_t)bits * (r * G + g);
          uint32_t v = 0;
          for (int k = 0; k < bits; ++k) {
            int64_t p = pos + k;
            v |= ((w[(p / 32) * total_tokens] >> (p % 32)) & 1u) << k;
          }
          out[code_off(d, total_tokens, kv, t, r, g)] = (uint8_t)v;
        }
    }
}
