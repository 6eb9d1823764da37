/*
 * svd_oracle.c -- plain double-precision CPU oracle (see svd_oracle.h).
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * CPU-baseline leg of the benchmark, never by the library.
 *
 * Build: gcc -O2 -std=c99 -fPIC -shared -ffp-contract=off -fno-fast-math
 *        svd_oracle.c -o liboracle.so -lm -lpthread
 * (no contraction and no fast-math, so every operation rounds as written.)
 */
#include "svd_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Counter-based uniforms.  The SplitMix64 output function is taken from its
 * published definition (Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014; Vigna's splitmix64 reference code): add the
 * golden-ratio increment, then two xor-shift-multiply rounds and a final
 * xor-shift.  One uniform per (seed, prefix row, position, purpose) stands in
 * for the per-test uniform draw of SpecDiff-2 appendix B.4. */

uint64_t svdo_splitmix64(uint64_t x)
{
  uint64_t z = x + 0x9E3779B97F4A7C15ULL;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t svdo_key(uint64_t seed, uint64_t row, uint64_t pos, uint64_t purpose)
{
  uint64_t h = svdo_splitmix64(seed);
  h = svdo_splitmix64(h ^ row);
  h = svdo_splitmix64(h ^ pos);
  h = svdo_splitmix64(h ^ purpose);
  return h;
}

double svdo_uniform(uint64_t seed, uint64_t row, uint64_t pos, uint64_t purpose)
{
  uint64_t k = svdo_key(seed, row, pos, purpose);
  return (double)(k >> 11) * 0x1.0p-53;
}

enum { PURPOSE_ACCEPT = 1, PURPOSE_RESIDUAL = 2, PURPOSE_BONUS = 3 };

/* ------------------------------------------------------------------------ */
/* Logit widening: fp32 widens exactly to double; a bf16 value is the upper
 * half of an fp32 bit pattern, so it also widens exactly. */

static double logit_at(const void *row, int dtype, int64_t v)
{
  if (dtype == SVDO_F32) return (double)((const float *)row)[v];
  uint32_t bits = (uint32_t)((const uint16_t *)row)[v] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static size_t elem_size(int dtype) { return dtype == SVDO_F32 ? 4 : 2; }

/* Softmax of one row at temperature T (SpecDiff-2 section 2: next-token
 * posteriors).  s_v = z_v / T (correctly rounded division of exact widenings),
 * m = max s, w_v = exp(s_v - m), S = sum w_v in index order, p_v = w_v / S.
 * Also returns m and S so that log p_v = (s_v - m) - log S is available. */
static int softmax_full(const void *row, int dtype, int32_t V, float T, double *prob,
                        double *m_out, double *S_out)
{
  const double Td = (double)T;
  double m = -INFINITY;
  int valid = 1;
  for (int32_t v = 0; v < V; ++v) {
    double z = logit_at(row, dtype, v);
    if (isnan(z) || z == INFINITY) valid = 0;
    double s = z / Td;
    prob[v] = s;
    if (s > m) m = s;
  }
  if (!valid || m == -INFINITY) return 0;
  double S = 0.0;
  for (int32_t v = 0; v < V; ++v) {
    double w = exp(prob[v] - m);
    prob[v] = w;
    S += w;
  }
  for (int32_t v = 0; v < V; ++v) prob[v] = prob[v] / S;
  if (m_out) *m_out = m;
  if (S_out) *S_out = S;
  return 1;
}

int svdo_softmax_row(const void *row, int dtype, int32_t V, float T, double *prob)
{
  return softmax_full(row, dtype, V, T, prob, NULL, NULL);
}

/* log p_x from the row's (m, S): (z_x / T - m) - log S. */
static double log_prob_at(const void *row, int dtype, float T, int32_t x, double m, double S)
{
  double s = logit_at(row, dtype, x) / (double)T;
  return (s - m) - log(S);
}

/* ------------------------------------------------------------------------ */
/* The draw (SpecDiff-2 section 2; DiffuSpec section 3): on a rejection the
 * replacement comes from the normalised residual max(0, p - q); after a fully
 * accepted window the bonus token comes from p.  Inverse CDF: the first token
 * whose running sum exceeds t = u * Z, so tokens of zero mass are never drawn. */

double svdo_draw_weights(const double *p, const double *q, int32_t V, double *r)
{
  double Z = 0.0;
  if (q) {
    for (int32_t v = 0; v < V; ++v) {
      double d = p[v] - q[v];
      r[v] = d > 0.0 ? d : 0.0;
      Z += r[v];
    }
    if (Z > 0.0) return Z;
  }
  /* bonus draw, or a residual without mass (p equals q numerically): draw from p */
  Z = 0.0;
  for (int32_t v = 0; v < V; ++v) {
    r[v] = p[v];
    Z += r[v];
  }
  return Z;
}

int32_t svdo_inverse_cdf(const double *r, int32_t V, double t, double *c_lo, double *c_hi)
{
  double C = 0.0;
  for (int32_t v = 0; v < V; ++v) {
    double before = C;
    C += r[v];
    if (C > t) {
      if (c_lo) *c_lo = before;
      if (c_hi) *c_hi = C;
      return v;
    }
  }
  /* t at or beyond the total through rounding: the last token with mass */
  for (int32_t v = V - 1; v >= 0; --v) {
    if (r[v] > 0.0) {
      if (c_lo) *c_lo = t;
      if (c_hi) *c_hi = t;
      return v;
    }
  }
  return -1;
}

/* ------------------------------------------------------------------------ */

typedef struct {
  const void *p, *q;
  const int32_t *drafts;
  int dtype;
  int64_t B;
  int32_t K, gamma, V;
  float tp, tq;
  uint64_t seed, row_base;
  const int32_t *force_k, *force_L;
  int32_t *selected, *accept_len, *next_token;
  double *scores, *alpha, *beta, *px, *qx, *accept_margin;
  svdo_diag_t *diag;
  int greedy;  /* greedy acceptance: alpha = p(x), no drafter rows */
  const int32_t *gamma_b;  /* per-prefix window (NULL: every window is gamma) */
  int32_t eos;             /* end-of-sequence token, or -1 */
  int nthreads, tid;
  int status;
} job_t;

static const void *p_row(const job_t *J, int64_t b, int32_t k, int32_t j)
{
  size_t idx = (((size_t)b * J->K + k) * (size_t)(J->gamma + 1) + j) * (size_t)J->V;
  return (const char *)J->p + idx * elem_size(J->dtype);
}

static const void *q_row(const job_t *J, int64_t b, int32_t k, int32_t j)
{
  size_t idx = (((size_t)b * J->K + k) * (size_t)J->gamma + j) * (size_t)J->V;
  return (const char *)J->q + idx * elem_size(J->dtype);
}

static void mark_invalid(const job_t *J, int64_t b)
{
  J->selected[b] = -1;
  J->accept_len[b] = -1;
  J->next_token[b] = -1;
}

/* One prefix, steps in the order the pages give them. */
static int do_prefix(const job_t *J, int64_t b, double *P, double *Q, double *R, double *a_buf,
                     double *s_buf, int32_t *m_buf)
{
  const int32_t K = J->K, G = J->gamma, V = J->V;
  const uint64_t row = J->row_base + (uint64_t)b;
  int valid = 1;

  /* The window: draft k proposes positions j < n (n = gamma_b[b], or gamma);
   * with an end-of-sequence token, a draft's usable positions stop at its
   * first EOS, included (DiffuSpec section 3, "Accepted prefix length": an
   * accepted EOS finishes the sequence).  m_k = that length. */
  const int32_t n = J->gamma_b ? J->gamma_b[b] : G;
  if (n < 1 || n > G) {
    mark_invalid(J, b);
    return 0;
  }
  for (int32_t k = 0; k < K; ++k) {
    m_buf[k] = n;
    for (int32_t j = 0; j < n && J->eos >= 0; ++j)
      if (J->drafts[((size_t)b * K + k) * G + j] == J->eos) {
        m_buf[k] = j + 1;
        break;
      }
  }

  /* drafted tokens must index the vocabulary */
  for (int32_t k = 0; k < K; ++k)
    for (int32_t j = 0; j < m_buf[k]; ++j) {
      int32_t x = J->drafts[((size_t)b * K + k) * G + j];
      if (x < 0 || x >= V) valid = 0;
    }

  /* 1-2. softmax of every scored row pair and the acceptance alpha_{k,j} */
  for (int32_t k = 0; k < K && valid && J->greedy; ++k) {
    /* greedy acceptance (SpecDiff-2 section 5.2 and appendix B.4): the test
     * compares the uniform with the verifier probability of the drafted
     * token, alpha = p(x); the drafter's probabilities are not used */
    for (int32_t j = 0; j < m_buf[k] && valid; ++j) {
      if (!softmax_full(p_row(J, b, k, j), J->dtype, V, J->tp, P, NULL, NULL)) {
        valid = 0;
        break;
      }
      int32_t x = J->drafts[((size_t)b * K + k) * G + j];
      size_t o = ((size_t)b * K + k) * G + j;
      a_buf[(size_t)k * G + j] = P[x];
      if (J->alpha) J->alpha[o] = P[x];
      if (J->px) J->px[o] = P[x];
    }
  }
  for (int32_t k = 0; k < K && valid && !J->greedy; ++k) {
    for (int32_t j = 0; j < m_buf[k] && valid; ++j) {
      const void *pr = p_row(J, b, k, j), *qr = q_row(J, b, k, j);
      double mp, Sp, mq, Sq;
      if (!softmax_full(pr, J->dtype, V, J->tp, P, &mp, &Sp) ||
          !softmax_full(qr, J->dtype, V, J->tq, Q, &mq, &Sq)) {
        valid = 0;
        break;
      }
      int32_t x = J->drafts[((size_t)b * K + k) * G + j];
      /* alpha = 1 when q(x) <= p(x), else p(x)/q(x); compared through log
       * probabilities so that it stays defined when both underflow */
      double lp = log_prob_at(pr, J->dtype, J->tp, x, mp, Sp);
      double lq = log_prob_at(qr, J->dtype, J->tq, x, mq, Sq);
      double a = (lq <= lp) ? 1.0 : exp(lp - lq);
      size_t o = ((size_t)b * K + k) * G + j;
      a_buf[(size_t)k * G + j] = a;
      if (J->alpha) J->alpha[o] = a;
      if (J->px) J->px[o] = P[x];
      if (J->qx) J->qx[o] = Q[x];
      if (J->beta) {
        /* 3. overlap mass sum_v min(p_v, q_v) */
        double s = 0.0;
        for (int32_t v = 0; v < V; ++v) s += (P[v] < Q[v]) ? P[v] : Q[v];
        J->beta[o] = s;
      }
    }
  }
  if (!valid) {
    mark_invalid(J, b);
    return 0;
  }

  /* 4. expected accepted streak of every draft: sum_j prod_{i<=j} alpha_i */
  for (int32_t k = 0; k < K; ++k) {
    double prod = 1.0, S = 0.0;
    for (int32_t j = 0; j < m_buf[k]; ++j) {
      prod *= a_buf[(size_t)k * G + j];
      S += prod;
    }
    s_buf[k] = S;
    if (J->scores) J->scores[(size_t)b * K + k] = S;
  }

  /* 5. self-selection: argmax, the lowest k on an exact tie */
  int32_t ks = 0;
  for (int32_t k = 1; k < K; ++k)
    if (s_buf[k] > s_buf[ks]) ks = k;
  double second = -INFINITY;
  for (int32_t k = 0; k < K; ++k)
    if (k != ks && s_buf[k] > second) second = s_buf[k];
  if (J->force_k && J->force_k[b] >= 0) {
    if (J->force_k[b] >= K) return -1;
    ks = J->force_k[b];
  }

  /* 6. left-to-right acceptance: accept position j iff u_j < alpha_{k*,j} */
  const int32_t m = m_buf[ks];
  int32_t L = m;
  for (int32_t j = 0; j < m; ++j) {
    double u = svdo_uniform(J->seed, row, (uint64_t)j, PURPOSE_ACCEPT);
    double a = a_buf[(size_t)ks * G + j];
    if (J->accept_margin) J->accept_margin[(size_t)b * G + j] = fabs(u - a);
    if (!(u < a) && L == m) L = j;
  }
  if (J->force_L && J->force_L[b] >= 0) {
    if (J->force_L[b] > m) return -1;
    L = J->force_L[b];
  }

  /* an accepted EOS ends the commit: nothing is drawn */
  if (L == m && J->eos >= 0 && J->drafts[((size_t)b * K + ks) * G + m - 1] == J->eos) {
    J->selected[b] = ks;
    J->accept_len[b] = L;
    J->next_token[b] = -2;
    if (J->diag) {
      svdo_diag_t *d = &J->diag[b];
      d->select_gap = (K > 1) ? s_buf[ks] - second : INFINITY;
      d->emit_margin = INFINITY;
      d->draw_z = 0.0;
      d->draw_t = 0.0;
    }
    return 0;
  }

  /* 7-8. residual draw at the first rejection, or bonus draw (p row n) after
   * the whole window is accepted */
  double Z, u;
  if (L < m && J->greedy) {
    /* the rejected token zeroed out (SpecDiff-2 appendix B.4): the residual
     * max(0, p - q) with q the point mass at the drafted token */
    softmax_full(p_row(J, b, ks, L), J->dtype, V, J->tp, P, NULL, NULL);
    for (int32_t v = 0; v < V; ++v) Q[v] = 0.0;
    Q[J->drafts[((size_t)b * K + ks) * G + L]] = 1.0;
    Z = svdo_draw_weights(P, Q, V, R);
    u = svdo_uniform(J->seed, row, (uint64_t)L, PURPOSE_RESIDUAL);
  } else if (L < m) {
    softmax_full(p_row(J, b, ks, L), J->dtype, V, J->tp, P, NULL, NULL);
    softmax_full(q_row(J, b, ks, L), J->dtype, V, J->tq, Q, NULL, NULL);
    Z = svdo_draw_weights(P, Q, V, R);
    u = svdo_uniform(J->seed, row, (uint64_t)L, PURPOSE_RESIDUAL);
  } else {
    if (!softmax_full(p_row(J, b, ks, n), J->dtype, V, J->tp, P, NULL, NULL)) {
      mark_invalid(J, b);
      return 0;
    }
    Z = svdo_draw_weights(P, NULL, V, R);
    u = svdo_uniform(J->seed, row, (uint64_t)n, PURPOSE_BONUS);
  }
  double t = u * Z, lo = 0.0, hi = 0.0;
  int32_t tok = svdo_inverse_cdf(R, V, t, &lo, &hi);

  /* 9. outputs */
  J->selected[b] = ks;
  J->accept_len[b] = L;
  J->next_token[b] = tok;
  if (J->diag) {
    svdo_diag_t *d = &J->diag[b];
    d->select_gap = (K > 1) ? s_buf[ks] - second : INFINITY;
    double m1 = t - lo, m2 = hi - t;
    d->emit_margin = (m1 < m2 ? m1 : m2) / Z;
    d->draw_z = Z;
    d->draw_t = t;
  }
  return 0;
}

static void *worker(void *arg)
{
  job_t *J = (job_t *)arg;
  double *P = (double *)malloc(sizeof(double) * (size_t)J->V);
  double *Q = (double *)malloc(sizeof(double) * (size_t)J->V);
  double *R = (double *)malloc(sizeof(double) * (size_t)J->V);
  double *A = (double *)malloc(sizeof(double) * (size_t)J->K * (size_t)J->gamma);
  double *S = (double *)malloc(sizeof(double) * (size_t)J->K);
  int32_t *M = (int32_t *)malloc(sizeof(int32_t) * (size_t)J->K);
  if (!P || !Q || !R || !A || !S || !M) {
    J->status = -1;
  } else {
    for (int64_t b = J->tid; b < J->B; b += J->nthreads)
      if (do_prefix(J, b, P, Q, R, A, S, M) != 0) J->status = -1;
  }
  free(P);
  free(Q);
  free(R);
  free(A);
  free(S);
  free(M);
  return NULL;
}

static int run_jobs(const job_t *base_in)
{
  job_t base = *base_in;
  int nthreads = base.nthreads < 1 ? 1 : base.nthreads;
  if ((int64_t)nthreads > base.B) nthreads = (int)base.B;
  base.nthreads = nthreads;
  job_t *jobs = (job_t *)malloc(sizeof(job_t) * (size_t)nthreads);
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  if (!jobs || !th) {
    free(jobs);
    free(th);
    return -1;
  }
  for (int i = 0; i < nthreads; ++i) {
    jobs[i] = base;
    jobs[i].tid = i;
  }
  int started = 0;
  for (int i = 1; i < nthreads; ++i) {
    if (pthread_create(&th[i], NULL, worker, &jobs[i]) != 0) break;
    started = i;
  }
  worker(&jobs[0]);
  for (int i = 1; i <= started; ++i) pthread_join(th[i], NULL);
  /* prefixes of threads that failed to start run here */
  for (int i = started + 1; i < nthreads; ++i) worker(&jobs[i]);

  int status = 0;
  for (int i = 0; i < nthreads; ++i)
    if (jobs[i].status != 0) status = -1;
  free(jobs);
  free(th);
  return status;
}

int svdo_select_and_verify(const void *p_logits, const void *q_logits, const int32_t *drafts,
                           int dtype, int64_t B, int32_t K, int32_t gamma, int32_t V,
                           float temp_p, float temp_q, uint64_t seed, uint64_t row_base,
                           const int32_t *force_k, const int32_t *force_L,
                           int32_t *selected, int32_t *accept_len, int32_t *next_token,
                           double *scores, double *alpha, double *beta, double *px, double *qx,
                           double *accept_margin, svdo_diag_t *diag, int nthreads)
{
  if (!p_logits || !q_logits || !drafts || !selected || !accept_len || !next_token) return -1;
  if (dtype != SVDO_F32 && dtype != SVDO_BF16) return -1;
  if (B < 1 || K < 1 || gamma < 1 || V < 1) return -1;
  if (!(temp_p > 0.0f) || !(temp_q > 0.0f) || isinf(temp_p) || isinf(temp_q)) return -1;

  job_t base;
  memset(&base, 0, sizeof base);
  base.p = p_logits;
  base.q = q_logits;
  base.drafts = drafts;
  base.dtype = dtype;
  base.B = B;
  base.K = K;
  base.gamma = gamma;
  base.V = V;
  base.tp = temp_p;
  base.tq = temp_q;
  base.seed = seed;
  base.row_base = row_base;
  base.force_k = force_k;
  base.force_L = force_L;
  base.selected = selected;
  base.accept_len = accept_len;
  base.next_token = next_token;
  base.scores = scores;
  base.alpha = alpha;
  base.beta = beta;
  base.px = px;
  base.qx = qx;
  base.accept_margin = accept_margin;
  base.diag = diag;
  base.eos = -1;
  base.nthreads = nthreads;
  return run_jobs(&base);
}

int svdo_greedy_select_and_verify(const void *p_logits, const int32_t *drafts, int dtype,
                                  int64_t B, int32_t K, int32_t gamma, int32_t V, float temp_p,
                                  uint64_t seed, uint64_t row_base, const int32_t *force_k,
                                  const int32_t *force_L, int32_t *selected, int32_t *accept_len,
                                  int32_t *next_token, double *scores, double *alpha,
                                  double *accept_margin, svdo_diag_t *diag, int nthreads)
{
  if (!p_logits || !drafts || !selected || !accept_len || !next_token) return -1;
  if (dtype != SVDO_F32 && dtype != SVDO_BF16) return -1;
  if (B < 1 || K < 1 || gamma < 1 || V < 1) return -1;
  if (!(temp_p > 0.0f) || isinf(temp_p)) return -1;

  job_t base;
  memset(&base, 0, sizeof base);
  base.p = p_logits;
  base.drafts = drafts;
  base.dtype = dtype;
  base.B = B;
  base.K = K;
  base.gamma = gamma;
  base.V = V;
  base.tp = temp_p;
  base.tq = temp_p;
  base.seed = seed;
  base.row_base = row_base;
  base.force_k = force_k;
  base.force_L = force_L;
  base.selected = selected;
  base.accept_len = accept_len;
  base.next_token = next_token;
  base.scores = scores;
  base.alpha = alpha;
  base.accept_margin = accept_margin;
  base.diag = diag;
  base.greedy = 1;
  base.eos = -1;
  base.nthreads = nthreads;
  return run_jobs(&base);
}

int svdo_window_select_and_verify(int greedy, const void *p_logits, const void *q_logits,
                                  const int32_t *drafts, const int32_t *gamma_b, int32_t eos,
                                  int dtype, int64_t B, int32_t K, int32_t gamma, int32_t V,
                                  float temp_p, float temp_q, uint64_t seed, uint64_t row_base,
                                  const int32_t *force_k, const int32_t *force_L,
                                  int32_t *selected, int32_t *accept_len, int32_t *next_token,
                                  double *scores, double *alpha, double *accept_margin,
                                  svdo_diag_t *diag, int nthreads)
{
  if (!p_logits || (!q_logits && !greedy) || !drafts || !selected || !accept_len || !next_token)
    return -1;
  if (dtype != SVDO_F32 && dtype != SVDO_BF16) return -1;
  if (B < 1 || K < 1 || gamma < 1 || V < 1 || eos >= V) return -1;
  if (!(temp_p > 0.0f) || isinf(temp_p)) return -1;
  if (!greedy && (!(temp_q > 0.0f) || isinf(temp_q))) return -1;

  job_t base;
  memset(&base, 0, sizeof base);
  base.p = p_logits;
  base.q = greedy ? NULL : q_logits;
  base.drafts = drafts;
  base.dtype = dtype;
  base.B = B;
  base.K = K;
  base.gamma = gamma;
  base.V = V;
  base.tp = temp_p;
  base.tq = greedy ? temp_p : temp_q;
  base.seed = seed;
  base.row_base = row_base;
  base.force_k = force_k;
  base.force_L = force_L;
  base.selected = selected;
  base.accept_len = accept_len;
  base.next_token = next_token;
  base.scores = scores;
  base.alpha = alpha;
  base.accept_margin = accept_margin;
  base.diag = diag;
  base.greedy = greedy != 0;
  base.gamma_b = gamma_b;
  base.eos = eos < 0 ? -1 : eos;
  base.nthreads = nthreads;
  return run_jobs(&base);
}

/* ------------------------------------------------------------------------ */
/* Causal-consistency path search (DiffuSpec section 4.2; its settings B = 3,
 * M_max = 15, tau = 0.8 in section 5.3).  The drafter's per-position
 * candidates form a lattice: each position keeps its most probable tokens
 * until their cumulative mass reaches tau (at most m_max of them), and the
 * lattice stops at the first position whose most probable token is EOS.  A
 * left-to-right beam search then scores paths by drafter confidence plus a
 * causal-proxy fluency term, which is an input here. */

/* the order of a row's tokens: larger logit first, the lower index on a tie */
static int before(const void *row, int dtype, int32_t a, int32_t b)
{
  double za = logit_at(row, dtype, a), zb = logit_at(row, dtype, b);
  return za > zb || (za == zb && a < b);
}

int svdo_cps_lattice(const void *q_logits, int dtype, int64_t B, int32_t G, int32_t V,
                     float temp_q, double tau, int32_t m_max, int32_t eos, int32_t *cand,
                     double *cand_logp, int32_t *n_cand, int32_t *len, double *cum_margin)
{
  if (!q_logits || !cand || !cand_logp || !n_cand || !len) return -1;
  if (B < 1 || G < 1 || V < 1 || m_max < 1 || !(tau > 0.0) || tau > 1.0) return -1;
  if (!(temp_q > 0.0f) || isinf(temp_q)) return -1;
  double *P = (double *)malloc(sizeof(double) * (size_t)V);
  if (!P) return -1;
  for (int64_t b = 0; b < B; ++b) {
    len[b] = G;
    for (int32_t j = 0; j < G; ++j) {
      const size_t o = (size_t)b * G + j;
      int32_t *c = cand + o * m_max;
      double *lp = cand_logp + o * m_max;
      for (int32_t i = 0; i < m_max; ++i) {
        c[i] = -1;
        lp[i] = -INFINITY;
      }
      n_cand[o] = 0;
      if (cum_margin) cum_margin[o] = INFINITY;
      if (j >= len[b]) continue;
      const void *row = (const char *)q_logits + o * (size_t)V * elem_size(dtype);
      double m, S;
      if (!softmax_full(row, dtype, V, temp_q, P, &m, &S)) {
        len[b] = -1;  /* invalid row: no lattice for this prefix */
        continue;
      }
      /* the m_max most probable tokens, in order (selection by repeated scans) */
      int32_t n = 0;
      double cum = 0.0, prev_cum = 0.0;
      for (int32_t i = 0; i < m_max && i < V; ++i) {
        int32_t best = -1;
        for (int32_t v = 0; v < V; ++v) {
          int taken = 0;
          for (int32_t t = 0; t < i; ++t) taken |= (c[t] == v);
          if (!taken && (best < 0 || before(row, dtype, v, best))) best = v;
        }
        c[i] = best;
        lp[i] = log_prob_at(row, dtype, temp_q, best, m, S);
        prev_cum = cum;
        cum += P[best];
        n = i + 1;
        if (cum >= tau) break;
      }
      n_cand[o] = n;
      if (cum_margin) {
        double mg = fabs(cum - tau);
        if (n > 1 && fabs(prev_cum - tau) < mg) mg = fabs(prev_cum - tau);
        cum_margin[o] = mg;
      }
      for (int32_t i = n; i < m_max; ++i) {
        c[i] = -1;
        lp[i] = -INFINITY;
      }
      /* the lattice stops at the first position whose most probable token is EOS */
      if (eos >= 0 && c[0] == eos) {
        for (int32_t i = 1; i < m_max; ++i) {
          c[i] = -1;
          lp[i] = -INFINITY;
        }
        n_cand[o] = 1;
        if (cum_margin) cum_margin[o] = INFINITY;
        len[b] = j + 1;
      }
    }
    if (len[b] < 0)
      for (int32_t j = 0; j < G; ++j) n_cand[(size_t)b * G + j] = 0;
  }
  free(P);
  return 0;
}

int svdo_cps_beam(const int32_t *cand, const double *cand_logp, const int32_t *n_cand,
                  const int32_t *len, const float *fluency, double lambda, int64_t B, int32_t G,
                  int32_t m_max, int32_t beam, int32_t *paths, double *path_score,
                  int32_t *path_len, double *rank_margin)
{
  if (!cand || !cand_logp || !n_cand || !len || !paths || !path_score || !path_len) return -1;
  if (B < 1 || G < 1 || m_max < 1 || beam < 1) return -1;
  const int32_t E = beam * m_max;  /* expansions per step, at most */
  int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)beam * G);  /* candidate ranks */
  int32_t *nidx = (int32_t *)malloc(sizeof(int32_t) * (size_t)beam * G);
  double *sc = (double *)malloc(sizeof(double) * (size_t)beam);
  double *nsc = (double *)malloc(sizeof(double) * (size_t)beam);
  double *es = (double *)malloc(sizeof(double) * (size_t)E);
  int32_t *ep = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
  int32_t *ei = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
  char *used = (char *)malloc((size_t)E);
  int status = 0;
  if (!idx || !nidx || !sc || !nsc || !es || !ep || !ei || !used) status = -1;
  for (int64_t b = 0; b < B && status == 0; ++b) {
    const int32_t n_len = len[b];
    double margin = INFINITY;
    int32_t nb = 1;  /* live paths, best first */
    sc[0] = 0.0;
    for (int32_t j = 0; j < n_len; ++j) {
      const size_t o = (size_t)b * G + j;
      const int32_t nc = n_cand[o];
      /* every expansion (path p, candidate i), in order: path rank, then candidate rank */
      int32_t ne = 0;
      for (int32_t p = 0; p < nb; ++p)
        for (int32_t i = 0; i < nc; ++i) {
          /* the proxy's transition from the path's last candidate (the context at j = 0) */
          const int32_t prev = (j == 0) ? 0 : idx[(size_t)p * G + j - 1];
          const double f = fluency ? (double)fluency[(o * m_max + prev) * m_max + i] : 0.0;
          es[ne] = sc[p] + cand_logp[o * m_max + i] + lambda * f;
          /* a score made NaN by the proxy ranks below every other one */
          if (isnan(es[ne])) es[ne] = -INFINITY;
          ep[ne] = p;
          ei[ne] = i;
          used[ne] = 0;
          ++ne;
        }
      /* keep the `beam` best, the earlier expansion on an exact tie */
      const int32_t keep = ne < beam ? ne : beam;
      double last = 0.0;
      for (int32_t r = 0; r < keep; ++r) {
        int32_t best = -1;
        for (int32_t e = 0; e < ne; ++e)
          if (!used[e] && (best < 0 || es[e] > es[best])) best = e;
        if (r > 0 && last - es[best] < margin) margin = last - es[best];
        last = es[best];
        used[best] = 1;
        for (int32_t t = 0; t < j; ++t) nidx[(size_t)r * G + t] = idx[(size_t)ep[best] * G + t];
        nidx[(size_t)r * G + j] = ei[best];
        nsc[r] = es[best];
      }
      if (keep < ne) {  /* the gap to the best expansion left out */
        int32_t best = -1;
        for (int32_t e = 0; e < ne; ++e)
          if (!used[e] && (best < 0 || es[e] > es[best])) best = e;
        if (last - es[best] < margin) margin = last - es[best];
      }
      for (int32_t r = 0; r < keep; ++r) {
        sc[r] = nsc[r];
        for (int32_t t = 0; t <= j; ++t) idx[(size_t)r * G + t] = nidx[(size_t)r * G + t];
      }
      nb = keep;
    }
    for (int32_t r = 0; r < beam; ++r) {
      int32_t *out = paths + ((size_t)b * beam + r) * G;
      for (int32_t t = 0; t < G; ++t) out[t] = -1;
      const int live = n_len > 0 && r < nb;
      path_len[(size_t)b * beam + r] = live ? n_len : 0;
      path_score[(size_t)b * beam + r] = live ? sc[r] : -INFINITY;
      if (live)
        for (int32_t t = 0; t < n_len; ++t)
          out[t] = cand[((size_t)b * G + t) * m_max + idx[(size_t)r * G + t]];
    }
    if (rank_margin) rank_margin[b] = margin;
  }
  free(idx); free(nidx); free(sc); free(nsc); free(es); free(ep); free(ei); free(used);
  return status;
}

/* ------------------------------------------------------------------------ */
/* Adaptive draft length (DiffuSpec section 4.3): the controller uses the
 * EOS-aware generated length and the accepted length; it grows the window
 * while acceptance keeps up with generation on average and stops growing it
 * once the generated length saturates at EOS.  Shrinking toward the recent
 * accepted length when acceptance lags is this oracle's reading of "avoid
 * over-drafting" (DiffuSpec section 6).  The averages are kept in 1/256ths of
 * a token so every decision is an exact integer comparison. */

/* x / 2^shift rounded toward minus infinity, for |x| < 2^31 */
static int32_t adl_floor_div(int32_t x, int32_t shift) {
  return (int32_t)floor((double)x / (double)((int64_t)1 << shift));
}

int svdo_adl_next(const int32_t *drafts, const int32_t *selected, const int32_t *accept_len,
                  const int32_t *gamma_b, int32_t eos, int64_t B, int32_t K, int32_t gamma,
                  int32_t k_min, int32_t k_max, int32_t step, int32_t shift, int32_t slack,
                  int32_t *avg, int32_t *next) {
  const int32_t lim = 1 << 20;
  if (B < 0 || K < 1 || K > 64 || gamma < 1 || gamma > 4096 || k_min < 1 || k_max < k_min ||
      k_max > 4096 || step < 0 || step > 4096 || shift < 0 || shift > 16 || slack < 0 ||
      slack > lim)
    return -1;
  for (int64_t b = 0; b < B; ++b) {
    const int32_t n = gamma_b ? gamma_b[b] : gamma;
    if (n < 1 || n > gamma) {
      next[b] = -1;
      continue;
    }
    const int32_t k = selected[b], L = accept_len[b];
    if (k < 0 || k >= K || L < 0 || L > n) {
      next[b] = n;
      continue;
    }
    int32_t A = avg[2 * b], G = avg[2 * b + 1];
    if (A < 0 || A > lim || G < 0 || G > lim) {
      next[b] = -1;
      continue;
    }
    /* the kept draft's generated length: up to and including its first EOS */
    int32_t g = n;
    if (eos >= 0)
      for (int32_t j = 0; j < n; ++j)
        if (drafts[((size_t)b * K + k) * gamma + j] == eos) {
          g = j + 1;
          break;
        }
    /* recent lengths, 1/256ths of a token */
    A = A + adl_floor_div(256 * L - A, shift);
    G = G + adl_floor_div(256 * g - G, shift);
    avg[2 * b] = A;
    avg[2 * b + 1] = G;
    int32_t w;
    if (g < n) {
      w = n;                                   /* generated length saturated: hold */
    } else if (A + slack >= G) {
      w = n + step;                            /* acceptance keeps pace: expand */
    } else {
      w = (int32_t)ceil((double)A / 256.0) + 1;  /* acceptance lags: shrink */
      if (w > n) w = n;
    }
    if (w < k_min) w = k_min;
    if (w > k_max) w = k_max;
    next[b] = w;
  }
  return 0;
}
