/*
 * oracle.c -- plain, slow CPU oracle for the DSpark draft -> schedule -> verify cycle.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h).  Straight loops in IEEE double, one request
 * at a time; OpenMP only splits independent requests across threads.  Each function
 * names the passage of the pages it writes out.
 *
 * Build: gcc -O2 -std=c99 -fopenmp -fPIC -shared oracle.c -o liboracle.so -lm
 * (no -ffast-math: denormals and IEEE rounding are part of the definition).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------------------
 * element access
 * ------------------------------------------------------------------------------------ */

/* bf16 is the top half of an IEEE binary32; widening is exact. */
static double bf16_to_double(uint16_t b) {
  uint32_t bits = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* element idx of an array whose elements are dt (ORA_F32 or ORA_BF16) */
static double elem(const void *base, int dt, size_t idx) {
  if (dt == ORA_BF16) return bf16_to_double(((const uint16_t *)base)[idx]);
  return (double)((const float *)base)[idx];
}

int ora_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void ora_set_num_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ------------------------------------------------------------------------------------
 * Philox4x32-10 (Salmon et al., SC'11, section on the Philox family).
 * One round maps (x0,x1,x2,x3) with round key (k0,k1) to
 *   (hi(M1*x2) ^ x1 ^ k0,  lo(M1*x2),  hi(M0*x0) ^ x3 ^ k1,  lo(M0*x0))
 * with multipliers M0 = 0xD2511F53, M1 = 0xCD9E8D57; between rounds the key is
 * advanced by the Weyl constants (0x9E3779B9, 0xBB67AE85).
 * ------------------------------------------------------------------------------------ */
void ora_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += W0;
      k1 += W1;
    }
    uint64_t p0 = (uint64_t)M0 * (uint64_t)x0;
    uint64_t p1 = (uint64_t)M1 * (uint64_t)x2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t y0 = hi1 ^ x1 ^ k0;
    uint32_t y1 = lo1;
    uint32_t y2 = hi0 ^ x3 ^ k1;
    uint32_t y3 = lo0;
    x0 = y0; x1 = y1; x2 = y2; x3 = y3;
  }
  out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

uint32_t ora_rand_word(uint64_t seed, uint64_t cycle, int stream, uint32_t r, uint32_t k,
                       uint32_t i) {
  uint32_t key[2] = {(uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32)};
  uint32_t ctr[4] = {i >> 2, r, k, (uint32_t)((cycle << 4) | (uint64_t)(stream & 15))};
  uint32_t out[4];
  ora_philox4x32_10(ctr, key, out);
  return out[i & 3u];
}

double ora_uniform(uint64_t seed, uint64_t cycle, int stream, uint32_t r, uint32_t k,
                   uint32_t i) {
  uint32_t w = ora_rand_word(seed, cycle, stream, r, k, i);
  return (2.0 * (double)(w >> 9) + 1.0) * ldexp(1.0, -24);
}

double ora_gumbel(uint64_t seed, uint64_t cycle, int stream, uint32_t r, uint32_t k,
                  uint32_t i) {
  double u = ora_uniform(seed, cycle, stream, r, k, i);
  return -log(-log(u));
}

/* ------------------------------------------------------------------------------------
 * Sampling from softmax(l): Gumbel-max applied per block of ORA_VB ids and then inside
 * the winning block.  The max of Gumbel-perturbed logits over a set is distributed as
 * Gumbel(log-sum-exp of the set) and is independent of where it is attained, so picking
 * the block with the largest LSE_b + g_b and then the largest l(v) + g_v inside it draws
 * exactly from softmax(l).  Ties go to the lower index.
 * ------------------------------------------------------------------------------------ */
int ora_sample_two_level(int n, const double *l, uint64_t seed, uint64_t cycle,
                         int stream_blk, int stream_in, uint32_t r, uint32_t k,
                         double *gap_blk, double *gap_in) {
  int nb = (n + ORA_VB - 1) / ORA_VB;
  double best = -INFINITY, second = -INFINITY;
  int bstar = -1;
  for (int b = 0; b < nb; ++b) {
    int lo = b * ORA_VB, hi = lo + ORA_VB < n ? lo + ORA_VB : n;
    double m = -INFINITY;
    for (int v = lo; v < hi; ++v)
      if (l[v] > m) m = l[v];
    if (m == -INFINITY) continue; /* the block holds no candidate */
    double s = 0.0;
    for (int v = lo; v < hi; ++v) s += exp(l[v] - m);
    double lse_b = m + log(s);
    double G = lse_b + ora_gumbel(seed, cycle, stream_blk, r, k, (uint32_t)b);
    if (G > best) {
      second = best;
      best = G;
      bstar = b;
    } else if (G > second) {
      second = G;
    }
  }
  if (bstar < 0) return -1;
  if (gap_blk) *gap_blk = best - second;
  int lo = bstar * ORA_VB, hi = lo + ORA_VB < n ? lo + ORA_VB : n;
  double ib = -INFINITY, is = -INFINITY;
  int x = -1;
  for (int v = lo; v < hi; ++v) {
    if (l[v] == -INFINITY) continue;
    double sc = l[v] + ora_gumbel(seed, cycle, stream_in, r, k, (uint32_t)v);
    if (sc > ib) {
      is = ib;
      ib = sc;
      x = v;
    } else if (sc > is) {
      is = sc;
    }
  }
  if (gap_in) *gap_in = ib - is;
  return x;
}

/* Repeated draws for distribution tests: trial t uses request counter r = t and
 * position k = 1, so every trial reads fresh random words.  counts[n] is incremented. */
void ora_sample_trials(int n, const double *l, uint64_t seed, uint64_t cycle, int stream_blk,
                       int stream_in, long ntrials, int64_t *counts) {
  for (long t = 0; t < ntrials; ++t) {
    int x = ora_sample_two_level(n, l, seed, cycle, stream_blk, stream_in, (uint32_t)t, 1u,
                                 NULL, NULL);
    if (x >= 0) counts[x] += 1;
  }
}

/* log sum_v exp(l(v)) */
static double log_sum_exp(int n, const double *l) {
  double m = -INFINITY;
  for (int v = 0; v < n; ++v)
    if (l[v] > m) m = l[v];
  if (m == -INFINITY) return -INFINITY;
  double s = 0.0;
  for (int v = 0; v < n; ++v) s += exp(l[v] - m);
  return m + log(s);
}

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* log(1 + e^x), split so that e^x never overflows */
static double softplus(double x) { return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x))); }

/* l(v) = U_row(v) + sum_i vec[i] * W2[i][v]   (bias(x_{k-1}, .) = W1[x_{k-1}] W2, eq. (5);
 * for the RNN head vec = tanh(W_o z_k) and the product is W2^T vec, eq. (6)) */
static void logits_row(int V, int rank, int dt, const void *U, size_t u_off, const void *W2,
                       const double *vec, double *l) {
  for (int v = 0; v < V; ++v) l[v] = elem(U, dt, u_off + (size_t)v);
  for (int i = 0; i < rank; ++i) {
    double e = vec[i];
    size_t row = (size_t)i * (size_t)V;
    for (int v = 0; v < V; ++v) l[v] += e * elem(W2, dt, row + (size_t)v);
  }
}

/* the confidence logit z_k = w^T [h_k ; W1[x_{k-1}]] of eq. (7): no bias term; c_k =
 * sigma(z_k / T_k) with the position's temperature from the STS calibration (Module D),
 * T_k = 1 when uncalibrated */
static double confidence_logit(int d, int rank, int dt, const void *h, size_t h_off,
                               const float *w, const double *e) {
  double z = 0.0;
  for (int i = 0; i < d; ++i) z += (double)w[i] * elem(h, dt, h_off + (size_t)i);
  for (int i = 0; i < rank; ++i) z += (double)w[d + i] * e[i];
  return z;
}

static int check_dims(int R, int gamma, int V, int rank, int d, int dt) {
  if (R < 0 || gamma < 1 || V < 1 || rank < 1 || d < 0) return -1;
  if (dt != ORA_F32 && dt != ORA_BF16) return -1;
  return 0;
}

/* ------------------------------------------------------------------------------------
 * Draft: the sequential block's left-to-right loop, eq. (4).  Position k (1-based) adds
 * the bias of the head to the backbone's base logits U_k, takes one exact softmax,
 * samples x_k and emits the confidence c_k (eq. (7)).  The anchor x_0 is the first
 * input; the parallel block's U_1..U_gamma and h_1..h_gamma are inputs.
 * Markov head: bias_k = W1[x_{k-1}] W2 (eq. (5)).
 * RNN head: z_k = [s_{k-1}; W1[x_{k-1}]; h_k]; s_k = sg(W_g z)*s_{k-1} +
 *   (1 - sg(W_g z))*tanh(W_c z); bias_k = W2^T tanh(W_o z_k), s_0 = 0 (eq. (6)).
 * ------------------------------------------------------------------------------------ */
static int draft_common(int R, int gamma, int V, int rank, int d, int dt, const void *U,
                        const void *h, const void *W1, const void *W2, const void *W_gco,
                        const float *w, const float *temps, const int32_t *x0,
                        const int32_t *req_ids, uint64_t seed, uint64_t cycle, int32_t *x,
                        double *c, double *zc, double *lse, double *logit_x,
                        double *bias_rows, double *gap_blk, double *gap_in) {
  if (check_dims(R, gamma, V, rank, d, dt)) return -1;
  if (temps)
    for (int k = 0; k < gamma; ++k)
      if (!(temps[k] > 0.0f)) return -1;
  int bad = 0;
  for (int r = 0; r < R; ++r)
    if (x0[r] < 0 || x0[r] >= V) bad = 1;
  if (bad) return -1;
  const int K = 2 * rank + d; /* RNN input width */

#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < R; ++r) {
    double *l = (double *)malloc(sizeof(double) * (size_t)V);
    double *e = (double *)malloc(sizeof(double) * (size_t)rank);
    double *s = (double *)calloc((size_t)rank, sizeof(double)); /* s_0 = 0 */
    double *z = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    double *G = (double *)malloc(sizeof(double) * (size_t)(3 * rank));
    double *o = (double *)malloc(sizeof(double) * (size_t)rank);
    int32_t prev = x0[r];
    for (int k = 1; k <= gamma; ++k) {
      size_t rk = (size_t)r * (size_t)gamma + (size_t)(k - 1);
      for (int i = 0; i < rank; ++i) e[i] = elem(W1, dt, (size_t)prev * (size_t)rank + i);
      const double *vec = e;
      if (W_gco) {
        for (int i = 0; i < rank; ++i) z[i] = s[i];
        for (int i = 0; i < rank; ++i) z[rank + i] = e[i];
        for (int i = 0; i < d; ++i) z[2 * rank + i] = elem(h, dt, rk * (size_t)d + i);
        for (int oi = 0; oi < 3 * rank; ++oi) {
          double acc = 0.0;
          for (int ci = 0; ci < K; ++ci)
            acc += elem(W_gco, dt, (size_t)oi * (size_t)K + ci) * z[ci];
          G[oi] = acc;
        }
        for (int i = 0; i < rank; ++i) {
          double g = sigmoid(G[i]);
          double cand = tanh(G[rank + i]);
          o[i] = tanh(G[2 * rank + i]);
          s[i] = g * s[i] + (1.0 - g) * cand; /* s_k; o used z_k, i.e. s_{k-1} */
        }
        vec = o;
      }
      logits_row(V, rank, dt, U, rk * (size_t)V, W2, vec, l);
      double L = log_sum_exp(V, l);
      double gb = INFINITY, gi = INFINITY;
      uint32_t rid = req_ids ? (uint32_t)req_ids[r] : (uint32_t)r;
      int xk = ora_sample_two_level(V, l, seed, cycle, ORA_S_DRAFT_BLK, ORA_S_DRAFT_IN, rid,
                                    (uint32_t)k, &gb, &gi);
      x[rk] = xk;
      const double zk = confidence_logit(d, rank, dt, h, rk * (size_t)d, w, e);
      c[rk] = sigmoid(zk / (temps ? (double)temps[k - 1] : 1.0));
      if (zc) zc[rk] = zk;
      lse[rk] = L;
      logit_x[rk] = l[xk];
      for (int i = 0; i < rank; ++i) bias_rows[rk * (size_t)rank + i] = vec[i];
      if (gap_blk) gap_blk[rk] = gb;
      if (gap_in) gap_in[rk] = gi;
      prev = xk;
    }
    free(l); free(e); free(s); free(z); free(G); free(o);
  }
  return 0;
}

int ora_draft_markov(int R, int gamma, int V, int rank, int d, int dt, const void *U,
                     const void *h, const void *W1, const void *W2, const float *w,
                     const float *temps, const int32_t *x0, const int32_t *req_ids,
                     uint64_t seed, uint64_t cycle, int32_t *x, double *c, double *zc,
                     double *lse, double *logit_x, double *bias_rows, double *gap_blk,
                     double *gap_in) {
  return draft_common(R, gamma, V, rank, d, dt, U, h, W1, W2, NULL, w, temps, x0, req_ids,
                      seed, cycle, x, c, zc, lse, logit_x, bias_rows, gap_blk, gap_in);
}

int ora_draft_rnn(int R, int gamma, int V, int rank, int d, int dt, const void *U,
                  const void *h, const void *W1, const void *W2, const void *W_gco,
                  const float *w, const float *temps, const int32_t *x0,
                  const int32_t *req_ids, uint64_t seed, uint64_t cycle, int32_t *x, double *c,
                  double *zc, double *lse, double *logit_x, double *bias_rows, double *gap_blk,
                  double *gap_in) {
  if (!W_gco) return -1;
  return draft_common(R, gamma, V, rank, d, dt, U, h, W1, W2, W_gco, w, temps, x0, req_ids,
                      seed, cycle, x, c, zc, lse, logit_x, bias_rows, gap_blk, gap_in);
}

/* ------------------------------------------------------------------------------------
 * Training objective, forward only (Module F, eqs. (8)-(12)), on teacher-forced blocks:
 * the head's previous token at position k is the reference token x*_{k-1} of the target
 * sequence (x*_0 = the anchor), so every position of a block is known up front.
 *   q_k   = softmax(U_k + W1[x*_{k-1}] W2)      (the Markov head, eq. (5))
 *   p_k   = softmax(target row k)
 *   tv_k  = sum_v |p_k(v) - q_k(v)|,  c*_k = 1 - tv_k / 2            (eq. (8))
 *   c_k   = sigma(w . [h_k ; W1[x*_{k-1}]])                          (eq. (7))
 *   w_k   = exp(-(k-1)/gamma)
 *   L_ce  = -sum_k w_k log q_k(x*_k)                                 (eq. (9))
 *   L_tv  =  sum_k w_k tv_k                                          (eq. (10))
 *   L_conf= -sum_k w_k [c*_k log c_k + (1 - c*_k) log(1 - c_k)]      (eq. (11))
 *   L     = a_ce L_ce + a_tv L_tv + a_conf L_conf                    (eq. (12))
 * per block (request); the batch objective is their mean.
 * ------------------------------------------------------------------------------------ */
int ora_train_forward(int R, int gamma, int V, int rank, int d, int dt, const void *U,
                      const void *h, const void *W1, const void *W2, const float *w,
                      const void *target, const int32_t *x0, const int32_t *xstar,
                      const double *alpha, double *c_star, double *c, double *logq,
                      double *tv_out, double *loss) {
  if (check_dims(R, gamma, V, rank, d, dt) || !alpha) return -1;
  for (int r = 0; r < R; ++r) {
    if (x0[r] < 0 || x0[r] >= V) return -1;
    for (int k = 0; k < gamma; ++k)
      if (xstar[(size_t)r * gamma + k] < 0 || xstar[(size_t)r * gamma + k] >= V) return -1;
  }

#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < R; ++r) {
    double *l = (double *)malloc(sizeof(double) * (size_t)V);
    double *t = (double *)malloc(sizeof(double) * (size_t)V);
    double *e = (double *)malloc(sizeof(double) * (size_t)rank);
    double Lce = 0.0, Ltv = 0.0, Lconf = 0.0;
    for (int k = 1; k <= gamma; ++k) {
      const size_t rk = (size_t)r * (size_t)gamma + (size_t)(k - 1);
      const int32_t prev = k == 1 ? x0[r] : xstar[rk - 1];
      const int32_t xs = xstar[rk];
      for (int i = 0; i < rank; ++i) e[i] = elem(W1, dt, (size_t)prev * (size_t)rank + i);
      logits_row(V, rank, dt, U, rk * (size_t)V, W2, e, l);
      const double Lq = log_sum_exp(V, l);
      for (int v = 0; v < V; ++v) t[v] = elem(target, dt, rk * (size_t)V + (size_t)v);
      const double Lp = log_sum_exp(V, t);
      double tv = 0.0;
      for (int v = 0; v < V; ++v) tv += fabs(exp(t[v] - Lp) - exp(l[v] - Lq));
      const double cs = 1.0 - 0.5 * tv;
      const double zk = confidence_logit(d, rank, dt, h, rk * (size_t)d, w, e);
      const double ck = sigmoid(zk);
      const double lq = l[xs] - Lq;
      const double wk = exp(-(double)(k - 1) / (double)gamma);
      Lce += -wk * lq;
      Ltv += wk * tv;
      /* log c = -softplus(-z), log(1 - c) = -softplus(z): the same logarithms, formed
       * without the cancellation of 1 - c when c rounds to 1 */
      Lconf += wk * (cs * softplus(-zk) + (1.0 - cs) * softplus(zk));
      if (c_star) c_star[rk] = cs;
      if (c) c[rk] = ck;
      if (logq) logq[rk] = lq;
      if (tv_out) tv_out[rk] = tv;
    }
    if (loss) {
      loss[4 * (size_t)r + 0] = Lce;
      loss[4 * (size_t)r + 1] = Ltv;
      loss[4 * (size_t)r + 2] = Lconf;
      loss[4 * (size_t)r + 3] = alpha[0] * Lce + alpha[1] * Ltv + alpha[2] * Lconf;
    }
    free(l); free(t); free(e);
  }
  return 0;
}

/* ------------------------------------------------------------------------------------
 * Multi-cycle decode on a toy chain (digest, overall cycle; explainer, section 06).
 * The target is a bigram model: its logits after token t are Tb[t] (V values).  The
 * parallel backbone is a table: for anchor a, U_k = Ub[a][k-1] and h_k = Hb[a][k-1].
 * One cycle, for every request with anchor a (the last emitted token):
 *   draft x_1..x_gamma from a (Markov head, eqs. (4), (5), (7); cycle counter = cycle);
 *   choose the lengths: Algorithm 1 and its production variants (policy 0..2; the lagged
 *   variant uses the confidences of two cycles before, and the no-break search while
 *   there are none), every drafted position (FIXED), or every position whose prefix
 *   survival a_j = c_1 ... c_j (fp32, left to right) is at least `threshold` (THRESHOLD);
 *   verify against the target rows Tb[a], Tb[x_1], ..., Tb[x_gamma];
 *   emit the accepted drafts and the correction or bonus token; the last one is the next
 *   anchor.
 * Counters: stats[k-1] (k = 1..gamma) = request-cycles in which position k was tested
 * (its prefix 1..k-1 accepted and k <= ell), stats[gamma + k-1] = those in which it was
 * accepted, then sum of ell, tokens emitted, request-cycles.
 * ------------------------------------------------------------------------------------ */
int ora_decode_run(int R, int gamma, int V, int rank, int d, int dt, int ncycles,
                   const void *Ub, const void *Hb, const void *W1, const void *W2,
                   const float *w, const float *temps, const void *Tb, const int32_t *x0,
                   int policy, float threshold, const float *sps, int sps_B0, int sps_len,
                   uint64_t seed, int32_t *tokens, int32_t *n_emitted, int64_t *stats) {
  if (check_dims(R, gamma, V, rank, d, dt) || R < 1 || ncycles < 0) return -1;
  if (policy < ORA_SYNC_BREAK || policy > ORA_POLICY_THRESHOLD) return -1;
  if (policy <= ORA_ASYNC_LAG2 && !sps) return -1;
  for (int q = 0; q < R; ++q)
    if (x0[q] < 0 || x0[q] >= V) return -1;
  const size_t RG = (size_t)R * gamma, esz = dt == ORA_BF16 ? 2 : 4;
  const int maxlen = ncycles * (gamma + 1);
  char *U = (char *)malloc(esz * RG * (size_t)V);
  char *h = (char *)malloc(esz * RG * (size_t)(d > 0 ? d : 1));
  char *tg = (char *)malloc(esz * (size_t)R * (gamma + 1) * (size_t)V);
  int32_t *anchor = (int32_t *)malloc(sizeof(int32_t) * R);
  int32_t *x = (int32_t *)malloc(sizeof(int32_t) * RG);
  int32_t *ell = (int32_t *)malloc(sizeof(int32_t) * R);
  int32_t *n_acc = (int32_t *)malloc(sizeof(int32_t) * R);
  int32_t *y = (int32_t *)malloc(sizeof(int32_t) * (size_t)R * (gamma + 1));
  double *c = (double *)malloc(sizeof(double) * RG);
  double *lse = (double *)malloc(sizeof(double) * RG);
  double *lx = (double *)malloc(sizeof(double) * RG);
  double *br = (double *)malloc(sizeof(double) * RG * rank);
  double *cs = (double *)malloc(sizeof(double) * RG);
  float *cf[3];
  for (int i = 0; i < 3; ++i) cf[i] = (float *)malloc(sizeof(float) * RG);
  int rc = 0;
  memcpy(anchor, x0, sizeof(int32_t) * R);
  for (int q = 0; q < R; ++q) n_emitted[q] = 0;
  for (size_t i = 0; i < (size_t)R * maxlen; ++i) tokens[i] = -1;
  for (int i = 0; i < 2 * gamma + 3; ++i) stats[i] = 0;

  for (int cyc = 0; cyc < ncycles && rc == 0; ++cyc) {
    /* backbone stand-in: the anchor's table rows */
    for (int q = 0; q < R; ++q) {
      const size_t a = (size_t)anchor[q];
      memcpy(U + esz * (size_t)q * gamma * V, (const char *)Ub + esz * a * gamma * V,
             esz * (size_t)gamma * V);
      if (d > 0)
        memcpy(h + esz * (size_t)q * gamma * d, (const char *)Hb + esz * a * gamma * d,
               esz * (size_t)gamma * d);
    }
    rc = ora_draft_markov(R, gamma, V, rank, d, dt, U, h, W1, W2, w, temps, anchor, NULL, seed,
                          (uint64_t)cyc, x, c, NULL, lse, lx, br, NULL, NULL);
    if (rc) break;
    float *ccur = cf[cyc % 3];
    for (size_t i = 0; i < RG; ++i) ccur[i] = (float)c[i];
    if (policy == ORA_POLICY_FIXED) {
      for (int q = 0; q < R; ++q) ell[q] = gamma;
    } else if (policy == ORA_POLICY_THRESHOLD) {
      for (int q = 0; q < R; ++q) {
        float run = 1.0f;
        int l = 0;
        for (int j = 1; j <= gamma; ++j) {
          volatile float prod = (j == 1) ? ccur[(size_t)q * gamma] : run * ccur[(size_t)q * gamma + j - 1];
          run = prod;
          if (run >= threshold && l == j - 1) l = j;
        }
        ell[q] = l;
      }
    } else {
      const int lag = policy == ORA_ASYNC_LAG2 && cyc >= 2;
      const int mode = lag ? ORA_ASYNC_LAG2 : (policy == ORA_ASYNC_LAG2 ? ORA_GLOBAL : policy);
      rc = ora_schedule(R, gamma, ccur, lag ? cf[(cyc - 2) % 3] : NULL, lag ? R : 0, sps,
                        sps_B0, sps_len, mode, ell, NULL, NULL, NULL);
      if (rc) break;
    }
    /* target rows Tb[a], Tb[x_1], ..., Tb[x_gamma] */
    for (int q = 0; q < R; ++q)
      for (int j = 0; j <= gamma; ++j) {
        const size_t prev = (size_t)(j == 0 ? anchor[q] : x[(size_t)q * gamma + j - 1]);
        memcpy(tg + esz * ((size_t)q * (gamma + 1) + j) * V, (const char *)Tb + esz * prev * V,
               esz * (size_t)V);
      }
    rc = ora_verify(R, gamma, V, rank, dt, tg, U, W2, br, x, ell, NULL, seed, (uint64_t)cyc,
                    n_acc, y, cs, NULL, NULL, NULL, NULL);
    if (rc) break;
    for (int q = 0; q < R; ++q) {
      for (int k = 1; k <= ell[q]; ++k) {
        if (n_acc[q] >= k - 1) stats[k - 1] += 1;
        if (n_acc[q] >= k) stats[gamma + k - 1] += 1;
      }
      stats[2 * gamma] += ell[q];
      stats[2 * gamma + 1] += n_acc[q] + 1;
      stats[2 * gamma + 2] += 1;
      for (int i = 0; i <= n_acc[q]; ++i)
        tokens[(size_t)q * maxlen + n_emitted[q] + i] = y[(size_t)q * (gamma + 1) + i];
      n_emitted[q] += n_acc[q] + 1;
      anchor[q] = y[(size_t)q * (gamma + 1) + n_acc[q]];
    }
  }
  free(U); free(h); free(tg); free(anchor); free(x); free(ell); free(n_acc); free(y);
  free(c); free(lse); free(lx); free(br); free(cs);
  for (int i = 0; i < 3; ++i) free(cf[i]);
  return rc;
}

/* ------------------------------------------------------------------------------------
 * STS calibration (Module D).  Each c_k is a conditional probability, so the probability
 * that the prefix through position k is accepted is the running product of c_1..c_k.
 * Left to right, position k gets the temperature (from the candidate grid) whose scaled
 * confidence sigma(z_k / T) makes that running product best calibrated -- smallest
 * expected calibration error over the held-out samples -- with the earlier positions'
 * temperatures fixed.  ECE over nbins equal-width bins of [0, 1]:
 *   ECE = sum_bins | sum_{n in bin} (o_n - P_n) | / N,
 * with P_n the sample's predicted prefix probability and o_n = 1 if its accepted length
 * reaches k (0 otherwise).  Ties go to the earlier grid entry.
 * ------------------------------------------------------------------------------------ */
int ora_sts_fit(int N, int gamma, const float *z, const int32_t *n_acc, const float *grid,
                int G, int nbins, float *T, double *ece) {
  if (N < 1 || gamma < 1 || G < 1 || nbins < 1 || !z || !n_acc || !grid || !T) return -1;
  for (int g = 0; g < G; ++g)
    if (!(grid[g] > 0.0f)) return -1;
  double *pref = (double *)malloc(sizeof(double) * (size_t)N);
  double *sums = (double *)malloc(sizeof(double) * (size_t)nbins);
  for (int n = 0; n < N; ++n) pref[n] = 1.0;
  for (int k = 0; k < gamma; ++k) {
    double best = INFINITY;
    int gbest = 0;
    for (int g = 0; g < G; ++g) {
      for (int b = 0; b < nbins; ++b) sums[b] = 0.0;
      for (int n = 0; n < N; ++n) {
        const double P = pref[n] * sigmoid((double)z[(size_t)n * gamma + k] / (double)grid[g]);
        const double o = n_acc[n] > k ? 1.0 : 0.0;
        int b = (int)(P * nbins);
        if (b > nbins - 1) b = nbins - 1;
        sums[b] += o - P;
      }
      double e = 0.0;
      for (int b = 0; b < nbins; ++b) e += fabs(sums[b]);
      e /= (double)N;
      if (e < best) {
        best = e;
        gbest = g;
      }
    }
    T[k] = grid[gbest];
    if (ece) ece[k] = best;
    for (int n = 0; n < N; ++n)
      pref[n] *= sigmoid((double)z[(size_t)n * gamma + k] / (double)T[k]);
  }
  free(pref);
  free(sums);
  return 0;
}

/* ------------------------------------------------------------------------------------
 * Scheduler: Module E and Algorithm 1, with the production variants.
 *   a_{r,j} = prod_{i<=j} c_{r,i}, formed left to right in fp32 (one rounding per
 *   product, no fused multiply-add, denormals kept).
 *   E = {(r,j) : a_{r,j} > 0}, in descending a; equal a go by r, then j, ascending.
 *   B = R + (number admitted); tau = R + sum of admitted a; Theta = tau * SPS(B).
 * tau is accumulated exactly: each admitted a adds floor(a * 2^32) to a 64-bit integer
 * tau_fx (a * 2^32 is exact in fp32, so this is a truncation only for a < 2^-9), and
 * Theta = (double)tau_fx * 2^-32 * (double)SPS(B), one rounding.
 * ------------------------------------------------------------------------------------ */
typedef struct {
  float a;
  int r, j; /* j is 1-based */
} cand_t;

static int cand_cmp(const void *pa, const void *pb) {
  const cand_t *x = (const cand_t *)pa, *y = (const cand_t *)pb;
  if (x->a > y->a) return -1;
  if (x->a < y->a) return 1;
  if (x->r != y->r) return x->r < y->r ? -1 : 1;
  if (x->j != y->j) return x->j < y->j ? -1 : 1;
  return 0;
}

static double sps_at(const float *sps, int sps_B0, int B) { return (double)sps[B - sps_B0]; }

/* prefix survival and the sorted candidate list; returns |E| or -1 on bad c */
static int build_candidates(int R, int gamma, const float *c, float *a, cand_t *E) {
  int n = 0;
  for (int r = 0; r < R; ++r) {
    float run = 1.0f;
    for (int j = 1; j <= gamma; ++j) {
      float cj = c[(size_t)r * gamma + (j - 1)];
      if (!(cj >= 0.0f && cj <= 1.0f)) return -1; /* NaN or out of [0,1] */
      volatile float prod = (j == 1) ? cj : run * cj;
      run = prod;
      a[(size_t)r * gamma + (j - 1)] = run;
    }
  }
  for (int r = 0; r < R; ++r)
    for (int j = 1; j <= gamma; ++j) {
      float av = a[(size_t)r * gamma + (j - 1)];
      if (av > 0.0f) {
        E[n].a = av;
        E[n].r = r;
        E[n].j = j;
        ++n;
      }
    }
  qsort(E, (size_t)n, sizeof(cand_t), cand_cmp);
  return n;
}

static uint64_t fx_increment(float a) {
  return (uint64_t)((double)a * 4294967296.0); /* truncation = floor for a >= 0 */
}

static double theta_of(uint64_t tau_fx, double sps) {
  return ((double)tau_fx * ldexp(1.0, -32)) * sps;
}

/* Algorithm 1 walked in sorted order.  With brk != 0 the loop stops at the first
 * candidate that does not raise Theta (line 8), so the admitted set is everything before
 * it; with brk == 0 it goes to the end and keeps the first n that reached the largest
 * Theta (the strict comparison of line 7).  Returns the number admitted. */
static int admit(int R, int n_cand, const cand_t *E, const float *sps, int sps_B0, int brk,
                 double *theta_trace) {
  int B = R;
  uint64_t tau_fx = (uint64_t)R << 32;
  double best = theta_of(tau_fx, sps_at(sps, sps_B0, B));
  if (theta_trace) theta_trace[0] = best;
  int n_adm = 0;
  for (int n = 1; n <= n_cand; ++n) {
    B += 1;
    tau_fx += fx_increment(E[n - 1].a);
    double theta = theta_of(tau_fx, sps_at(sps, sps_B0, B));
    if (theta_trace) theta_trace[n] = theta;
    if (theta > best) {
      best = theta;
      n_adm = n;
    } else if (brk) {
      if (theta_trace) /* the rest is still useful to a test; no decision uses it */
        for (int m = n + 1; m <= n_cand; ++m) {
          B += 1;
          tau_fx += fx_increment(E[m - 1].a);
          theta_trace[m] = theta_of(tau_fx, sps_at(sps, sps_B0, B));
        }
      break;
    }
  }
  return n_adm;
}

int ora_schedule(int R, int gamma, const float *c, const float *c_lag, int R_lag,
                 const float *sps, int sps_B0, int sps_len, int mode, int32_t *ell,
                 float *a, double *stats, double *theta_trace) {
  if (R < 1 || gamma < 1 || !c || !sps || !ell || sps_len < 1) return -1;
  if (mode != ORA_SYNC_BREAK && mode != ORA_GLOBAL && mode != ORA_ASYNC_LAG2) return -1;
  if (mode == ORA_ASYNC_LAG2 && (!c_lag || R_lag < 1)) return -1;
  /* the table must cover B = R .. R(1+gamma) (and the lagged batch's range) */
  if (sps_B0 > R || sps_B0 + sps_len - 1 < R * (1 + gamma)) return -2;
  if (mode == ORA_ASYNC_LAG2 && (sps_B0 > R_lag || sps_B0 + sps_len - 1 < R_lag * (1 + gamma)))
    return -2;

  size_t N = (size_t)R * (size_t)gamma;
  float *aa = (float *)malloc(sizeof(float) * N);
  cand_t *E = (cand_t *)malloc(sizeof(cand_t) * (N ? N : 1));
  int n_cand = build_candidates(R, gamma, c, aa, E);
  if (n_cand < 0) {
    free(aa); free(E);
    return -1;
  }
  if (theta_trace)
    for (size_t n = 0; n <= N; ++n) theta_trace[n] = NAN;

  int n_adm;
  if (mode == ORA_ASYNC_LAG2) {
    /* capacity from the lagged confidences (no-break search), order from the current */
    size_t NL = (size_t)R_lag * (size_t)gamma;
    float *al = (float *)malloc(sizeof(float) * NL);
    cand_t *EL = (cand_t *)malloc(sizeof(cand_t) * (NL ? NL : 1));
    int nl = build_candidates(R_lag, gamma, c_lag, al, EL);
    if (nl < 0) {
      free(aa); free(E); free(al); free(EL);
      return -1;
    }
    int n_lag = admit(R_lag, nl, EL, sps, sps_B0, 0, NULL);
    int B_cap = R_lag + n_lag;
    int K = B_cap - R > 0 ? B_cap - R : 0;
    n_adm = K < n_cand ? K : n_cand;
    free(al); free(EL);
    if (theta_trace) (void)admit(R, n_cand, E, sps, sps_B0, 0, theta_trace);
  } else {
    n_adm = admit(R, n_cand, E, sps, sps_B0, mode == ORA_SYNC_BREAK, theta_trace);
  }

  for (int r = 0; r < R; ++r) ell[r] = 0;
  uint64_t tau_fx = (uint64_t)R << 32;
  for (int n = 0; n < n_adm; ++n) {
    ell[E[n].r] += 1;
    tau_fx += fx_increment(E[n].a);
  }
  if (a) memcpy(a, aa, sizeof(float) * N);
  if (stats) {
    int B = R + n_adm;
    stats[0] = (double)B;
    stats[1] = (double)tau_fx * ldexp(1.0, -32);
    stats[2] = theta_of(tau_fx, sps_at(sps, sps_B0, B));
    stats[3] = (double)n_adm;
  }
  free(aa);
  free(E);
  return 0;
}

/* The same walk with single-precision running sums, as Algorithm 1 prints them:
 * tau <- tau + a (float), Theta = tau * SPS(B) (float), the comparison Theta > Theta_best. */
int ora_schedule_literal(int R, int gamma, const float *c, const float *sps, int sps_B0,
                         int sps_len, int brk, int32_t *ell, double *theta_trace) {
  if (R < 1 || gamma < 1 || !c || !sps || !ell || sps_len < 1) return -1;
  if (sps_B0 > R || sps_B0 + sps_len - 1 < R * (1 + gamma)) return -2;
  size_t N = (size_t)R * (size_t)gamma;
  float *aa = (float *)malloc(sizeof(float) * N);
  cand_t *E = (cand_t *)malloc(sizeof(cand_t) * (N ? N : 1));
  int n_cand = build_candidates(R, gamma, c, aa, E);
  if (n_cand < 0) {
    free(aa); free(E);
    return -1;
  }
  if (theta_trace)
    for (size_t n = 0; n <= N; ++n) theta_trace[n] = NAN;
  volatile float tau = (float)R;
  volatile float best = tau * sps[R - sps_B0];
  if (theta_trace) theta_trace[0] = best;
  int n_adm = 0;
  for (int n = 1; n <= n_cand; ++n) {
    tau = tau + E[n - 1].a;
    volatile float theta = tau * sps[R + n - sps_B0];
    if (theta_trace) theta_trace[n] = theta;
    if (theta > best) {
      best = theta;
      n_adm = n;
    } else if (brk) {
      break;
    }
  }
  for (int r = 0; r < R; ++r) ell[r] = 0;
  for (int n = 0; n < n_adm; ++n) ell[E[n].r] += 1;
  free(aa);
  free(E);
  return 0;
}

/* ------------------------------------------------------------------------------------
 * Verification.  For request r with scheduled length l = ell[r], positions j = 1..l:
 *   p_j = softmax(target row j), q_j = softmax(U_j + bias_j W2) (recomputed here),
 *   c*_j = 1 - 1/2 sum_v |p_j(v) - q_j(v)|                               (eq. (8))
 *   accept x_j iff u < p_j(x_j) / q_j(x_j), u uniform (stream 2), the rule
 *   "accept with probability min(1, p/q)"; the first rejection j* ends acceptance.
 * At j*: emit a sample of normalise(max(0, p - q)) (the residual), streams 3/4.
 * If all l are accepted: emit a sample of the target row l+1 (the bonus), streams 5/6.
 * Output: accepted drafts followed by the correction or bonus token.
 * ------------------------------------------------------------------------------------ */
int ora_verify(int R, int gamma, int V, int rank, int dt, const void *target,
               const void *U, const void *W2, const double *bias_rows, const int32_t *x,
               const int32_t *ell, const int32_t *req_ids, uint64_t seed, uint64_t cycle,
               int32_t *n_acc,
               int32_t *y, double *c_star, double *pq_ratio, double *u_acc,
               double *gap_blk, double *gap_in) {
  if (check_dims(R, gamma, V, rank, 0, dt)) return -1;
  for (int r = 0; r < R; ++r) {
    if (ell[r] < 0 || ell[r] > gamma) return -1;
    for (int j = 0; j < ell[r]; ++j)
      if (x[(size_t)r * gamma + j] < 0 || x[(size_t)r * gamma + j] >= V) return -1;
  }
  const size_t G1 = (size_t)gamma + 1;

#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < R; ++r) {
    double *t = (double *)malloc(sizeof(double) * (size_t)V);
    double *p = (double *)malloc(sizeof(double) * (size_t)V);
    double *q = (double *)malloc(sizeof(double) * (size_t)V);
    double *wk = (double *)malloc(sizeof(double) * (size_t)V);
    const int l = ell[r];
    const uint32_t rid = req_ids ? (uint32_t)req_ids[r] : (uint32_t)r;
    int jstar = 0; /* first rejected position, 0 = none */
    int32_t last = -1;
    double gb = INFINITY, gi = INFINITY;
    for (int j = 1; j <= gamma; ++j) {
      size_t rj = (size_t)r * gamma + (size_t)(j - 1);
      c_star[rj] = NAN;
      if (pq_ratio) pq_ratio[rj] = NAN;
      if (u_acc) u_acc[rj] = NAN;
    }
    for (int j = 1; j <= l; ++j) {
      size_t rj = (size_t)r * gamma + (size_t)(j - 1);
      size_t trow = ((size_t)r * G1 + (size_t)(j - 1)) * (size_t)V;
      for (int v = 0; v < V; ++v) t[v] = elem(target, dt, trow + (size_t)v);
      double Lt = log_sum_exp(V, t);
      for (int v = 0; v < V; ++v) p[v] = exp(t[v] - Lt);
      logits_row(V, rank, dt, U, rj * (size_t)V, W2, bias_rows + rj * (size_t)rank, wk);
      double Lq = log_sum_exp(V, wk);
      for (int v = 0; v < V; ++v) q[v] = exp(wk[v] - Lq);
      double tv = 0.0;
      for (int v = 0; v < V; ++v) tv += fabs(p[v] - q[v]);
      c_star[rj] = 1.0 - 0.5 * tv;
      if (jstar) continue;
      int32_t xj = x[rj];
      double ratio = p[xj] / q[xj];
      double u = ora_uniform(seed, cycle, ORA_S_ACCEPT, rid, (uint32_t)j, 0u);
      if (pq_ratio) pq_ratio[rj] = ratio;
      if (u_acc) u_acc[rj] = u;
      if (u < ratio) continue; /* accepted */
      jstar = j;
      /* residual max(0, p - q), sampled through its logarithm (zeros excluded) */
      double mass = 0.0;
      for (int v = 0; v < V; ++v) {
        double rho = p[v] - q[v];
        if (rho > 0.0) {
          wk[v] = log(rho);
          mass += rho;
        } else {
          wk[v] = -INFINITY;
        }
      }
      if (!(mass > 0.0)) /* degenerate in floating point: fall back to p */
        for (int v = 0; v < V; ++v) wk[v] = t[v];
      last = ora_sample_two_level(V, wk, seed, cycle, ORA_S_RESID_BLK, ORA_S_RESID_IN, rid,
                                  (uint32_t)j, &gb, &gi);
    }
    int na = jstar ? jstar - 1 : l;
    if (!jstar) {
      size_t trow = ((size_t)r * G1 + (size_t)l) * (size_t)V; /* row l+1 */
      for (int v = 0; v < V; ++v) t[v] = elem(target, dt, trow + (size_t)v);
      last = ora_sample_two_level(V, t, seed, cycle, ORA_S_BONUS_BLK, ORA_S_BONUS_IN, rid,
                                  (uint32_t)(l + 1), &gb, &gi);
    }
    n_acc[r] = na;
    for (size_t j = 0; j < G1; ++j) y[(size_t)r * G1 + j] = -1;
    for (int j = 0; j < na; ++j) y[(size_t)r * G1 + j] = x[(size_t)r * gamma + j];
    y[(size_t)r * G1 + na] = last;
    if (gap_blk) gap_blk[r] = gb;
    if (gap_in) gap_in[r] = gi;
    free(t); free(p); free(q); free(wk);
  }
  return 0;
}
