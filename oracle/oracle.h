/*
 * oracle.h -- plain, slow CPU oracle for the DSpark draft -> schedule -> verify cycle.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link, load or
 * call this code: only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it.  It shares no code, header, table or helper with the HIP library.
 *
 * Sources (three web pages on one paper, "DSpark: confidence-scheduled speculative
 * decoding"):
 *   [digest]    the technical digest page (slinene.github.io, ai-papers-daily):
 *               core idea eq. (1); Module B eqs. (4)-(6); Module C eqs. (7)-(8);
 *               Module D (sequential temperature scaling);
 *               Module E (prefix survival, B, tau, Theta, Algorithm 1, Appendix-A
 *               counterexample); production section (no-break search, two-step lag).
 *   [explainer] the interactive explainer (share.concentrate1.com): section 06,
 *               the single-token rejection rule.
 *
 * Floating point: every quantity of the method is computed in IEEE double, except the
 * scheduler's prefix survival a_{r,j}, which is fp32 by definition here (see
 * ora_schedule) so that a GPU implementation can match it bit for bit.
 * Inputs given as bf16 are widened exactly (bits << 16).
 *
 * Random numbers: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers:
 * as easy as 1, 2, 3", SC'11), keyed and countered as ora_rand_word documents.  The
 * pages fix no generator; this counter layout is this project's convention.
 */
#ifndef DSPARK_ORACLE_H
#define DSPARK_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element type of the big operands (U, h, W1, W2, W_gco, target logits) */
enum { ORA_F32 = 0, ORA_BF16 = 1 };

/* scheduler variants */
enum {
  ORA_SYNC_BREAK = 0, /* Algorithm 1 as printed, early-stop break           */
  ORA_GLOBAL = 1,     /* no break: unconstrained search over all prefixes    */
  ORA_ASYNC_LAG2 = 2  /* capacity from confidences two cycles old, top-K now */
};

/* length policies of the multi-cycle driver beyond the scheduler's three */
enum {
  ORA_POLICY_FIXED = 3,    /* verify every drafted position (scheduler off)       */
  ORA_POLICY_THRESHOLD = 4 /* verify positions whose prefix survival >= threshold */
};

/* random streams (counter word 3 low nibble) */
enum {
  ORA_S_DRAFT_BLK = 0, ORA_S_DRAFT_IN = 1, ORA_S_ACCEPT = 2,
  ORA_S_RESID_BLK = 3, ORA_S_RESID_IN = 4, ORA_S_BONUS_BLK = 5, ORA_S_BONUS_IN = 6
};

/* block size of the two-level Gumbel-max sampler */
#define ORA_VB 64

/* Philox4x32 with 10 rounds on one counter block. */
void ora_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

/* One 32-bit word: key = (seed lo, seed hi), counter = (i >> 2, r, k, cycle<<4 | stream),
 * word i & 3 of the output.  cycle must be < 2^28, stream < 16. */
uint32_t ora_rand_word(uint64_t seed, uint64_t cycle, int stream, uint32_t r, uint32_t k,
                       uint32_t i);
/* u = (2*(word >> 9) + 1) * 2^-24, in (0,1), exact in fp32 */
double ora_uniform(uint64_t seed, uint64_t cycle, int stream, uint32_t r, uint32_t k,
                   uint32_t i);
/* g = -ln(-ln u) */
double ora_gumbel(uint64_t seed, uint64_t cycle, int stream, uint32_t r, uint32_t k,
                  uint32_t i);

/* Two-level Gumbel-max sample of softmax(l) over n entries (l may hold -inf for
 * excluded entries; at least one must be finite).  Blocks are ORA_VB consecutive ids
 * (the last one may be short).  Returns the index; writes the gap between the top two
 * block scores and between the top two in-block scores (INFINITY if only one
 * candidate).  Returns -1 if every entry is -inf. */
int ora_sample_two_level(int n, const double *l, uint64_t seed, uint64_t cycle,
                         int stream_blk, int stream_in, uint32_t r, uint32_t k,
                         double *gap_blk, double *gap_in);

/* ntrials draws of ora_sample_two_level on the same l, trial t using counter r = t,
 * k = 1; counts[n] accumulates the drawn indices (distribution tests). */
void ora_sample_trials(int n, const double *l, uint64_t seed, uint64_t cycle, int stream_blk,
                       int stream_in, long ntrials, int64_t *counts);

/* Markov-head draft, eqs. (4), (5), (7).  Layouts (row-major):
 *   U [R][gamma][V], h [R][gamma][d], W1 [V][rank], W2 [rank][V]   (dt)
 *   w [d + rank] fp32, order [h-part ; W1-row part]; x0 [R]
 *   temps [gamma] (nullable): STS temperatures (Module D), c_k = sigma(z_k / temps[k-1]);
 *     NULL means 1 at every position; each must be > 0
 *   req_ids [R] (nullable): the request index each row uses in the random counters
 *     (default: its position 0..R-1), so a subset of a batch can be checked alone
 * Outputs: x [R][gamma], c, lse, logit_x [R][gamma] (double), zc [R][gamma] (double,
 *   nullable): the confidence logit z_k = w . [h_k ; W1[x_{k-1}]] before the temperature,
 *   bias_rows [R][gamma][rank] (double): the vector that multiplies W2 at step k,
 *   gap_blk, gap_in [R][gamma] (nullable).
 * Returns 0, or -1 on a bad argument / token out of range. */
int ora_draft_markov(int R, int gamma, int V, int rank, int d, int dt, const void *U,
                     const void *h, const void *W1, const void *W2, const float *w,
                     const float *temps, const int32_t *x0, const int32_t *req_ids,
                     uint64_t seed, uint64_t cycle, int32_t *x, double *c, double *zc,
                     double *lse, double *logit_x, double *bias_rows, double *gap_blk,
                     double *gap_in);

/* RNN-head draft, eq. (6) with eq. (7) for c.  W_gco [3*rank][2*rank + d] (dt): rows
 * [0,rank) gate, [rank,2rank) candidate, [2rank,3rank) output; columns ordered
 * [s ; W1 row ; h].  s_0 = 0.  bias_rows receives tanh(W_o z_k).  Other arguments as
 * ora_draft_markov. */
int ora_draft_rnn(int R, int gamma, int V, int rank, int d, int dt, const void *U,
                  const void *h, const void *W1, const void *W2, const void *W_gco,
                  const float *w, const float *temps, const int32_t *x0,
                  const int32_t *req_ids, uint64_t seed, uint64_t cycle, int32_t *x, double *c,
                  double *zc, double *lse, double *logit_x, double *bias_rows, double *gap_blk,
                  double *gap_in);

/* Training objective forward (Module F, eqs. (8)-(12)) with the Markov head on
 * teacher-forced blocks: position k's previous token is x*_{k-1} (x*_0 = x0[r]).
 *   target [R][gamma][V] (dt): target logits of positions 1..gamma
 *   xstar [R][gamma]: reference tokens x*_1..x*_gamma; alpha[3] = (a_ce, a_tv, a_conf)
 * Outputs (each nullable), [R][gamma]: c_star = 1 - tv/2, c = sigma(w.[h;W1[x*_{k-1}]]),
 *   logq = log q_k(x*_k), tv = ||p_k - q_k||_1;  loss [R][4] = (L_ce, L_tv, L_conf, L)
 *   with position weights exp(-(k-1)/gamma).
 * Returns 0, or -1 on a bad argument (a token out of range). */
int ora_train_forward(int R, int gamma, int V, int rank, int d, int dt, const void *U,
                      const void *h, const void *W1, const void *W2, const float *w,
                      const void *target, const int32_t *x0, const int32_t *xstar,
                      const double *alpha, double *c_star, double *c, double *logq,
                      double *tv, double *loss);

/* Multi-cycle decode on a toy chain: bigram target Tb [V][V] (logits after token t are
 * row t), table backbone Ub [V][gamma][V] and Hb [V][gamma][d] (U_k, h_k for anchor a are
 * row a, k-1).  policy: ORA_SYNC_BREAK / ORA_GLOBAL / ORA_ASYNC_LAG2 (sps as in
 * ora_schedule; the lagged variant searches without the break until two cycles exist),
 * ORA_POLICY_FIXED (ell = gamma) or ORA_POLICY_THRESHOLD (ell = the positions whose
 * prefix survival is >= threshold).  Cycle c uses random-counter cycle c.
 * Outputs: tokens [R][ncycles*(gamma+1)] (emitted tokens, -1 after the last), n_emitted
 * [R], stats [2*gamma+3] = tested per position, accepted per position, sum of ell,
 * tokens emitted, request-cycles.  Returns 0, -1 bad argument, -2 SPS range. */
int ora_decode_run(int R, int gamma, int V, int rank, int d, int dt, int ncycles,
                   const void *Ub, const void *Hb, const void *W1, const void *W2,
                   const float *w, const float *temps, const void *Tb, const int32_t *x0,
                   int policy, float threshold, const float *sps, int sps_B0, int sps_len,
                   uint64_t seed, int32_t *tokens, int32_t *n_emitted, int64_t *stats);

/* STS calibration (Module D): per-position temperatures fitted left to right on held-out
 * samples, each minimising the expected calibration error of the running product of the
 * scaled confidences, earlier positions fixed.
 *   z [N][gamma] fp32: confidence logits (before any temperature)
 *   n_acc [N]: accepted length of each sample's drafted block (0..gamma)
 *   grid [G] fp32 candidate temperatures (> 0); nbins equal-width bins of [0, 1]
 * Outputs: T [gamma]; ece [gamma] (nullable): the ECE reached at each position.
 * Returns 0, or -1 on a bad argument. */
int ora_sts_fit(int N, int gamma, const float *z, const int32_t *n_acc, const float *grid,
                int G, int nbins, float *T, double *ece);

/* Prefix scheduler (Module E, Algorithm 1 and the production variants).
 *   c [R][gamma] fp32; c_lag [R_lag][gamma] (ASYNC_LAG2 only, else NULL)
 *   SPS(B) = sps[B - sps_B0] for B in [sps_B0, sps_B0 + sps_len)
 * Outputs: ell [R]; a [R][gamma] (nullable); stats [4] = {B, tau, Theta, n_admitted}
 * (nullable); theta_trace [R*gamma + 1] (nullable) = Theta_n for n = 0..|E| in sorted
 * order of the current confidences (NaN past |E|).
 * Returns 0, -1 bad argument, -2 SPS table does not cover the batches needed. */
int ora_schedule(int R, int gamma, const float *c, const float *c_lag, int R_lag,
                 const float *sps, int sps_B0, int sps_len, int mode, int32_t *ell,
                 float *a, double *stats, double *theta_trace);

/* Algorithm 1 with its running sums taken literally in single precision (digest, Module E:
 * tau* <- tau* + a and Theta = tau* x SPS(B) as float operations, tau* starting at R), on
 * the same candidate order as ora_schedule.  brk != 0: the early-stop break (SYNC_BREAK);
 * brk == 0: no break, the first largest Theta (GLOBAL).  Used to measure how often the
 * exact fixed-point reading of ora_schedule decides differently (only where two Theta
 * values lie within the single-precision rounding of each other).  theta_trace [R*gamma+1]
 * (nullable) receives the float Theta_n of every prefix (NaN past |E|). */
int ora_schedule_literal(int R, int gamma, const float *c, const float *sps, int sps_B0,
                         int sps_len, int brk, int32_t *ell, double *theta_trace);

/* Lossless verification of the scheduled prefixes ([digest] overall cycle step 3,
 * [explainer] section 06 rule, eq. (8) for c*).
 *   target [R][gamma+1][V] (dt): target logits for draft positions 1..gamma and the
 *     bonus position gamma+1 (row l_r + 1 gives the bonus distribution).
 *   U [R][gamma][V] (dt), W2 [rank][V] (dt), bias_rows [R][gamma][rank] (double):
 *     q_j is recomputed from them as softmax(U_j + bias_j W2).
 *   x [R][gamma] drafted tokens, ell [R] scheduled lengths, req_ids as in the draft.
 * Outputs: n_acc [R]; y [R][gamma+1] emitted tokens (n_acc+1 valid, rest -1);
 *   c_star [R][gamma] (NaN for j > ell); pq_ratio [R][gamma] p_j(x_j)/q_j(x_j) and
 *   u_acc [R][gamma] the acceptance uniforms (both nullable, NaN where not tested);
 *   gap_blk, gap_in [R] for the final sample (nullable).
 * Returns 0 or -1. */
int ora_verify(int R, int gamma, int V, int rank, int dt, const void *target,
               const void *U, const void *W2, const double *bias_rows, const int32_t *x,
               const int32_t *ell, const int32_t *req_ids, uint64_t seed, uint64_t cycle,
               int32_t *n_acc, int32_t *y, double *c_star, double *pq_ratio, double *u_acc,
               double *gap_blk, double *gap_in);

/* Number of OpenMP threads the oracle uses (1 when built without OpenMP). */
int ora_num_threads(void);
/* Sets the number of OpenMP threads of later calls (n >= 1; no effect without OpenMP). */
void ora_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
