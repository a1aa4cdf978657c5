/*
 * dspark.h -- C ABI of the DSpark draft -> schedule -> verify hot path on MI355X (gfx950).
 *
 * The method ("DSpark: confidence-scheduled speculative decoding"; the technical digest
 * page, the interactive explainer page): a parallel backbone gives base logits U_k and
 * hidden states h_k for draft positions k = 1..gamma; a light sequential head adds a
 * prefix-dependent bias to U_k, samples x_k from one exact softmax and emits a confidence
 * c_k; a hardware-aware scheduler picks how many drafted tokens of each request the target
 * verifies; rejection sampling keeps the target's distribution exactly.
 *
 * Conventions shared by every entry point
 *   - Every array argument is a DEVICE pointer unless its comment says otherwise.  The
 *     caller owns all memory; the library never allocates, frees, retains a pointer or
 *     synchronises.  All work is enqueued on `stream` and the call returns at once.
 *   - Arrays are dense and row-major with the shapes given; element type "dt" means the
 *     dtype argument (DSPARK_F32: float, DSPARK_BF16: bfloat16 bit patterns).
 *   - A negative return value means the call was rejected on the host before anything was
 *     enqueued (DSPARK_EINVAL bad scalar, shape or null pointer; DSPARK_ERANGE a table that
 *     does not cover what the call needs; DSPARK_EWORKSPACE ws_bytes below the matching
 *     *_workspace_bytes(); DSPARK_EDEVICE a HIP error when launching).
 *   - Faults in device data (a token outside [0,V), a confidence that is NaN or outside
 *     [0,1], a length outside [0,gamma]) OR bits into *dev_status (nullable); the
 *     offending value is clamped so every access stays in bounds, and the outputs of that
 *     call are then unspecified.
 *   - Randomness is Philox4x32-10 keyed by `seed` (64 bits), with the counter
 *     (i >> 2, request, position, cycle << 4 | stream) and word i & 3; `cycle` < 2^28.
 *     Same inputs + (seed, cycle) give bit-identical outputs.
 *   - Sampling from softmax(l) is Gumbel-max taken in two levels: the block of 64
 *     consecutive ids with the largest log-sum-exp + Gumbel noise, then the id inside it
 *     with the largest l + Gumbel noise (exact in distribution).
 *   - Size limits (DSPARK_EINVAL otherwise): V % 8 == 0; r in {16,32,64,128,256};
 *     d % 8 == 0; 1 <= gamma <= 64; R >= 0 (R == 0 is a no-op); R*gamma <= 8192 for the
 *     scheduler; with bf16 operands U and the target logits below 4 GiB each.
 *   - Thread safety: the only global state is per-device caches of device attributes and
 *     of kernel launch settings, kept in atomics; concurrent calls on different streams
 *     with disjoint outputs and workspaces are safe.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { DSPARK_F32 = 0, DSPARK_BF16 = 1 } dspark_dtype;

typedef enum {
  /* Algorithm 1 as printed on the digest page (Module E): admit candidates in descending
   * prefix survival while Theta = tau * SPS(B) rises, stop at the first one that does not */
  DSPARK_SCHED_SYNC_BREAK = 0,
  /* the production variant without the break: the admitted count is the first one that
   * reaches the largest Theta over all prefixes of the sorted order (digest, production
   * deployment, first conflict) */
  DSPARK_SCHED_GLOBAL = 1,
  /* the asynchronous variant: the batch capacity comes from a GLOBAL search over the
   * confidences of two cycles before, the candidates are ranked by the current ones and
   * the top K = capacity - R are admitted (digest, production deployment, second conflict) */
  DSPARK_SCHED_ASYNC_LAG2 = 2
} dspark_sched_mode;

enum {
  DSPARK_OK = 0,
  DSPARK_EINVAL = -1,
  DSPARK_ERANGE = -2,
  DSPARK_EWORKSPACE = -3,
  DSPARK_EDEVICE = -4
};

/* bits OR-ed into *dev_status */
enum { DSPARK_FAULT_TOKEN = 1, DSPARK_FAULT_CONF = 2, DSPARK_FAULT_LEN = 4 };

/* ------------------------------------------------------------------------------------
 * W2 re-layout (digest, Module B eq. (5): the Markov head's bias is W1[x] W2 with
 * W2 in R^{r x V}).  The pages' W2 is [r][V] (row i holds coordinate i of every id); the
 * draft, verify, training and decode calls read it transposed, W2t [V][r] (row v holds
 * column v of W2, so a tile of consecutive ids is one contiguous run).  This call writes
 *   W2t[v][i] = W2[i][v]   for v < V, i < r
 * into caller memory (device pointers, V * r elements of dt each, not overlapping),
 * asynchronously on `stream`.  Once per weight load; exact (a copy).
 * DSPARK_EINVAL for V % 8 != 0, r outside {16,32,64,128,256}, a bad dt, a NULL or
 * aliased pointer.
 * ------------------------------------------------------------------------------------ */
int dspark_w2_relayout(int V, int r, dspark_dtype dt, const void *W2, void *W2t,
                       hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Benchmark hook (a measurement, not part of the method): reads `bytes` bytes at `buf`
 * (device memory, 16-byte aligned, bytes % 16 == 0) with `grid` workgroups of 256 threads,
 * each streaming its own contiguous slice, asynchronously on `stream`, and writes to
 * sink[b] (device, grid uint32 values) the XOR of the 32-bit words workgroup b read (so the
 * XOR of all of sink is the XOR of the whole buffer).  ev_begin / ev_end (both or neither;
 * events the caller created) are attached to the dispatch, which timestamps its own start
 * and end: their elapsed time is the kernel's duration, the read rate this device sustains,
 * the practical ceiling beside the published HBM peak.
 * DSPARK_EINVAL for a NULL pointer, a misaligned buffer or size, grid outside 1..65536, or
 * only one of the two events.
 * ------------------------------------------------------------------------------------ */
int dspark_read_probe(const void *buf, size_t bytes, int grid, uint32_t *sink,
                      hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end);

/* ------------------------------------------------------------------------------------
 * Draft (digest, Module B eq. (4) with the Markov head of eq. (5) or the RNN head of
 * eq. (6); confidence head eq. (7)).
 *
 * For every request q and k = 1..gamma (x_{q,0} = x0[q], the anchor, which is the first
 * predicted position per Module A):
 *   e            = W1[x_{q,k-1}]                                     (gather, r values)
 *   bias row     = e (Markov)  |  tanh(W_o z_k), z_k = [s_{k-1}; e; h_k] (RNN)
 *   l(v)         = U_k(v) + sum_i biasrow[i] * W2[i][v]              (never stored)
 *   lse[q][k]    = log sum_v exp l(v);   q_k = softmax(l)
 *   x[q][k]      = two-level Gumbel-max sample of q_k (streams 0, 1)
 *   logit_x      = l(x_k);  so q_k(x_k) = exp(logit_x - lse)
 *   z[q][k]      = sum_i w[i] h_k[i] + sum_i w[d+i] e[i]           (no bias term)
 *   c[q][k]      = sigmoid(z / T_k), T_k = temps[k-1] (the STS temperatures of Module D;
 *                  1 when temps is NULL)
 *
 * Inputs
 *   U   [R][gamma][V] dt   base logits U_1..U_gamma of the parallel backbone
 *   h   [R][gamma][d] dt   hidden states h_1..h_gamma
 *   W1  [V][r] dt          token embedding table (the low-rank factor W_1)
 *   W2t [V][r] dt          W_2 transposed: row v holds column v of W_2 in R^{r x V}
 *                          (the usual storage of an output projection; from the pages'
 *                          [r][V] layout by dspark_w2_relayout)
 *   w   [d + r] float      confidence weights, ordered [h part ; W1-row part]
 *   temps [gamma] float    per-position temperatures (> 0), or NULL; a value that is not
 *                          > 0 sets DSPARK_FAULT_CONF and that position uses 1
 *   x0  [R] int32          anchors
 * Outputs
 *   x, c, lse, logit_x [R][gamma] (int32, float, float, float)
 *   z [R][gamma] float (NULL: not written): the confidence logits before the temperature,
 *     the held-out data dspark_sts_fit calibrates on
 *   bias_rows [R][gamma][r]: the vector that multiplied W2 at each step, for verify;
 *     Markov: type dt (exact copy of W1 rows);  RNN: float.
 * Workspace: ws_bytes >= dspark_draft_workspace_bytes(...), any 256-byte aligned buffer.
 * ------------------------------------------------------------------------------------ */
size_t dspark_draft_workspace_bytes(int R, int gamma, int V, int r, int d);

int dspark_draft_markov(int R, int gamma, int V, int r, int d, dspark_dtype dt,
                        const void *U, const void *h, const void *W1, const void *W2t,
                        const float *w, const float *temps, const int32_t *x0, uint64_t seed,
                        uint64_t cycle, int32_t *x, float *c, float *z, float *lse,
                        float *logit_x, void *bias_rows, int32_t *dev_status, void *ws,
                        size_t ws_bytes, hipStream_t stream);

/* Benchmark hook: exactly dspark_draft_markov, and additionally records ev_begin[k-1] and
 * ev_end[k-1] (events the caller created, gamma of each) at the start and end of the
 * vocabulary-sweep kernel of draft position k, so that kernel can be timed alone with
 * hipEventElapsedTime: with bf16 operands the events are attached to the sweep's own
 * dispatch (its start and completion timestamps); with float operands they are recorded
 * on `stream` immediately before and after it.  A NULL entry (in either array) skips that
 * position.  DSPARK_EINVAL if either array is NULL. */
int dspark_draft_markov_timed(int R, int gamma, int V, int r, int d, dspark_dtype dt,
                              const void *U, const void *h, const void *W1, const void *W2t,
                              const float *w, const float *temps, const int32_t *x0,
                              uint64_t seed, uint64_t cycle, int32_t *x, float *c, float *z,
                              float *lse, float *logit_x, void *bias_rows, int32_t *dev_status,
                              void *ws, size_t ws_bytes, hipStream_t stream,
                              hipEvent_t *ev_begin, hipEvent_t *ev_end);

/* Allocation-free variant of dspark_draft_markov, for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Arguments and results are those of dspark_draft_markov without
 * ws / ws_bytes: the workspace is a library-owned device array of
 * dspark_draft_markov_noalloc_max_bytes() bytes (16 MiB), one per GPU, which that GPU holds
 * until the process ends.  The call allocates nothing.  DSPARK_ERANGE if the shapes need
 * more than that (dspark_draft_workspace_bytes(...) larger than the maximum; R = 512,
 * V = 151936, r = 256 needs about 8.3 MiB).  Every call on one GPU shares its array:
 * calls that overlap on one GPU (different streams, or host threads) race and must be
 * serialised by the caller; calls on one stream are ordered and safe. */
size_t dspark_draft_markov_noalloc_max_bytes(void);

int dspark_draft_markov_noalloc(int R, int gamma, int V, int r, int d, dspark_dtype dt,
                                const void *U, const void *h, const void *W1, const void *W2t,
                                const float *w, const float *temps, const int32_t *x0,
                                uint64_t seed, uint64_t cycle, int32_t *x, float *c, float *z,
                                float *lse, float *logit_x, void *bias_rows,
                                int32_t *dev_status, hipStream_t stream);

/* The parallel block's drafter alone, without the sequential head (the baseline the pages
 * compare the head against; digest, Module B, and the latency analysis of the sequential
 * module): x_k is sampled from softmax(U_k) itself (no bias; eq. (4) with the head's term
 * removed), with the same two-level sampler, random streams and outputs as
 * dspark_draft_markov (lse and logit_x of U_k; c and z from eq. (7) with W1[x_{k-1}];
 * bias_rows = W1[x_{k-1}]).  bf16 operands only (DSPARK_EINVAL otherwise); workspace as
 * dspark_draft_markov.  Timing it beside dspark_draft_markov gives the cost of the
 * sequential head. */
int dspark_draft_parallel(int R, int gamma, int V, int r, int d, dspark_dtype dt, const void *U,
                          const void *h, const void *W1, const float *w, const float *temps,
                          const int32_t *x0, uint64_t seed, uint64_t cycle, int32_t *x, float *c,
                          float *z, float *lse, float *logit_x, void *bias_rows,
                          int32_t *dev_status, void *ws, size_t ws_bytes, hipStream_t stream);

/* RNN head, eq. (6): W_gco [3r][2r + d] dt stacks the gate, candidate and output
 * projections (row blocks in that order; columns ordered [s ; W1 row ; h]; no biases);
 * s_0 = 0.  The bias row of step k is tanh(W_o z_k) with z_k holding s_{k-1}; c uses eq.
 * (7) with W1[x_{k-1}] unchanged.  bias_rows is float [R][gamma][r].  With bf16
 * operands, h (R * gamma * d * 2 bytes) must also stay below 4 GiB (DSPARK_EINVAL). */
size_t dspark_draft_rnn_workspace_bytes(int R, int gamma, int V, int r, int d);

int dspark_draft_rnn(int R, int gamma, int V, int r, int d, dspark_dtype dt, const void *U,
                     const void *h, const void *W1, const void *W2t, const void *W_gco,
                     const float *w, const float *temps, const int32_t *x0, uint64_t seed,
                     uint64_t cycle, int32_t *x, float *c, float *z, float *lse,
                     float *logit_x, float *bias_rows, int32_t *dev_status, void *ws,
                     size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Schedule (digest, Module E and Algorithm 1; production deployment for the variants).
 *   a[q][j]   = c[q][1] * ... * c[q][j] in float, left to right (prefix survival)
 *   E         = {(q,j) : a[q][j] > 0} in descending a (ties: q, then j, ascending)
 *   admitting the first n entries of E gives B_n = R + n and
 *   tau_n     = R + sum of their a, kept exactly as floor(a * 2^32) integer increments,
 *   Theta_n   = double(tau_fx_n) * 2^-32 * double(SPS(B_n)), one rounding.
 *   SYNC_BREAK: n = (first n >= 1 with Theta_n <= Theta_{n-1}) - 1, or |E|;
 *   GLOBAL: the smallest n with the largest Theta_n;
 *   ASYNC_LAG2: cap = R_lag + n_GLOBAL(c_lag); n = min(max(cap - R, 0), |E|).
 *   ell[q] = number of q's entries among the first n (always a prefix 1..ell[q]).
 * Inputs
 *   c [R][gamma] float in [0,1]; c_lag [R_lag][gamma] float (ASYNC_LAG2 only, else NULL)
 *   sps: DEVICE float table, SPS(B) = sps[B - sps_B0]; it must cover B = R .. R(1+gamma)
 *   (and R_lag .. R_lag(1+gamma) in ASYNC_LAG2), else DSPARK_ERANGE.
 * Outputs: ell [R] int32; a [R][gamma] float (nullable);
 *   stats [4] double (nullable) = {B, tau, Theta, n admitted}.
 * Workspace: ws of at least dspark_schedule_workspace_bytes(R, gamma) device bytes
 *   (DSPARK_EWORKSPACE otherwise; 0 for shapes beyond R * gamma <= 8192).  It needs no
 *   preparation (any contents on the first call) and may be captured in a graph: it holds an
 *   epoch word that each call advances, the workgroups' publications of that call, and in
 *   ASYNC_LAG2 each entry's admission rank and tau.  Calls sharing one workspace must not
 *   overlap.
 * ------------------------------------------------------------------------------------ */
size_t dspark_schedule_workspace_bytes(int R, int gamma);

int dspark_schedule(int R, int gamma, const float *c, const float *c_lag, int R_lag,
                    const float *sps, int sps_B0, int sps_len, dspark_sched_mode mode,
                    int32_t *ell, float *a, double *stats, int32_t *dev_status, void *ws,
                    size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Verify (digest, overall cycle step 3; explainer, section 06; eq. (8) for c*).
 * For each request q with scheduled length L = ell[q] and positions j = 1..L:
 *   p_j = softmax(target row j); q_j = softmax(U_j + bias_j W2) normalised by lse
 *   c_star[q][j] = 1 - 1/2 sum_v |p_j(v) - q_j(v)|   (NaN for j > L)
 *   x_j is accepted iff u < p_j(x_j) / q_j(x_j), u uniform (stream 2, index 0),
 *   with q_j(x_j) = exp(logit_x - lse) as drafted; the first rejection j* stops it.
 * If some j* <= L is rejected: emit x_1..x_{j*-1}, then a two-level Gumbel sample of
 *   max(0, p_j* - q_j*) (streams 3, 4; if that mass is 0 in floating point, of p_j*).
 * Otherwise: emit x_1..x_L, then a sample of target row L+1 (the bonus; streams 5, 6).
 * Inputs
 *   target [R][gamma+1][V] dt   target logits for positions 1..gamma+1
 *   U [R][gamma][V] dt, W2t [V][r] dt      as in draft
 *   bias_rows [R][gamma][r] of type bias_dt (as the draft wrote them)
 *   x, lse, logit_x [R][gamma]              draft outputs
 *   ell [R] int32                           schedule output (or any lengths in [0,gamma])
 * Outputs: n_acc [R] int32; y [R][gamma+1] int32 (first n_acc+1 valid, rest -1);
 *   c_star [R][gamma] float; x_next [R] int32 (nullable) = y[q][n_acc[q]], the last token
 *   emitted for q, from which q's next cycle drafts (its anchor x0; written by the kernel
 *   that draws it, so a cycle can pass it to the next draft call with no copy).
 * ------------------------------------------------------------------------------------ */
size_t dspark_verify_workspace_bytes(int R, int gamma, int V, int r);

int dspark_verify(int R, int gamma, int V, int r, dspark_dtype dt, const void *target,
                  const void *U, const void *W2t, const void *bias_rows,
                  dspark_dtype bias_dt, const int32_t *x, const float *lse,
                  const float *logit_x, const int32_t *ell, uint64_t seed, uint64_t cycle,
                  int32_t *n_acc, int32_t *y, float *c_star, int32_t *x_next,
                  int32_t *dev_status, void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Training objective, forward (digest, Module F, eqs. (8)-(12)), Markov head, on
 * teacher-forced blocks: position k of block q conditions on the reference token
 * x*_{k-1} (x*_0 = x0[q], x*_k = xstar[q][k-1]), so the R * gamma rows are independent.
 *   q_k    = softmax(U_k + W1[x*_{k-1}] W2);  p_k = softmax(target[q][k-1])
 *   tv     = sum_v |p_k(v) - q_k(v)|;  c_star = 1 - tv / 2                  (eq. (8))
 *   c      = sigmoid(w . [h_k ; W1[x*_{k-1}]])                              (eq. (7))
 *   logq   = log q_k(x*_k)
 *   w_k    = exp(-(k-1)/gamma)
 *   loss[q] = {L_ce, L_tv, L_conf, L}:  L_ce = -sum_k w_k logq,  L_tv = sum_k w_k tv,
 *            L_conf = sum_k w_k [c* softplus(-z) + (1 - c*) softplus(z)]
 *            (= -sum_k w_k [c* log c + (1 - c*) log(1 - c)]),
 *            L = a_ce L_ce + a_tv L_tv + a_conf L_conf   (the pages' mix: 0.1, 0.9, 1.0)
 * Inputs (device): U, h, W1, W2t, w as in dspark_draft_markov; target [R][gamma][V] dt;
 *   x0 [R], xstar [R][gamma] int32.  dt must be DSPARK_BF16 (float operands: EINVAL).
 * Outputs (device, each nullable): c_star, c, logq, tv [R][gamma] float;
 *   loss [R][4] float.  The batch objective is the mean of loss[:, 3].
 * A token out of range sets DSPARK_FAULT_TOKEN (token 0 is used in its place).
 * Workspace: ws_bytes >= dspark_train_forward_workspace_bytes(...) (0: sizes out of
 * range; R * gamma * V * 2 must stay below 4 GiB).
 * ------------------------------------------------------------------------------------ */
size_t dspark_train_forward_workspace_bytes(int R, int gamma, int V, int r, int d);

int dspark_train_forward(int R, int gamma, int V, int r, int d, dspark_dtype dt,
                         const void *U, const void *h, const void *W1, const void *W2t,
                         const float *w, const void *target, const int32_t *x0,
                         const int32_t *xstar, float a_ce, float a_tv, float a_conf,
                         float *c_star, float *c, float *logq, float *tv, float *loss,
                         int32_t *dev_status, void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Multi-cycle decode on a toy chain (digest, overall cycle; explainer, section 06), with
 * the pages' diagnostics.  The target is a bigram model: its logits after token t are row
 * t of Tb [V][V].  The parallel backbone is a table: for anchor a, U_k = Ub[a][k-1] and
 * h_k = Hb[a][k-1] (Ub [V][gamma][V], Hb [V][gamma][d]).  Each cycle c (random-counter
 * cycle c, key seed), for every request with anchor a (x0 at the start, then the last
 * emitted token):
 *   draft x_1..x_gamma (dspark_draft_markov, with temps);
 *   lengths by policy: SYNC_BREAK / GLOBAL / ASYNC_LAG2 as dspark_schedule (the lagged
 *     variant uses the confidences of cycle c-2, and the no-break search for c < 2);
 *     FIXED: every drafted position (scheduler off); THRESHOLD: the leading positions
 *     whose prefix survival c_1 ... c_j (fp32, left to right) is >= threshold;
 *   verify against Tb[a], Tb[x_1], ..., Tb[x_gamma] (dspark_verify);
 *   append the emitted tokens; the last becomes the anchor.
 * Outputs (device): tokens [R][ncycles*(gamma+1)] int32 (emitted tokens, -1 after the
 *   last), n_emitted [R], stats [2*gamma+3] int64: tested[k-1] = request-cycles in which
 *   position k was tested (k <= ell and positions 1..k-1 accepted), accepted[k-1] (at
 *   stats[gamma + k-1]) = those in which it was accepted, then the sum of ell, the tokens
 *   emitted and the request-cycles.  accepted/tested is the per-position conditional
 *   acceptance; sum of ell / request-cycles the mean verification budget.
 * Inputs: W1, W2t, w, temps as in dspark_draft_markov; sps (device) as in dspark_schedule
 *   (unused for FIXED and THRESHOLD; DSPARK_ERANGE if it does not cover R .. R(1+gamma)).
 * Workspace: ws_bytes >= dspark_decode_workspace_bytes(R, gamma, V, r, d, dt).
 * Tokens out of range set DSPARK_FAULT_TOKEN (token 0 is used in their place).  On an
 * error return the outputs are undefined.
 * ------------------------------------------------------------------------------------ */
typedef enum {
  DSPARK_DECODE_SYNC_BREAK = 0,
  DSPARK_DECODE_GLOBAL = 1,
  DSPARK_DECODE_ASYNC_LAG2 = 2,
  DSPARK_DECODE_FIXED = 3,
  DSPARK_DECODE_THRESHOLD = 4
} dspark_decode_policy;

size_t dspark_decode_workspace_bytes(int R, int gamma, int V, int r, int d, dspark_dtype dt);

int dspark_decode_run(int R, int gamma, int V, int r, int d, dspark_dtype dt, int ncycles,
                      const void *Ub, const void *Hb, const void *W1, const void *W2t,
                      const float *w, const float *temps, const void *Tb, const int32_t *x0,
                      dspark_decode_policy policy, float threshold, const float *sps,
                      int sps_B0, int sps_len, uint64_t seed, int32_t *tokens,
                      int32_t *n_emitted, int64_t *stats, int32_t *dev_status, void *ws,
                      size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * SPS(B) profiling (digest, Module E: the engine's steps per second against the
 * verification batch B, profiled once at start-up, looked up at run time).  The
 * verification pass stands in for the target engine.  For each B_list[i] (ascending,
 * R <= B <= R(1+gamma)) the lengths are spread so that R + sum(ell) = B
 * (ell[q] = floor((B-R)/R) + (q < (B-R) mod R)), dspark_verify runs once untimed and then
 * `reps` times between two events on `stream`, and
 *   sps_at[i] = reps / elapsed seconds   (HOST array [nB]).
 * The verify operands are as in dspark_verify; ell [R] (device) receives the last lengths
 * used; n_acc, y, c_star are verify's outputs (device, overwritten).  Unlike the other
 * calls this one SYNCHRONISES with the stream (once per profiled B).
 * DSPARK_ERANGE if a B lies outside [R, R(1+gamma)]; DSPARK_EINVAL for an unsorted list.
 * ------------------------------------------------------------------------------------ */
int dspark_sps_profile(int R, int gamma, int V, int r, dspark_dtype dt, const void *target,
                       const void *U, const void *W2t, const void *bias_rows,
                       dspark_dtype bias_dt, const int32_t *x, const float *lse,
                       const float *logit_x, int nB, const int *B_list, int reps,
                       float *sps_at, int32_t *ell, int32_t *n_acc, int32_t *y, float *c_star,
                       int32_t *dev_status, void *ws, size_t ws_bytes, hipStream_t stream);

/* The SPS table between profiled points (host only, no device): out[B - B0] for
 * B = B0 .. B1 is the linear interpolation of sps_at over B_list (ascending, sps_at > 0);
 * a B equal to a profiled point takes its value.  DSPARK_ERANGE unless
 * B_list[0] <= B0 <= B1 <= B_list[nB-1]. */
int dspark_sps_interpolate(int nB, const int *B_list, const float *sps_at, int B0, int B1,
                           float *out);

/* ------------------------------------------------------------------------------------
 * STS calibration (digest, Module D): per-position temperatures for the confidence head,
 * fitted left to right on held-out cycles.  For k = 1..gamma in order, with T_1..T_{k-1}
 * fixed, T_k is the grid entry minimising
 *   ECE_k(T) = sum_{b < nbins} | sum_{n : bin(P_n) = b} (o_n - P_n) | / N,
 *   P_n = prod_{j<k} sigmoid(z[n][j] / T_j) * sigmoid(z[n][k] / T),
 *   o_n = (n_acc[n] >= k),   bin(P) = min(floor(P * nbins), nbins - 1),
 * in double; ties go to the earlier grid entry.  Each (o - P) is added in fixed point with
 * 2^-38 resolution, so the bin sums (and the choice) do not depend on the launch shape.
 * Inputs (device unless noted)
 *   z     [N][gamma] float  confidence logits of drafted positions (dspark_draft_* `z`),
 *                           finite
 *   n_acc [N] int32         accepted length of each sample's verified block
 *   grid  [G] float, HOST   candidate temperatures, each finite and > 0
 *   1 <= N <= 2^24, 1 <= G <= 128, 1 <= nbins <= 256, G * nbins <= 4096
 * Outputs: T [gamma] float (device; usable as dspark_draft_* temps); ece [gamma] double
 *   (device, nullable): ECE_k at the chosen T_k.
 * Workspace: ws_bytes >= dspark_sts_workspace_bytes(N, G, nbins) (0: sizes out of range).
 * DSPARK_EINVAL for sizes or grid values out of range or a NULL required pointer.
 * ------------------------------------------------------------------------------------ */
size_t dspark_sts_workspace_bytes(int N, int G, int nbins);

int dspark_sts_fit(int N, int gamma, const float *z, const int32_t *n_acc, const float *grid,
                   int G, int nbins, float *T, double *ece, void *ws, size_t ws_bytes,
                   hipStream_t stream);

/* Library version string (static storage). */
const char *dspark_version(void);

#ifdef __cplusplus
}
#endif
#endif
