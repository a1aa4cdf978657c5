/* Drives every oracle entry point once on small seeded inputs, for a build of the oracle
 * under AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_oracle_sanitize.py).
 * The values are arbitrary; what is checked is that no access leaves its buffer and no
 * operation is undefined.  Exit status 0 when every call returned as expected. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../oracle/oracle.h"

static uint64_t st = 0x9E3779B97F4A7C15ull;
static double unif(void) { /* xorshift64*, in [0, 1) */
  st ^= st >> 12; st ^= st << 25; st ^= st >> 27;
  return (double)((st * 0x2545F4914F6CDD1Dull) >> 11) * 0x1p-53;
}
static double gauss(void) { /* sum of 12 uniforms - 6: roughly N(0, 1) */
  double s = 0.0;
  for (int i = 0; i < 12; ++i) s += unif();
  return s - 6.0;
}
static uint16_t bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
static void *fill(size_t n, int dt, double scale) {
  if (dt == ORA_BF16) {
    uint16_t *p = malloc(2 * n);
    for (size_t i = 0; i < n; ++i) p[i] = bf16((float)(scale * gauss()));
    return p;
  }
  float *p = malloc(4 * n);
  for (size_t i = 0; i < n; ++i) p[i] = (float)(scale * gauss());
  return p;
}

#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                  \
    }                                                            \
  } while (0)

static int run(int dt) {
  const int R = 5, G = 3, V = 200, rk = 16, d = 24; /* V % 64 != 0: a short last block */
  void *U = fill((size_t)R * G * V, dt, 1.5), *h = fill((size_t)R * G * d, dt, 1.0);
  void *W1 = fill((size_t)V * rk, dt, 0.25), *W2 = fill((size_t)rk * V, dt, 0.25);
  void *Wg = fill((size_t)3 * rk * (2 * rk + d), dt, 0.15);
  void *tgt = fill((size_t)R * (G + 1) * V, dt, 1.5);
  float w[24 + 16], temps[3] = {1.0f, 1.5f, 0.7f};
  for (int i = 0; i < d + rk; ++i) w[i] = (float)(0.2 * gauss());
  int32_t x0[5], x[15], rid[5];
  for (int q = 0; q < R; ++q) { x0[q] = (int32_t)(unif() * V); rid[q] = 7 * q + 1; }
  double c[15], zc[15], lse[15], lx[15], br[15 * 16], gb[15], gi[15];
  CHECK(ora_draft_markov(R, G, V, rk, d, dt, U, h, W1, W2, w, temps, x0, rid, 3, 4, x, c, zc,
                         lse, lx, br, gb, gi) == 0);
  CHECK(ora_draft_rnn(R, G, V, rk, d, dt, U, h, W1, W2, Wg, w, NULL, x0, NULL, 3, 4, x, c, zc,
                      lse, lx, br, gb, gi) == 0);
  CHECK(ora_draft_markov(R, G, V, rk, 0, dt, U, NULL, W1, W2, w, NULL, x0, NULL, 3, 4, x, c,
                         NULL, lse, lx, br, NULL, NULL) == 0); /* d = 0 */
  x0[2] = V; /* a token out of range is rejected */
  CHECK(ora_draft_markov(R, G, V, rk, d, dt, U, h, W1, W2, w, NULL, x0, NULL, 3, 4, x, c, NULL,
                         lse, lx, br, NULL, NULL) == -1);
  x0[2] = 0;
  CHECK(ora_draft_markov(R, G, V, rk, d, dt, U, h, W1, W2, w, NULL, x0, NULL, 3, 4, x, c, NULL,
                         lse, lx, br, NULL, NULL) == 0);

  /* scheduler: every mode, the literal reading, traces */
  float cf[15], clag[15], a[15], sps[64];
  for (int i = 0; i < 15; ++i) { cf[i] = (float)c[i]; clag[i] = (float)unif(); }
  cf[4] = 0.0f; cf[7] = 1.0f;
  for (int B = 1; B <= 64; ++B) sps[B - 1] = 1.0f / (1.0f + 0.05f * B);
  int32_t ell[5];
  double stats[4], theta[16];
  for (int mode = 0; mode <= 2; ++mode)
    CHECK(ora_schedule(R, G, cf, mode == 2 ? clag : NULL, mode == 2 ? R : 0, sps, 1, 64, mode,
                       ell, a, stats, theta) == 0);
  CHECK(ora_schedule(R, G, cf, NULL, 0, sps, 1, 10, 0, ell, a, stats, NULL) == -2);
  CHECK(ora_schedule_literal(R, G, cf, sps, 1, 64, 1, ell, theta) == 0);
  CHECK(ora_schedule_literal(R, G, cf, sps, 1, 64, 0, ell, NULL) == 0);
  CHECK(ora_schedule(R, G, cf, NULL, 0, sps, 1, 64, 1, ell, NULL, NULL, NULL) == 0);

  /* verify on the drafted block: scheduled lengths, then all and none */
  int32_t nacc[5], y[20];
  double cs[15], pq[15], ua[15], vgb[5], vgi[5];
  CHECK(ora_verify(R, G, V, rk, dt, tgt, U, W2, br, x, ell, rid, 3, 4, nacc, y, cs, pq, ua, vgb,
                   vgi) == 0);
  for (int q = 0; q < R; ++q) ell[q] = G;
  CHECK(ora_verify(R, G, V, rk, dt, tgt, U, W2, br, x, ell, NULL, 3, 4, nacc, y, cs, NULL, NULL,
                   NULL, NULL) == 0);
  for (int q = 0; q < R; ++q) ell[q] = 0;
  CHECK(ora_verify(R, G, V, rk, dt, tgt, U, W2, br, x, ell, NULL, 3, 4, nacc, y, cs, pq, ua, vgb,
                   vgi) == 0);

  /* training forward on teacher-forced blocks */
  int32_t xs[15];
  for (int i = 0; i < 15; ++i) xs[i] = (int32_t)(unif() * V);
  const double alpha[3] = {0.1, 0.9, 1.0};
  double tcs[15], tc[15], lq[15], tv[15], loss[20];
  CHECK(ora_train_forward(R, G, V, rk, d, dt, U, h, W1, W2, w, tgt, x0, xs, alpha, tcs, tc, lq,
                          tv, loss) == 0);

  /* decode on a toy chain: every policy */
  const int Vt = 72, Gt = 3;
  void *Tb = fill((size_t)Vt * Vt, dt, 1.0), *Ub = fill((size_t)Vt * Gt * Vt, dt, 1.0);
  void *Hb = fill((size_t)Vt * Gt * d, dt, 1.0), *W1t = fill((size_t)Vt * rk, dt, 0.25);
  void *W2t = fill((size_t)rk * Vt, dt, 0.25);
  float spst[5 * 4];
  for (int B = 1; B <= 20; ++B) spst[B - 1] = 1.0f / (1.0f + 0.02f * B);
  int32_t toks[5 * 4 * 4], nem[5];
  int64_t dst[2 * 3 + 3];
  for (int q = 0; q < R; ++q) x0[q] = (int32_t)(unif() * Vt);
  for (int pol = 0; pol <= 4; ++pol)
    CHECK(ora_decode_run(R, Gt, Vt, rk, d, dt, 4, Ub, Hb, W1t, W2t, w, NULL, Tb, x0, pol, 0.3f,
                         spst, 1, 20, 9, toks, nem, dst) == 0);
  free(Tb); free(Ub); free(Hb); free(W1t); free(W2t);

  /* sampler edge cases */
  double l[130];
  for (int v = 0; v < 130; ++v) l[v] = -1.0 / 0.0;
  double g1, g2;
  CHECK(ora_sample_two_level(130, l, 0, 0, 0, 1, 0, 1, &g1, &g2) == -1);
  l[129] = 0.5;
  CHECK(ora_sample_two_level(130, l, 0, 0, 0, 1, 0, 1, &g1, &g2) == 129);
  int64_t counts[130] = {0};
  ora_sample_trials(130, l, 1, 2, 3, 4, 50, counts);
  CHECK(counts[129] == 50);

  free(U); free(h); free(W1); free(W2); free(Wg); free(tgt);
  return 0;
}

int main(void) {
  /* STS fit (dtype-free) */
  const int N = 300, G = 4;
  float *z = malloc(sizeof(float) * N * G), grid[5] = {0.5f, 1.0f, 1.5f, 2.0f, 3.0f}, T[4];
  int32_t *na = malloc(sizeof(int32_t) * N);
  for (int n = 0; n < N; ++n) {
    for (int k = 0; k < G; ++k) z[n * G + k] = (float)(1.5 + 2.0 * gauss());
    na[n] = (int32_t)(unif() * (G + 1));
  }
  double ece[4];
  if (ora_sts_fit(N, G, z, na, grid, 5, 15, T, ece) != 0) return 1;
  free(z);
  free(na);
  uint32_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, out[4];
  ora_philox4x32_10(ctr, key, out);
  if (run(ORA_F32) || run(ORA_BF16)) return 1;
  printf("oracle sanitizer run ok\n");
  return 0;
}
