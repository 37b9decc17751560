/*
 * sanitize_driver.c -- runs the fp64 oracle (ssm_oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer (TEST INFRASTRUCTURE ONLY: built and run by
 * tests/test_oracle_sanitize.py on the host; nothing else loads it).
 *
 * It calls oracle_fwd and oracle_bwd on small problems that reach every branch of the
 * oracle's indexing: head and per-row decay, static real rows, rotating pairs,
 * two-endpoint writes with the carried previous token, an initial state and an upstream
 * gradient of the final state, head groups shared by several heads, different write and
 * readout ranks, a subset of the slices, length 1 and length 0.  The inputs are deterministic
 * pseudo-random values from a small linear congruential generator: the sanitizers, not
 * the values, are what this run checks.  Exit status 0 when every call returned 0 and
 * every output is finite.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include "ssm_oracle.h"

static unsigned long long rng_state = 12345;
static double uniform(void) {  /* Knuth's MMIX LCG, top 53 bits */
  rng_state = rng_state * 6364136223846793005ULL + 1442695040888963407ULL;
  return (double)(rng_state >> 11) / 9007199254740992.0;
}
static float *fill(size_t n, double lo, double hi) {
  float *a = malloc(sizeof(float) * (n ? n : 1));
  for (size_t i = 0; i < n; ++i) a[i] = (float)(lo + (hi - lo) * uniform());
  return a;
}
static double *fill64(size_t n) {
  double *a = malloc(sizeof(double) * (n ? n : 1));
  for (size_t i = 0; i < n; ++i) a[i] = uniform() - 0.5;
  return a;
}
static int finite_all(const double *a, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(a[i])) return 0;
  return 1;
}

static int run_case(oracle_desc d, int carry, int half_slices) {
  const size_t b = d.batch, T = d.seqlen, H = d.nheads, G = d.ngroups, P = d.headdim;
  const size_t N = d.dstate, R = d.rank_in, O = d.rank_out;
  const size_t nA = d.decay_mode == ORACLE_DECAY_HEAD ? 1 : (size_t)(d.n_real + d.n_pairs);
  float *x = fill(b * T * H * R * P, -1, 1), *B = fill(b * T * G * R * N, -1, 1);
  /* raw steps (softplus in the recurrence), or positive steps given directly */
  float *C = fill(b * T * G * O * N, -1, 1);
  float *dt = d.dt_softplus ? fill(b * T * H, -2.5, 0.5) : fill(b * T * H, 0.01, 0.3);
  float *A = fill(H * nA, 1, 16), *om = fill(H * (d.n_pairs ? d.n_pairs : 1), 0, 3.14);
  float *be = fill(b * T * H, 0, 1), *ga = fill(b * T * H, 0, 1), *D = fill(H, -1, 1);
  float *dy = fill(b * T * H * O * P, -1, 1);
  float *xp = carry ? fill(b * H * R * P, -1, 1) : NULL;
  float *bp = carry ? fill(b * G * R * N, -1, 1) : NULL;
  double *h0 = fill64(b * H * N * P), *dhf = carry ? fill64(b * H * N * P) : NULL;
  const size_t ns_all = b * H;
  const size_t ns = half_slices ? (ns_all + 1) / 2 : ns_all;
  int *sl = malloc(sizeof(int) * 2 * (ns ? ns : 1));
  for (size_t i = 0; i < ns; ++i) {
    const size_t k = half_slices ? 2 * i : i;
    sl[2 * i] = (int)(k / H);
    sl[2 * i + 1] = (int)(k % H);
  }
  double *y = calloc(b * T * H * O * P + 1, sizeof(double)), *hf = calloc(b * H * N * P + 1, sizeof(double));
  double *dx = calloc(b * T * H * R * P + 1, sizeof(double)), *dB = calloc(b * T * G * R * N + 1, sizeof(double));
  double *dC = calloc(b * T * G * O * N + 1, sizeof(double)), *ddt = calloc(b * T * H + 1, sizeof(double));
  double *dA = calloc(ns * nA + 1, sizeof(double)), *dw = calloc(ns * (d.n_pairs ? d.n_pairs : 1) + 1, sizeof(double));
  double *dbe = calloc(b * T * H + 1, sizeof(double)), *dga = calloc(b * T * H + 1, sizeof(double));
  double *dD = calloc(ns + 1, sizeof(double)), *dh0 = calloc(b * H * N * P + 1, sizeof(double));
  double *dxp = calloc(b * H * R * P + 1, sizeof(double)), *dbp = calloc(b * G * R * N + 1, sizeof(double));
  int rc = oracle_fwd(&d, x, B, C, dt, A, d.n_pairs ? om : NULL, d.two_endpoint ? be : NULL,
                      d.two_endpoint ? ga : NULL, d.has_D ? D : NULL, h0, xp, bp, y, hf, sl, (int)ns);
  if (rc == 0)
    rc = oracle_bwd(&d, x, B, C, dt, A, d.n_pairs ? om : NULL, d.two_endpoint ? be : NULL,
                    d.two_endpoint ? ga : NULL, d.has_D ? D : NULL, h0, xp, bp, dy, dhf, dx, dB,
                    dC, ddt, dA, dw, dbe, dga, dD, dh0, carry ? dxp : NULL, carry ? dbp : NULL,
                    sl, (int)ns);
  int ok = rc == 0;
  if (ok && !half_slices)
    ok = finite_all(y, b * T * H * O * P) && finite_all(hf, b * H * N * P) &&
         finite_all(dx, b * T * H * R * P) && finite_all(dB, b * T * G * R * N) &&
         finite_all(ddt, b * T * H) && finite_all(dh0, b * H * N * P) &&
         finite_all(dA, ns * nA) && finite_all(dxp, b * H * R * P) && finite_all(dbp, b * G * R * N);
  free(x); free(B); free(C); free(dt); free(A); free(om); free(be); free(ga); free(D); free(dy);
  free(xp); free(bp); free(h0); free(dhf); free(sl); free(y); free(hf); free(dx); free(dB);
  free(dC); free(ddt); free(dA); free(dw); free(dbe); free(dga); free(dD); free(dh0); free(dxp);
  free(dbp);
  return ok;
}

int main(void) {
  /* batch, seqlen, nheads, ngroups, headdim, dstate, rank_in, rank_out, n_real, n_pairs,
     decay_mode, dt_softplus, two_endpoint, has_D, n_static */
  const oracle_desc cases[] = {
      {2, 70, 3, 3, 5, 4, 1, 1, 4, 0, ORACLE_DECAY_HEAD, 1, 0, 1},
      {1, 130, 4, 2, 3, 6, 2, 2, 2, 2, ORACLE_DECAY_COORD, 1, 1, 1},
      {2, 65, 2, 1, 4, 8, 3, 2, 4, 2, ORACLE_DECAY_COORD, 0, 1, 0},
      {1, 1, 2, 2, 2, 4, 2, 1, 0, 2, ORACLE_DECAY_COORD, 1, 1, 0},
      {1, 0, 2, 2, 2, 4, 1, 1, 2, 1, ORACLE_DECAY_COORD, 1, 1, 1},
      {2, 9, 2, 2, 2, 6, 1, 3, 6, 0, ORACLE_DECAY_COORD, 1, 0, 0},
      /* static real rows next to dynamic rows and pairs */
      {1, 40, 2, 1, 3, 10, 2, 2, 4, 3, ORACLE_DECAY_COORD, 1, 1, 1, 2},
  };
  const int n = (int)(sizeof(cases) / sizeof(cases[0]));
  int failures = 0;
  for (int i = 0; i < n; ++i)
    for (int carry = 0; carry < 2; ++carry)
      for (int half = 0; half < 2; ++half)
        if (!run_case(cases[i], carry && cases[i].two_endpoint, half)) {
          fprintf(stderr, "case %d carry %d half %d failed\n", i, carry, half);
          ++failures;
        }
  printf("oracle sanitizer run: %d cases, %d failures\n", 4 * n, failures);
  return failures ? 1 : 0;
}
