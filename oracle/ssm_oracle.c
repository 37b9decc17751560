/*
 * ssm_oracle.c -- plain fp64 CPU oracle for the state-mediated kernel of
 * diagonal-equivalent selective SSMs.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The GPU product path
 * never calls it and shares no code, header, table or helper with it.
 *
 * What it computes (one independent recurrence per (batch, head) slice):
 *
 *   h_t = A_t h_{t-1} + gamma_t B_t X_t + beta_t B_{t-1} X_{t-1}
 *   y_t = C_t^T h_t + D_h X_t
 *
 * following:
 *   - "When a Diagonal State Is Not Enough" (sungsoo.github.io), Part 01
 *     (definition: h_t = A_t h_{t-1} + B_t u_t, y_t = C_t h_t + D_t u_t) and
 *     Part 03 (selective recurrence h_t = Abar_t h_{t-1} + Bbar_t x_t; Theorem 24,
 *     which includes the initial state and the direct feedthrough);
 *   - the same page, Part 03 (Theorem 8): a commuting family diagonalizable over
 *     the reals gives real scalar modes; complex eigenvalues give rotating
 *     pairs, kept here as 2x2 blocks rho*R(theta);
 *   - the same page, Parts 03/08.3 and the arXiv abstract (mlinfo.pages.dev):
 *     SSD-MIMO writes R values per step (B_t is N x R, X_t is R x P) and reads
 *     O rows (C_t is N x O); HybridMamba mixes real per-coordinate-decay rows with
 *     complex rotating pairs and two-endpoint writes (x_{t-1}, x_t);
 *   - the same page, Part 08 section 3: HybridMamba mixes real static, real dynamic
 *     and complex dynamic rows.  Read here as: a static row's decay does not depend
 *     on the input (its per-token factor is exp(-A_{h,n}) whatever Delta_t is), a
 *     dynamic row's decay is exp(-Delta_t A_{h,n}); writes and readouts are the same
 *     for every row.
 *
 * The transition A_t is block diagonal:
 *   real row n < n_real:   a_t[n]  = exp(-Delta_t * A_{h,n})   (dynamic rows)
 *   static row n < n_static (the first n_static real rows):
 *                          a_t[n]  = exp(-A_{h,n}), the same at every token
 *   pair k (rows n_real+2k, n_real+2k+1):
 *                          rho_t   = exp(-Delta_t * Ac_{h,k}),
 *                          theta_t = Delta_t * omega_{h,k},
 *                          block   = rho_t * [[cos, -sin], [sin, cos]](theta_t)
 *   head decay mode: every row uses the single rate A_h (no pairs).
 *   Delta_t = softplus(dt_t) when the softplus flag is set, else dt_t.
 *
 * The reverse mode is the hand-derived adjoint of that recurrence
 * (g_t = C_t dy_t + A_{t+1}^T g_{t+1}), with the states h_{t-1} recomputed
 * from checkpoints taken every CKPT steps.  Everything is fp64; inputs arrive
 * as fp32 values (bf16 inputs are exactly representable in fp32).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#include "ssm_oracle.h"

#define CKPT 64

static double softplus(double v) { return v > 20.0 ? v : log1p(exp(v)); }
static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

/* One slice's inputs gathered into contiguous fp64 arrays. */
typedef struct {
  int T, N, P, R, O, n_real, n_pairs, n_static;
  int two_endpoint, has_D;
  double *x;     /* [T][R][P] */
  double *B;     /* [T][R][N] */
  double *C;     /* [T][O][N] */
  double *delta; /* [T]  (after softplus if flagged) */
  double *draw;  /* [T]  raw dt as given */
  double *beta;  /* [T]  (two-endpoint only) */
  double *gamma; /* [T]  (two-endpoint only; 1 otherwise) */
  double *rate;  /* [N]  decay rate per row (pairs: both rows share Ac_k) */
  double *omega; /* [n_pairs] */
  double D;
  /* two-endpoint carry: the previous call's last token (written at t = 0 with beta_0) */
  int has_prev;
  double *xprev; /* [R][P] */
  double *Bprev; /* [R][N] */
} slice_t;

static void gather_slice(const oracle_desc *d, int b, int h, const float *x, const float *B,
                         const float *C, const float *dt, const float *A, const float *omega,
                         const float *beta, const float *gamma, const float *D, slice_t *s) {
  const int T = d->seqlen, H = d->nheads, G = d->ngroups, P = d->headdim, N = d->dstate;
  const int R = d->rank_in, O = d->rank_out, g = h / (H / G);
  s->T = T; s->N = N; s->P = P; s->R = R; s->O = O;
  s->n_real = d->n_real; s->n_pairs = d->n_pairs; s->n_static = d->n_static;
  s->two_endpoint = d->two_endpoint; s->has_D = d->has_D;
  for (int t = 0; t < T; ++t) {
    const size_t bt = (size_t)b * T + t;
    for (int r = 0; r < R; ++r)
      for (int p = 0; p < P; ++p)
        s->x[((size_t)t * R + r) * P + p] = x[((bt * H + h) * R + r) * P + p];
    for (int r = 0; r < R; ++r)
      for (int n = 0; n < N; ++n)
        s->B[((size_t)t * R + r) * N + n] = B[((bt * G + g) * R + r) * N + n];
    for (int o = 0; o < O; ++o)
      for (int n = 0; n < N; ++n)
        s->C[((size_t)t * O + o) * N + n] = C[((bt * G + g) * O + o) * N + n];
    const double raw = dt[bt * H + h];
    s->draw[t] = raw;
    s->delta[t] = d->dt_softplus ? softplus(raw) : raw;
    s->beta[t] = d->two_endpoint ? beta[bt * H + h] : 0.0;
    s->gamma[t] = d->two_endpoint ? gamma[bt * H + h] : 1.0;
  }
  if (d->decay_mode == ORACLE_DECAY_HEAD) {
    for (int n = 0; n < N; ++n) s->rate[n] = A[h];
  } else {
    const int nr = d->n_real, np = d->n_pairs;
    for (int n = 0; n < nr; ++n) s->rate[n] = A[(size_t)h * (nr + np) + n];
    for (int k = 0; k < np; ++k) {
      s->rate[nr + 2 * k] = A[(size_t)h * (nr + np) + nr + k];
      s->rate[nr + 2 * k + 1] = A[(size_t)h * (nr + np) + nr + k];
    }
  }
  for (int k = 0; k < d->n_pairs; ++k) s->omega[k] = omega[(size_t)h * d->n_pairs + k];
  s->D = d->has_D ? D[h] : 0.0;
}

/* The token before the sequence (two-endpoint carry): x_prev [b][h][R][P], B_prev [b][g][R][N]. */
static void gather_prev(const oracle_desc *d, int b, int h, const float *x_prev,
                        const float *B_prev, slice_t *s) {
  const int H = d->nheads, G = d->ngroups, P = d->headdim, N = d->dstate, R = d->rank_in;
  const int g = h / (H / G);
  s->has_prev = d->two_endpoint && x_prev && B_prev;
  for (int r = 0; r < R; ++r) {
    for (int p = 0; p < P; ++p)
      s->xprev[(size_t)r * P + p] = s->has_prev ? x_prev[(((size_t)b * H + h) * R + r) * P + p] : 0.0;
    for (int n = 0; n < N; ++n)
      s->Bprev[(size_t)r * N + n] = s->has_prev ? B_prev[(((size_t)b * G + g) * R + r) * N + n] : 0.0;
  }
}

static slice_t alloc_slice(const oracle_desc *d) {
  slice_t s;
  const size_t T = d->seqlen;
  s.x = malloc(sizeof(double) * T * d->rank_in * d->headdim);
  s.B = malloc(sizeof(double) * T * d->rank_in * d->dstate);
  s.C = malloc(sizeof(double) * T * d->rank_out * d->dstate);
  s.delta = malloc(sizeof(double) * T);
  s.draw = malloc(sizeof(double) * T);
  s.beta = malloc(sizeof(double) * T);
  s.gamma = malloc(sizeof(double) * T);
  s.rate = malloc(sizeof(double) * d->dstate);
  s.omega = malloc(sizeof(double) * (d->n_pairs > 0 ? d->n_pairs : 1));
  s.has_prev = 0;
  s.xprev = calloc((size_t)d->rank_in * d->headdim, sizeof(double));
  s.Bprev = calloc((size_t)d->rank_in * d->dstate, sizeof(double));
  return s;
}

static void free_slice(slice_t *s) {
  free(s->x); free(s->B); free(s->C); free(s->delta); free(s->draw);
  free(s->beta); free(s->gamma); free(s->rate); free(s->omega); free(s->xprev); free(s->Bprev);
}

/* B and X of token t - 1 for the beta write of token t (the carried token at t = 0), or
   NULL when there is none. */
static const double *prev_B(const slice_t *s, int t, int r) {
  if (t > 0) return s->B + ((size_t)(t - 1) * s->R + r) * s->N;
  return s->has_prev ? s->Bprev + (size_t)r * s->N : NULL;
}
static const double *prev_X(const slice_t *s, int t, int r) {
  if (t > 0) return s->x + ((size_t)(t - 1) * s->R + r) * s->P;
  return s->has_prev ? s->xprev + (size_t)r * s->P : NULL;
}

/* The step a real row's decay takes at token t: Delta_t, or 1 on a static row. */
static double row_step(const slice_t *s, int t, int n) { return n < s->n_static ? 1.0 : s->delta[t]; }

/* h <- A_t h  (block-diagonal transition of step t). */
static void apply_transition(const slice_t *s, int t, double *h) {
  const int N = s->N, P = s->P, nr = s->n_real;
  const double dl = s->delta[t];
  for (int n = 0; n < nr; ++n) {
    const double a = exp(-row_step(s, t, n) * s->rate[n]);
    for (int p = 0; p < P; ++p) h[(size_t)n * P + p] *= a;
  }
  for (int k = 0; k < s->n_pairs; ++k) {
    const int i = nr + 2 * k, j = i + 1;
    const double rho = exp(-dl * s->rate[i]);
    const double th = dl * s->omega[k];
    const double c = cos(th), sn = sin(th);
    for (int p = 0; p < P; ++p) {
      const double hi = h[(size_t)i * P + p], hj = h[(size_t)j * P + p];
      h[(size_t)i * P + p] = rho * (c * hi - sn * hj);
      h[(size_t)j * P + p] = rho * (sn * hi + c * hj);
    }
  }
  (void)N;
}

/* h <- A_t^T h  (adjoint of the transition of step t). */
static void apply_transition_T(const slice_t *s, int t, double *h) {
  const int P = s->P, nr = s->n_real;
  const double dl = s->delta[t];
  for (int n = 0; n < nr; ++n) {
    const double a = exp(-row_step(s, t, n) * s->rate[n]);
    for (int p = 0; p < P; ++p) h[(size_t)n * P + p] *= a;
  }
  for (int k = 0; k < s->n_pairs; ++k) {
    const int i = nr + 2 * k, j = i + 1;
    const double rho = exp(-dl * s->rate[i]);
    const double th = dl * s->omega[k];
    const double c = cos(th), sn = sin(th);
    for (int p = 0; p < P; ++p) {
      const double gi = h[(size_t)i * P + p], gj = h[(size_t)j * P + p];
      h[(size_t)i * P + p] = rho * (c * gi + sn * gj);
      h[(size_t)j * P + p] = rho * (-sn * gi + c * gj);
    }
  }
}

/* h += gamma_t B_t X_t + beta_t B_{t-1} X_{t-1} */
static void add_write(const slice_t *s, int t, double *h) {
  const int N = s->N, P = s->P, R = s->R;
  for (int r = 0; r < R; ++r) {
    const double *Bt = s->B + ((size_t)t * R + r) * N;
    const double *Xt = s->x + ((size_t)t * R + r) * P;
    const double gm = s->gamma[t];
    for (int n = 0; n < N; ++n) {
      const double bn = gm * Bt[n];
      for (int p = 0; p < P; ++p) h[(size_t)n * P + p] += bn * Xt[p];
    }
    if (s->two_endpoint && prev_B(s, t, r)) {
      const double *Bp = prev_B(s, t, r);
      const double *Xp = prev_X(s, t, r);
      const double bt = s->beta[t];
      for (int n = 0; n < N; ++n) {
        const double bn = bt * Bp[n];
        for (int p = 0; p < P; ++p) h[(size_t)n * P + p] += bn * Xp[p];
      }
    }
  }
}

/* One forward step: h_{t-1} -> h_t. */
static void step(const slice_t *s, int t, double *h) {
  apply_transition(s, t, h);
  add_write(s, t, h);
}

/* y_t = C_t^T h_t + D X_t, into yt[O][P]. */
static void readout(const slice_t *s, int t, const double *h, double *yt) {
  const int N = s->N, P = s->P, O = s->O, R = s->R;
  for (int o = 0; o < O; ++o) {
    const double *Ct = s->C + ((size_t)t * O + o) * N;
    for (int p = 0; p < P; ++p) {
      double acc = 0.0;
      for (int n = 0; n < N; ++n) acc += Ct[n] * h[(size_t)n * P + p];
      if (s->has_D && O == R) acc += s->D * s->x[((size_t)t * R + o) * P + p];
      yt[(size_t)o * P + p] = acc;
    }
  }
}

static int check_desc(const oracle_desc *d) {
  if (d->batch < 0 || d->seqlen < 0 || d->nheads <= 0 || d->ngroups <= 0 || d->headdim <= 0 ||
      d->dstate <= 0 || d->rank_in <= 0 || d->rank_out <= 0)
    return -2;
  if (d->nheads % d->ngroups) return -2;
  if (d->decay_mode == ORACLE_DECAY_HEAD && (d->n_pairs != 0 || d->n_real != d->dstate)) return -2;
  if (d->n_static < 0 || d->n_static > d->n_real) return -2;
  if (d->decay_mode == ORACLE_DECAY_HEAD && d->n_static != 0) return -2;
  if (d->n_real + 2 * d->n_pairs != d->dstate) return -2;
  if (d->has_D && d->rank_in != d->rank_out) return -2;
  return 0;
}

int oracle_fwd(const oracle_desc *d, const float *x, const float *B, const float *C,
               const float *dt, const float *A, const float *omega, const float *beta,
               const float *gamma, const float *D, const double *h0, const float *x_prev,
               const float *B_prev, double *y, double *h_final, const int *slices,
               int n_slices) {
  int rc = check_desc(d);
  if (rc) return rc;
  const int T = d->seqlen, H = d->nheads, P = d->headdim, N = d->dstate, O = d->rank_out;
#pragma omp parallel for schedule(dynamic, 1)
  for (int si = 0; si < n_slices; ++si) {
    const int b = slices[2 * si], hh = slices[2 * si + 1];
    slice_t s = alloc_slice(d);
    gather_slice(d, b, hh, x, B, C, dt, A, omega, beta, gamma, D, &s);
    gather_prev(d, b, hh, x_prev, B_prev, &s);
    double *h = calloc((size_t)N * P, sizeof(double));
    double *yt = malloc(sizeof(double) * O * P);
    if (h0) memcpy(h, h0 + ((size_t)b * H + hh) * N * P, sizeof(double) * N * P);
    for (int t = 0; t < T; ++t) {
      step(&s, t, h);
      readout(&s, t, h, yt);
      for (int o = 0; o < O; ++o)
        for (int p = 0; p < P; ++p)
          y[((((size_t)b * T + t) * H + hh) * O + o) * P + p] = yt[(size_t)o * P + p];
    }
    if (h_final) memcpy(h_final + ((size_t)b * H + hh) * N * P, h, sizeof(double) * N * P);
    free(h); free(yt);
    free_slice(&s);
  }
  return 0;
}

int oracle_bwd(const oracle_desc *d, const float *x, const float *B, const float *C,
               const float *dt, const float *A, const float *omega, const float *beta,
               const float *gamma, const float *D, const double *h0, const float *x_prev,
               const float *B_prev, const float *dy, const double *dh_final, double *dx,
               double *dB, double *dC, double *ddt, double *dA_slices, double *domega_slices,
               double *dbeta, double *dgamma, double *dD_slices, double *dh0, double *dx_prev,
               double *dB_prev, const int *slices, int n_slices) {
  int rc = check_desc(d);
  if (rc) return rc;
  const int T = d->seqlen, H = d->nheads, G = d->ngroups, P = d->headdim, N = d->dstate;
  const int R = d->rank_in, O = d->rank_out, nr = d->n_real, np = d->n_pairs;
  const int nA = d->decay_mode == ORACLE_DECAY_HEAD ? 1 : nr + np;
#pragma omp parallel for schedule(dynamic, 1)
  for (int si = 0; si < n_slices; ++si) {
    const int b = slices[2 * si], hh = slices[2 * si + 1], g = hh / (H / G);
    slice_t s = alloc_slice(d);
    gather_slice(d, b, hh, x, B, C, dt, A, omega, beta, gamma, D, &s);
    gather_prev(d, b, hh, x_prev, B_prev, &s);
    const size_t NP = (size_t)N * P;
    const int nck = (T + CKPT - 1) / CKPT;
    /* checkpoints: state h_{c*CKPT - 1} entering segment c */
    double *ck = malloc(sizeof(double) * NP * (nck > 0 ? nck : 1));
    double *h = calloc(NP, sizeof(double));
    if (h0) memcpy(h, h0 + ((size_t)b * H + hh) * NP, sizeof(double) * NP);
    for (int t = 0; t < T; ++t) {
      if (t % CKPT == 0) memcpy(ck + (size_t)(t / CKPT) * NP, h, sizeof(double) * NP);
      step(&s, t, h);
    }
    /* seg[i] holds h_{t0-1+i}, i = 0..CKPT */
    double *seg = malloc(sizeof(double) * NP * (CKPT + 1));
    double *gs = calloc(NP, sizeof(double));   /* running adjoint */
    /* an upstream gradient of the final state enters as the adjoint after the last token */
    if (dh_final) memcpy(gs, dh_final + ((size_t)b * H + hh) * NP, sizeof(double) * NP);
    double *dxp = calloc((size_t)R * P, sizeof(double));  /* carried token's gradients */
    double *dBp = calloc((size_t)R * N, sizeof(double));
    double *dA_loc = calloc(nA, sizeof(double));
    double *dw_loc = calloc(np > 0 ? np : 1, sizeof(double));
    double dD_loc = 0.0;
    /* per-slice per-token outputs */
    double *dxs = calloc((size_t)T * R * P, sizeof(double));
    double *dBs = calloc((size_t)T * R * N, sizeof(double));
    double *dCs = calloc((size_t)T * O * N, sizeof(double));
    double *dDel = calloc(T > 0 ? T : 1, sizeof(double));
    double *dbs = calloc(T > 0 ? T : 1, sizeof(double));
    double *dgs = calloc(T > 0 ? T : 1, sizeof(double));
    for (int c = nck - 1; c >= 0; --c) {
      const int t0 = c * CKPT, t1 = (t0 + CKPT < T) ? t0 + CKPT : T;
      memcpy(seg, ck + (size_t)c * NP, sizeof(double) * NP);
      for (int t = t0; t < t1; ++t) {
        memcpy(seg + (size_t)(t - t0 + 1) * NP, seg + (size_t)(t - t0) * NP, sizeof(double) * NP);
        step(&s, t, seg + (size_t)(t - t0 + 1) * NP);
      }
      for (int t = t1 - 1; t >= t0; --t) {
        const double *ht = seg + (size_t)(t - t0 + 1) * NP;
        const double *hp = seg + (size_t)(t - t0) * NP;
        const float *dyt = dy + (((size_t)b * T + t) * H + hh) * O * P;
        /* g_t = C_t dy_t + A_{t+1}^T g_{t+1}  (gs already holds the second term) */
        for (int o = 0; o < O; ++o) {
          const double *Ct = s.C + ((size_t)t * O + o) * N;
          for (int n = 0; n < N; ++n)
            for (int p = 0; p < P; ++p) gs[(size_t)n * P + p] += Ct[n] * (double)dyt[o * P + p];
        }
        /* dC_t = h_t dy_t^T */
        for (int o = 0; o < O; ++o)
          for (int n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int p = 0; p < P; ++p) acc += ht[(size_t)n * P + p] * (double)dyt[o * P + p];
            dCs[((size_t)t * O + o) * N + n] = acc;
          }
        /* feedthrough: dX_t += D dy_t ; dD += <dy_t, X_t> */
        if (s.has_D && O == R) {
          for (int r = 0; r < R; ++r)
            for (int p = 0; p < P; ++p) {
              dxs[((size_t)t * R + r) * P + p] += s.D * (double)dyt[r * P + p];
              dD_loc += (double)dyt[r * P + p] * s.x[((size_t)t * R + r) * P + p];
            }
        }
        /* write of step t: gamma_t B_t X_t  and  beta_t B_{t-1} X_{t-1} */
        for (int r = 0; r < R; ++r) {
          const double *Bt = s.B + ((size_t)t * R + r) * N;
          const double *Xt = s.x + ((size_t)t * R + r) * P;
          double dgam = 0.0;
          for (int n = 0; n < N; ++n)
            for (int p = 0; p < P; ++p) {
              const double gv = gs[(size_t)n * P + p];
              dxs[((size_t)t * R + r) * P + p] += s.gamma[t] * Bt[n] * gv;
              dBs[((size_t)t * R + r) * N + n] += s.gamma[t] * gv * Xt[p];
              dgam += gv * Bt[n] * Xt[p];
            }
          dgs[t] += dgam;
          if (s.two_endpoint && prev_B(&s, t, r)) {
            const double *Bp = prev_B(&s, t, r);
            const double *Xp = prev_X(&s, t, r);
            /* token t - 1's gradients, or the carried token's at t = 0 */
            double *gx = t > 0 ? dxs + ((size_t)(t - 1) * R + r) * P : dxp + (size_t)r * P;
            double *gb = t > 0 ? dBs + ((size_t)(t - 1) * R + r) * N : dBp + (size_t)r * N;
            double dbet = 0.0;
            for (int n = 0; n < N; ++n)
              for (int p = 0; p < P; ++p) {
                const double gv = gs[(size_t)n * P + p];
                gx[p] += s.beta[t] * Bp[n] * gv;
                gb[n] += s.beta[t] * gv * Xp[p];
                dbet += gv * Bp[n] * Xp[p];
              }
            dbs[t] += dbet;
          }
        }
        /* transition of step t: parameter grads use h_{t-1} */
        double dl = 0.0;
        for (int n = 0; n < nr; ++n) {
          const double st = row_step(&s, t, n);
          const double a = exp(-st * s.rate[n]);
          double e = 0.0;
          for (int p = 0; p < P; ++p) e += gs[(size_t)n * P + p] * hp[(size_t)n * P + p];
          if (n >= s.n_static) dl += -s.rate[n] * a * e;  /* a static row ignores Delta */
          dA_loc[d->decay_mode == ORACLE_DECAY_HEAD ? 0 : n] += -st * a * e;
        }
        for (int k = 0; k < np; ++k) {
          const int i = nr + 2 * k, j = i + 1;
          const double rho = exp(-s.delta[t] * s.rate[i]);
          const double th = s.delta[t] * s.omega[k];
          const double cth = cos(th), sth = sin(th);
          double G2[2][2] = {{0, 0}, {0, 0}};
          for (int p = 0; p < P; ++p) {
            const double gi = gs[(size_t)i * P + p], gj = gs[(size_t)j * P + p];
            const double hi = hp[(size_t)i * P + p], hj = hp[(size_t)j * P + p];
            G2[0][0] += gi * hi; G2[0][1] += gi * hj;
            G2[1][0] += gj * hi; G2[1][1] += gj * hj;
          }
          /* R = [[c,-s],[s,c]],  R' = [[-s,-c],[c,-s]] */
          const double drho = G2[0][0] * cth - G2[0][1] * sth + G2[1][0] * sth + G2[1][1] * cth;
          const double dth =
              rho * (-G2[0][0] * sth - G2[0][1] * cth + G2[1][0] * cth - G2[1][1] * sth);
          dl += -s.rate[i] * rho * drho + s.omega[k] * dth;
          dA_loc[nr + k] += -s.delta[t] * rho * drho;
          dw_loc[k] += s.delta[t] * dth;
        }
        dDel[t] = dl;
        /* carry: g <- A_t^T g_t */
        apply_transition_T(&s, t, gs);
      }
    }
    /* scatter */
    for (int t = 0; t < T; ++t) {
      const size_t bt = (size_t)b * T + t;
      for (int r = 0; r < R; ++r)
        for (int p = 0; p < P; ++p)
          dx[((bt * H + hh) * R + r) * P + p] = dxs[((size_t)t * R + r) * P + p];
      /* dB, dC: slices are grouped so that one thread owns a whole (b, g) group
         only when H == G; otherwise accumulate with a critical section. */
      if (G == H) {
        for (int r = 0; r < R; ++r)
          for (int n = 0; n < N; ++n)
            dB[((bt * G + g) * R + r) * N + n] = dBs[((size_t)t * R + r) * N + n];
        for (int o = 0; o < O; ++o)
          for (int n = 0; n < N; ++n)
            dC[((bt * G + g) * O + o) * N + n] = dCs[((size_t)t * O + o) * N + n];
      }
      const double dd = dDel[t];
      ddt[bt * H + hh] = d->dt_softplus ? dd * sigmoid(s.draw[t]) : dd;
      if (dbeta) dbeta[bt * H + hh] = d->two_endpoint ? dbs[t] : 0.0;
      if (dgamma) dgamma[bt * H + hh] = d->two_endpoint ? dgs[t] : 0.0;
    }
    if (G != H) {
#pragma omp critical(oracle_group_accum)
      {
        for (int t = 0; t < T; ++t) {
          const size_t bt = (size_t)b * T + t;
          for (int r = 0; r < R; ++r)
            for (int n = 0; n < N; ++n)
              dB[((bt * G + g) * R + r) * N + n] += dBs[((size_t)t * R + r) * N + n];
          for (int o = 0; o < O; ++o)
            for (int n = 0; n < N; ++n)
              dC[((bt * G + g) * O + o) * N + n] += dCs[((size_t)t * O + o) * N + n];
        }
      }
    }
    /* per-slice parameter-gradient partials; the caller sums them in a fixed order */
    for (int i = 0; i < nA; ++i) dA_slices[(size_t)si * nA + i] = dA_loc[i];
    for (int k = 0; k < np; ++k) domega_slices[(size_t)si * np + k] = dw_loc[k];
    dD_slices[si] = dD_loc;
    if (dh0) memcpy(dh0 + ((size_t)b * H + hh) * NP, gs, sizeof(double) * NP);
    if (dx_prev)
      for (size_t i = 0; i < (size_t)R * P; ++i) dx_prev[((size_t)b * H + hh) * R * P + i] = dxp[i];
    if (dB_prev) {
      /* per group: the sum over its heads (accumulated; the caller zeroes it) */
#pragma omp critical(oracle_group_accum)
      for (size_t i = 0; i < (size_t)R * N; ++i) dB_prev[((size_t)b * G + g) * R * N + i] += dBp[i];
    }
    free(dxp); free(dBp);
    free(ck); free(h); free(seg); free(gs); free(dA_loc); free(dw_loc);
    free(dxs); free(dBs); free(dCs); free(dDel); free(dbs); free(dgs);
    free_slice(&s);
  }
  return 0;
}
