/*
 * ssm_oracle.h -- fp64 CPU oracle (TEST INFRASTRUCTURE ONLY).
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
 * load this.  It shares nothing with the GPU library.
 *
 * Array layouts (row-major, last index fastest), b = batch, t = time,
 * h = head, g = group (= h / (nheads / ngroups)):
 *   x     [b][t][h][r][p]     B  [b][t][g][r][n]     C  [b][t][g][o][n]
 *   dt, beta, gamma [b][t][h]
 *   A     head mode: [h]; coordinate mode: [h][n_real + n_pairs]
 *         (first n_real entries: real-row rates, the first n_static of them static rows;
 *         then one rate per pair)
 *   omega [h][n_pairs]        D [h]        h0, h_final, dh0, dh_final [b][h][n][p]
 *   x_prev, dx_prev [b][h][r][p], B_prev, dB_prev [b][g][r][n]: the token before the
 *         sequence (two-endpoint carry: its write beta_0 B_prev X_prev enters at token 0);
 *         NULL = none.  dh_final: upstream gradient of the final state (NULL = zero).
 *         dB_prev is accumulated (+=) per group and must be zeroed by the caller.
 *   y, dy [b][t][h][o][p]
 * Inputs are fp32 values, outputs fp64.  `slices` lists (b, h) pairs to
 * compute; outputs of other slices are left untouched.  With ngroups < nheads
 * dB and dC are accumulated (+=) and must be zeroed by the caller.
 * Per-slice parameter-gradient partials (dA, domega, dD) are written per
 * listed slice: dA_slices [n_slices][nA] (nA = 1 in head mode, else
 * n_real + n_pairs), domega_slices [n_slices][n_pairs], dD_slices [n_slices].
 * Returns 0, or -2 for an inconsistent descriptor.
 */
#ifndef SSM_ORACLE_H
#define SSM_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_DECAY_HEAD = 0, ORACLE_DECAY_COORD = 1 };

typedef struct {
  int batch, seqlen, nheads, ngroups, headdim, dstate, rank_in, rank_out;
  int n_real, n_pairs, decay_mode;
  int dt_softplus, two_endpoint, has_D;
  int n_static; /* the first n_static real rows decay by exp(-A) per token, whatever
                   Delta is (coordinate mode only; 0 = every real row is dynamic) */
} oracle_desc;

int oracle_fwd(const oracle_desc *d, const float *x, const float *B, const float *C,
               const float *dt, const float *A, const float *omega, const float *beta,
               const float *gamma, const float *D, const double *h0, const float *x_prev,
               const float *B_prev, double *y, double *h_final, const int *slices,
               int n_slices);

int oracle_bwd(const oracle_desc *d, const float *x, const float *B, const float *C,
               const float *dt, const float *A, const float *omega, const float *beta,
               const float *gamma, const float *D, const double *h0, const float *x_prev,
               const float *B_prev, const float *dy, const double *dh_final, double *dx,
               double *dB, double *dC, double *ddt, double *dA_slices, double *domega_slices,
               double *dbeta, double *dgamma, double *dD_slices, double *dh0, double *dx_prev,
               double *dB_prev, const int *slices, int n_slices);

#ifdef __cplusplus
}
#endif
#endif
