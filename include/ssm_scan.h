/*
 * ssm_scan.h -- C ABI of the MI355X (gfx950) state-mediated selective SSM kernel.
 *
 * The operation (one independent recurrence per (batch, head) slice):
 *
 *   h_t = A_t h_{t-1} + gamma_t B_t X_t + beta_t B_{t-1} X_{t-1}
 *   y_t = C_t^T h_t + D_h X_t
 *
 * Sources: "When a Diagonal State Is Not Enough" (sungsoo.github.io), Part 01
 * (h_t = A_t h_{t-1} + B_t u_t, y_t = C_t h_t + D_t u_t) and Part 03 (selective
 * recurrence; Theorem 24: with time-shared token-local maps the state-mediated
 * kernel is unnormalized scalar-mode linear attention under a multiplicative
 * mask; Theorem 8: commuting transitions diagonalizable over the reals give real
 * scalar modes, complex eigenvalues give rotating pairs); Parts 03 and 08.3
 * (SSD-MIMO: R values written and O rows read per step, decay shared within a
 * head; HybridMamba: per-coordinate real rows, rotating pairs, two-endpoint
 * writes); arXiv abstract on mlinfo.pages.dev (same architectures, fused GPU
 * kernels timed forward + backward at SSM-core scope).
 *
 * Transition A_t (block diagonal, N = n_real + 2 n_pairs rows):
 *   real row n:  a_t[n] = exp(-Delta_t * A_{h,n})   (head mode: A_{h,n} = A_h)
 *   static row n < n_static (coordinate mode): a_t[n] = exp(-A_{h,n}), whatever Delta_t
 *                is -- the "real static" rows HybridMamba mixes with real dynamic and
 *                complex dynamic rows (same page, Part 08 section 3)
 *   pair k (rows n_real+2k, n_real+2k+1):
 *                rho_t = exp(-Delta_t * A_{h, n_real+k}),  theta_t = Delta_t * omega_{h,k},
 *                block = rho_t [[cos theta, -sin theta], [sin theta, cos theta]]
 *   Delta_t = softplus(dt_t) if SSM_F_DT_SOFTPLUS, else dt_t.
 *   Without SSM_F_TWO_ENDPOINT: beta = 0, gamma = 1.  h_{-1} = 0, B_{-1} X_{-1} = 0.
 *
 * Layouts: row-major, last index fastest; g = h / (nheads / ngroups).
 *   x   [batch][seqlen][nheads][rank_in][headdim]       (io dtype)
 *   B   [batch][seqlen][ngroups][rank_in][dstate]       (io dtype)
 *   C   [batch][seqlen][ngroups][rank_out][dstate]      (io dtype)
 *   y, dy [batch][seqlen][nheads][rank_out][headdim]    (io dtype)
 *   dt, beta, gamma, ddt, dbeta, dgamma [batch][seqlen][nheads]   (fp32)
 *   A   head mode [nheads]; coordinate mode [nheads][n_real + n_pairs] (fp32)
 *   omega [nheads][n_pairs], D [nheads]                           (fp32)
 *   dA, domega, dD: same shapes as A, omega, D (fp32)
 *   dx, dB, dC: same shapes and dtype as x, B, C.
 *
 * Ownership and behaviour:
 *   - Every pointer is a caller-owned DEVICE pointer, 16-byte aligned.  The
 *     library never allocates, frees or synchronizes; all work is enqueued on
 *     `stream` (a hipStream_t, NULL = default stream) and is asynchronous.
 *   - Validation happens before any launch; an error returns a negative status
 *     and enqueues nothing.  A failed launch returns SSM_ERR_HIP.
 *   - Outputs (including parameter gradients) are overwritten, never
 *     accumulated, and are bitwise reproducible run to run.
 *   - Optional pointers may be NULL: omega iff n_pairs == 0; beta and gamma iff
 *     SSM_F_TWO_ENDPOINT is clear; D iff SSM_F_HAS_D is clear (D requires
 *     rank_out == rank_in).  In the backward, a NULL gradient output is not
 *     computed; dx, dB, dC, ddt must be non-NULL.
 *   - rank_in (R) and rank_out (O) may differ ("SSD-MIMO" with different input
 *     and output widths); the scans tile with the larger of the two (at most 4)
 *     and treat the narrower side's missing rows as zero.
 *   - `saved` (ssm_saved_bytes(desc) bytes) receives the chunk-boundary states
 *     from the forward when non-NULL, stored in the io dtype (they enter the
 *     reverse pass's products in that dtype); ssm_scan_bwd requires the buffer a
 *     forward with the same descriptor and inputs filled.  Its contents are
 *     internal to the library.
 *   - State carry (all optional, fp32, [batch][nheads][N][P], 16-byte aligned):
 *     h0 is the state before token 0 (NULL = zero), h_final receives the state
 *     after the last token, dh0 receives dLoss/dh0 = A_0^T g_0.  The backward
 *     takes h0 through `saved` (the forward stores it as the first boundary
 *     state), so a forward with h0 must precede a backward that wants dh0 or
 *     the h0-dependent parts of the other gradients.  The two-endpoint term of
 *     token 0 (beta_0 B_{-1} X_{-1}) is zero unless the carried token x_prev /
 *     B_prev is given (see the args).
 *   - Empty problems (batch = 0 or seqlen = 0) read no inputs, and the pointers
 *     of empty tensors may be NULL.  The outputs that are not empty are still
 *     written: ssm_scan_fwd sets h_final to h0 (zero without h0);
 *     ssm_scan_bwd zeroes dA, domega, dD and dh0, the sums over no tokens.
 *   - `ws` is device scratch of at least ssm_workspace_bytes(desc, dir) bytes
 *     (may be NULL when that is 0).  Calls that share a workspace on one
 *     stream are ordered; concurrent calls need separate workspaces.
 *   - The library is thread-safe and keeps no per-call state.
 *   - Any step is valid: chunks whose per-row decay is too steep for the chunked
 *     kernels' folded operands are recomputed token by token on the GPU (the
 *     per-row scans therefore always need a small workspace for their flags).
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 6

typedef enum {
  SSM_OK = 0,
  SSM_ERR_NULL = -1,        /* a required pointer is NULL (or a forbidden one is set) */
  SSM_ERR_SHAPE = -2,       /* inconsistent sizes */
  SSM_ERR_DTYPE = -3,       /* unknown io dtype */
  SSM_ERR_ALIGN = -4,       /* pointer not 16-byte aligned */
  SSM_ERR_UNSUPPORTED = -5, /* valid but not implemented for this shape / mode */
  SSM_ERR_WORKSPACE = -6,   /* workspace smaller than ssm_workspace_bytes() */
  SSM_ERR_HIP = -7,         /* a HIP launch failed */
  SSM_ERR_SCRATCH = -8      /* ssm_scan_fwd_noalloc: the workspace the problem needs exceeds
                               the static scratch array (ssm_scratch_bytes()) */
} ssm_status;

typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype;

typedef enum {
  SSM_DECAY_HEAD = 0,  /* one rate per head (Mamba-2-style SSD); n_pairs must be 0 */
  SSM_DECAY_COORD = 1  /* one rate per real row and per pair (HybridMamba rows) */
} ssm_decay_mode;

enum {
  SSM_F_DT_SOFTPLUS = 1u,  /* Delta = softplus(dt) inside the kernel */
  SSM_F_TWO_ENDPOINT = 2u, /* write beta_t B_{t-1} X_{t-1} + gamma_t B_t X_t */
  SSM_F_HAS_D = 4u         /* add the feedthrough D_h X_t (rank_out == rank_in) */
};

typedef struct {
  int32_t batch, seqlen, nheads, ngroups;
  int32_t headdim;  /* P */
  int32_t dstate;   /* N = n_real + 2 n_pairs */
  int32_t rank_in;  /* R: values written per step */
  int32_t rank_out; /* O: rows read per step */
  int32_t n_real, n_pairs;
  int32_t chunk;    /* tokens per chunk; 0 = library's choice */
  int32_t io_dtype;   /* ssm_dtype: storage of x, B, C, y, dy, dx, dB, dC */
  int32_t decay_mode; /* ssm_decay_mode */
  uint32_t flags;     /* SSM_F_* */
  int32_t n_static;   /* coordinate mode: the first n_static real rows are static (decay
                         exp(-A) per token, no dependence on the step); 0 <= n_static <=
                         n_real, even; must be 0 in head mode */
} ssm_desc;

typedef struct {
  const void *x, *B, *C;
  const float *dt, *A, *omega, *beta, *gamma, *D;
  void *y;
  void *saved;  /* optional: chunk-boundary states for the backward */
  const float *h0;  /* optional: state before token 0 (NULL = zero) */
  float *h_final;   /* optional: receives the state after the last token */
  void *const *events; /* optional: 2 hipEvent_t recorded on `stream` before and after
                          the kernel (per-kernel timing); NULL = none, and a NULL entry
                          is not recorded */
  /* optional two-endpoint carry: the token before the sequence (x_prev
     [batch][nheads][rank_in][headdim], B_prev [batch][ngroups][rank_in][dstate], io
     dtype), whose write beta_0 B_prev x_prev enters at token 0; both or neither, and
     only with SSM_F_TWO_ENDPOINT.  A run continued with h0 = the previous call's h_final
     and these = its last token's x and B equals one run over both parts. */
  const void *x_prev, *B_prev;
} ssm_fwd_args;

typedef struct {
  const void *x, *B, *C, *dy;
  const float *dt, *A, *omega, *beta, *gamma, *D;
  const void *saved; /* filled by ssm_scan_fwd with the same inputs */
  void *dx, *dB, *dC;
  float *ddt, *dA, *domega, *dbeta, *dgamma, *dD;
  float *dh0;       /* optional: receives dLoss/dh0 */
  void *const *events; /* optional: 4 hipEvent_t recorded on `stream` around the three
                          kernels of the pass (boundary adjoints, chunk gradients,
                          parameter sums); NULL = none, and a NULL entry is not
                          recorded */
  /* optional carry across calls: x_prev / B_prev as given to the forward; dh_final, the
     upstream gradient of the forward's h_final (fp32 [batch][nheads][N][P], NULL =
     zero); dx_prev / dB_prev receive the carried token's gradients (shapes and dtype of
     x_prev / B_prev; dB_prev summed over a group's heads), which need x_prev / B_prev.
     Chained backwards (dh0 of a call -> dh_final of the call before it, dx_prev /
     dB_prev added to its last token) the calls give the gradients of one run. */
  const void *x_prev, *B_prev;
  const float *dh_final;
  void *dx_prev, *dB_prev;
} ssm_bwd_args;

/* Library ABI version (SSM_ABI_VERSION of the build). */
int ssm_abi_version(void);

/* Human-readable text for a status code (static storage). */
const char *ssm_status_string(int status);

/* Validate a descriptor without launching anything; returns SSM_OK or an error. */
int ssm_check_desc(const ssm_desc *desc);

/* Chunk length the library uses for this descriptor (after validation), or a
   negative status. */
int ssm_chunk_tokens(const ssm_desc *desc);

/* Bytes of the `saved` buffer (chunk-boundary states in the io dtype); 0 on an invalid
   descriptor. */
size_t ssm_saved_bytes(const ssm_desc *desc);

/* Device scratch needed by ssm_scan_fwd (for_backward = 0) or ssm_scan_bwd
   (for_backward = 1); 0 on an invalid descriptor. */
size_t ssm_workspace_bytes(const ssm_desc *desc, int for_backward);

/* Forward chunked scan: writes y (and `saved` when non-NULL).
   Steps of the method run on the GPU: chunk-local cumulative decay (wave
   prefix), rotation folding and two-endpoint write prologue, masked
   intra-chunk products on MFMA, chunk state and inter-chunk state passing kept
   in registers, readout + feedthrough + store. */
int ssm_scan_fwd(const ssm_desc *desc, const ssm_fwd_args *args, void *ws, size_t ws_bytes,
                 void *stream);

/* Fused reverse-mode pass: dx, dB, dC, ddt and the requested parameter
   gradients (dA, domega, dbeta, dgamma, dD), given dy and the forward's
   `saved` states.  It is the adjoint of the recurrence above (g_t = C_t dy_t +
   A_{t+1}^T g_{t+1}); "When a Diagonal State Is Not Enough", Part 04, checks the
   method by outputs, input gradients and parameter gradients alike, and the arXiv
   abstract times the kernels forward + backward.  When groups are shared by several heads (ngroups < nheads),
   dB and dC of a group are the sums over its heads, taken in a fixed head order
   from per-head partials in the workspace, so every call gives the same bits. */
int ssm_scan_bwd(const ssm_desc *desc, const ssm_bwd_args *args, void *ws, size_t ws_bytes,
                 void *stream);

/* ---------------------------------------------------------------- no allocation
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): ssm_scan_fwd with its workspace in
 * a static array inside the library instead of a caller buffer.  Same descriptor,
 * arguments, outputs and errors as ssm_scan_fwd; nothing is allocated or freed.
 *   - The array holds ssm_scratch_bytes() bytes (32 MiB) on every device the library
 *     runs on, from the device's first call until the process ends.  A problem whose
 *     forward workspace (ssm_workspace_bytes(desc, 0)) exceeds it is rejected with
 *     SSM_ERR_SCRATCH before anything is enqueued.
 *   - All calls on one device share that device's array, and it keeps the last call's
 *     contents (no call relies on them: every region a call reads is written by the
 *     same call first).  Calls that overlap in time on one device -- concurrent
 *     streams, or host threads -- race on it: order them on one stream.
 *   - The first call on a device looks up the array's device address (not a kernel
 *     launch); SSM_ERR_HIP if that fails. */
size_t ssm_scratch_bytes(void);
int ssm_scan_fwd_noalloc(const ssm_desc *desc, const ssm_fwd_args *args, void *stream);

/* ---------------------------------------------------------------- recurrent step
 * One token of the same recurrence, run step by step with a constant-size state
 * (the inference mode of "When a Diagonal State Is Not Enough", Part 01: the
 * state-space recurrence h_t = A_t h_{t-1} + B_t u_t, y_t = C_t h_t + D_t u_t, and
 * Part 03: its selective, rotating-pair and two-endpoint forms):
 *
 *   state <- A_t state + gamma_t B_t X_t + beta_t B_{t-1} X_{t-1}
 *   y_t    = C_t^T state + D_h X_t
 *
 * with A_t, Delta_t, beta, gamma and D exactly as in the scan above.  The
 * descriptor is the scan's with seqlen = 1 (chunk is ignored); rank_in and
 * rank_out may differ, each at most 8; headdim must be a multiple of 4 and at
 * most 1024; n_real must be even; and dstate * (1 + 2 rank_in + rank_out) +
 * 1024 rank_out must not exceed 16384 (the step's per-slice tables in LDS);
 * otherwise SSM_ERR_UNSUPPORTED.
 * Layouts (the scan's at seqlen = 1):
 *   x, x_prev [batch][nheads][rank_in][headdim]   B, B_prev [batch][ngroups][rank_in][dstate]
 *   C [batch][ngroups][rank_out][dstate]          y [batch][nheads][rank_out][headdim]
 *   dt, beta, gamma [batch][nheads]               A, omega, D as in the scan
 *   state [batch][nheads][dstate][headdim] fp32, read and overwritten in place
 *       (the layout of h0 / h_final: a scan's h_final continues as this state).
 * x_prev and B_prev (the previous token's x and B) are used only with
 * SSM_F_TWO_ENDPOINT, where both NULL means the first token (no previous write)
 * and otherwise both are set; without the flag both must be NULL.
 * Same ownership, alignment and error rules as the scan (state 16-byte aligned).
 * The step needs no workspace; y does not alias state. */
typedef struct {
  const void *x, *B, *C;
  const float *dt, *A, *omega, *beta, *gamma, *D;
  const void *x_prev, *B_prev;
  float *state;
  void *y;
} ssm_decode_args;

int ssm_decode_step(const ssm_desc *desc, const ssm_decode_args *args, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* SSM_SCAN_H */
