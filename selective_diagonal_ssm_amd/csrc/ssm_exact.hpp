// ssm_exact.hpp -- token-by-token forward and reverse passes for the chunks whose per-row
// decay is too steep for the chunk-midpoint fold of the chunked kernels (gfx950).
//
// The per-row chunked kernels fold a row's decay into its operands around the chunk
// midpoint, q_t = C~_t e^{-A_n (CD_t - CD_end/2)} and k_s = K~_s e^{A_n (CD_s - CD_end/2)},
// so the intra-chunk product stays one MFMA contraction.  The folded factors reach
// e^{A_n CD_end / 2}: when a chunk's summed step times the largest rate of its rows
// passes kFoldLimit, those kernels flag the chunk and a kernel here redoes the work with
// the recurrence itself, whose factors are the decays a_t = e^{-A_n Delta_t} <= 1 (e^{-A_n}
// on a static row) and the pair rotations -- exact for any step:
//
//   ssm_fwd_exact  one workgroup per (slice, sequence segment, value-column block) whose
//                  segment holds a flagged chunk: h_t = A_t h_{t-1} + gamma_t B_t X_t +
//                  beta_t B_{t-1} X_{t-1}, y_t = C_t^T h_t + D X_t from the state entering
//                  the segment (h0, or the combined segment state, both formed with
//                  factors <= 1), writing y, the chunk-boundary states and h_final.
//   ssm_bwd_exact  persistent; for each flagged (slice, chunk) item the states of the
//                  chunk are rebuilt from the saved incoming state, and the adjoint
//                  g_t = C_t dy_t + A_{t+1}^T g_{t+1} runs backwards from the adjoint at
//                  the next chunk's first token (the boundary-adjoint sweep, also formed
//                  with factors <= 1), giving every per-token gradient of the chunk and
//                  the item's parameter-gradient partials.
//
// The adjoint and its parameter terms follow the reverse mode of the recurrence: with
// e_t[n] = sum_p g_t[n,p] h_{t-1}[n,p] on a real row, dDelta_t -= A_n a_t[n] e_t[n]; on a
// pair with G = sum_p g_t h_{t-1}^T (2 x 2), drho = <G, R(theta)>, dtheta = rho <G, R'(theta)>,
// dDelta_t += -A rho drho + omega dtheta.
//
// Sources: "When a Diagonal State Is Not Enough" (sungsoo.github.io), Part 01 (the
// recurrence h_t = A_t h_{t-1} + B_t u_t, y_t = C_t h_t + D_t u_t), Part 02 (per-coordinate
// dynamics weaken the common-mask optimisation of the chunked form), Part 03 (Theorem 8
// rotating pairs; the two-endpoint write), Part 04 (outputs, input and parameter
// gradients checked against a reference).
#pragma once
#include <algorithm>

#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

namespace ssm {

namespace {

// per-row rate (head rates: the head's one rate) and pair frequency
__device__ __forceinline__ float row_rate(const float* A, int h, int n, int nreal, int npairs,
                                          int head_rates) {
  if (head_rates) return A[h];
  const int na = nreal + npairs;
  return n < nreal ? A[(size_t)h * na + n] : A[(size_t)h * na + nreal + ((n - nreal) >> 1)];
}

// Per-token transition table of one token: real row n -> a_t[n]; the rows (n0, n0 + 1) of
// a pair -> (rho cos theta, rho sin theta).  A static row (n < nstatic) takes a unit step.
__device__ __forceinline__ void transition_entry(float* dst, int n, float delta,
                                                 const float* rate, const float* om,
                                                 int nreal, int nstatic) {
  if (n < nreal) {
    dst[n] = __expf(-rate[n] * (n < nstatic ? 1.f : delta));
  } else if (((n - nreal) & 1) == 0) {
    const float rho = __expf(-rate[n] * delta);
    float sn, cs;
    fast_sincos(om[(n - nreal) >> 1] * delta, &sn, &cs);
    dst[n] = rho * cs;
    dst[n + 1] = rho * sn;
  }
}

// (u0, u1) <- A (u0, u1) on rows (n0, n0 + 1) of one column: a pair turns by R(theta) and
// decays by rho; two real rows decay each by its own factor.  `tr` is the token's table.
__device__ __forceinline__ void apply_transition(float& u0, float& u1, const float* tr, int n0,
                                                 int nreal) {
  if (n0 >= nreal) {
    const float c = tr[n0], s = tr[n0 + 1];
    const float a = u0, b = u1;
    u0 = c * a - s * b;
    u1 = s * a + c * b;
  } else {
    u0 *= tr[n0];
    u1 *= tr[n0 + 1];
  }
}

// (u0, u1) <- A^T (u0, u1)
__device__ __forceinline__ void apply_transition_t(float& u0, float& u1, const float* tr, int n0,
                                                   int nreal) {
  if (n0 >= nreal) {
    const float c = tr[n0], s = tr[n0 + 1];
    const float a = u0, b = u1;
    u0 = c * a + s * b;
    u1 = -s * a + c * b;
  } else {
    u0 *= tr[n0];
    u1 *= tr[n0 + 1];
  }
}

}  // namespace

// ============================================================== forward
// Thread layout: TPC consecutive threads share a value column; thread q0 = tid % TPC of a
// column holds the row pairs q = q0 + TPC j (rows 2q, 2q + 1) of that column in
// registers, so a pair's rotation needs no exchange, and the readout's sum over rows is a
// TPC-lane DPP sum.  Tokens are staged in blocks of kExactTokens.
template <bool BF16, int N, int R, int TPC>
__global__ __launch_bounds__(256) void ssm_fwd_exact(FwdParams p, int qtk) {
  using T = typename Elem<BF16>::T;
  constexpr int PBX = 256 / TPC;                   // value columns per workgroup
  constexpr int MAXQ = (N / 2 + TPC - 1) / TPC;    // row pairs per thread
  constexpr int TB = kExactTokens;
  __shared__ float sRate[N], sOm[N / 2 + 1];
  __shared__ float sTr[TB][N];                     // per-token transition tables
  __shared__ float sB[(TB + 1) * R * N];           // rows of tokens t0 - 1 .. t0 + TB - 1
  __shared__ float sX[(TB + 1) * R * PBX];
  __shared__ float sC[TB * R * N];
  __shared__ float sGa[TB], sBe[TB];
  __shared__ float sY[TB * R * PBX];

  const int npx = p.P / PBX;
  const int unit = blockIdx.x / npx, px = blockIdx.x % npx;
  const int slice = unit / p.nseg, seg = unit % p.nseg;
  // a main-kernel workgroup of this (slice, segment) met a chunk too steep for the fold
  int wild = 0;
  for (int k = 0; k < p.npblk; ++k) wild |= p.wild[(size_t)unit * p.npblk + k];
  if (!wild) return;

  const int tid = threadIdx.x, q0 = tid % TPC, pl = tid / TPC;
  const int b = slice / p.H, h = slice % p.H, g = h / (p.H / p.G);
  const int L = p.L, H = p.H, G = p.G, P = p.P, nreal = p.n_real;
  const int rin = p.rin, rout = p.rout;
  const int col = px * PBX + pl;
  const int c0 = seg * p.cps, c1 = min(p.nchunks, c0 + p.cps);
  const int ta = c0 * qtk, tb = min(c1 * qtk, L);  // tokens [ta, tb)
  const bool te = p.beta != nullptr;

  for (int n = tid; n < N; n += 256) sRate[n] = row_rate(p.A, h, n, nreal, p.n_pairs, p.head_rates);
  for (int k = tid; k < p.n_pairs; k += 256) sOm[k] = p.omega[(size_t)h * p.n_pairs + k];

  const T* xg = static_cast<const T*>(p.x) + ((size_t)b * L * H + h) * rin * P;
  const T* Bg = static_cast<const T*>(p.B) + ((size_t)b * L * G + g) * rin * N;
  const T* Cg = static_cast<const T*>(p.C) + ((size_t)b * L * G + g) * rout * N;
  T* yg = static_cast<T*>(p.y) + ((size_t)b * L * H + h) * rout * P;
  const size_t tsB = (size_t)G * rin * N, tsC = (size_t)G * rout * N;
  const size_t tsX = (size_t)H * rin * P, tsY = (size_t)H * rout * P;
  const float* dtg = p.dt + (size_t)b * L * H + h;
  // the carried token before the sequence, or null
  const T* Bpv = p.B_prev ? static_cast<const T*>(p.B_prev) + ((size_t)b * G + g) * rin * N : nullptr;
  const T* xpv = p.x_prev ? static_cast<const T*>(p.x_prev) + ((size_t)b * H + h) * rin * P : nullptr;

  // the state entering the segment: h0, the combined segment state, or zero
  const float* hin = seg == 0 ? (p.h0 ? p.h0 + (size_t)slice * N * P : nullptr)
                              : p.seg_in + ((size_t)slice * p.nseg + seg) * N * P;
  float hs[MAXQ][2];
#pragma unroll
  for (int j = 0; j < MAXQ; ++j) {
    const int n0 = 2 * (q0 + TPC * j);
    hs[j][0] = (hin && n0 < N) ? hin[(size_t)n0 * P + col] : 0.f;
    hs[j][1] = (hin && n0 < N) ? hin[(size_t)(n0 + 1) * P + col] : 0.f;
  }
  T* saved = static_cast<T*>(p.saved);
  const size_t sl_saved = (size_t)slice * (p.save_nchunks + 1);
  auto save_state = [&](int slot) {
#pragma unroll
    for (int j = 0; j < MAXQ; ++j) {
      const int n0 = 2 * (q0 + TPC * j);
      if (n0 < N) {
        saved[((sl_saved + slot) * N + n0) * P + col] = from_f32<T>(hs[j][0]);
        saved[((sl_saved + slot) * N + n0 + 1) * P + col] = from_f32<T>(hs[j][1]);
      }
    }
  };
  if (saved && seg == 0) save_state(0);
  const float Dh = p.has_D ? p.D[h] : 0.f;

  for (int t0 = ta; t0 < tb; t0 += TB) {
    const int nt = min(TB, tb - t0);
    __syncthreads();  // the previous block is done with the staged rows
    for (int i = tid; i < (nt + 1) * R * N; i += 256) {
      const int tau = i / (R * N) - 1, r = (i / N) % R, n = i % N, t = t0 + tau;
      sB[i] = (t >= 0 && r < rin) ? to_f32(Bg[(size_t)t * tsB + r * N + n])
              : (t == -1 && r < rin && Bpv) ? to_f32(Bpv[r * N + n]) : 0.f;
    }
    for (int i = tid; i < (nt + 1) * R * PBX; i += 256) {
      const int tau = i / (R * PBX) - 1, r = (i / PBX) % R, c = i % PBX, t = t0 + tau;
      sX[i] = (t >= 0 && r < rin) ? to_f32(xg[(size_t)t * tsX + r * P + px * PBX + c])
              : (t == -1 && r < rin && xpv) ? to_f32(xpv[r * P + px * PBX + c]) : 0.f;
    }
    for (int i = tid; i < nt * R * N; i += 256) {
      const int tau = i / (R * N), o = (i / N) % R, n = i % N;
      sC[i] = o < rout ? to_f32(Cg[(size_t)(t0 + tau) * tsC + o * N + n]) : 0.f;
    }
    if (tid < nt) {
      const size_t idx = (size_t)(t0 + tid) * H;
      sGa[tid] = te ? p.gamma[(size_t)b * L * H + idx + h] : 1.f;
      sBe[tid] = te ? p.beta[(size_t)b * L * H + idx + h] : 0.f;
    }
    __syncthreads();
    for (int i = tid; i < nt * N; i += 256) {
      const int tau = i / N, n = i % N;
      const float raw = dtg[(size_t)(t0 + tau) * H];
      const float delta = p.softplus ? softplus_f32(raw) : raw;
      transition_entry(sTr[tau], n, delta, sRate, sOm, nreal, p.n_static);
    }
    __syncthreads();
    for (int tau = 0; tau < nt; ++tau) {
      const float ga = sGa[tau], be = sBe[tau];
      const float* bc = sB + (tau + 1) * R * N;  // B_t rows
      const float* bp = sB + tau * R * N;        // B_{t-1} rows
#pragma unroll
      for (int j = 0; j < MAXQ; ++j) {
        const int n0 = 2 * (q0 + TPC * j);
        if (n0 < N) {
          float u0 = hs[j][0], u1 = hs[j][1];
          apply_transition(u0, u1, sTr[tau], n0, nreal);
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const float xv = ga * sX[((tau + 1) * R + r) * PBX + pl];
            const float xq = be * sX[(tau * R + r) * PBX + pl];
            u0 += bc[r * N + n0] * xv + bp[r * N + n0] * xq;
            u1 += bc[r * N + n0 + 1] * xv + bp[r * N + n0 + 1] * xq;
          }
          hs[j][0] = u0;
          hs[j][1] = u1;
        }
      }
#pragma unroll
      for (int o = 0; o < R; ++o) {
        float part = 0.f;
#pragma unroll
        for (int j = 0; j < MAXQ; ++j) {
          const int n0 = 2 * (q0 + TPC * j);
          if (n0 < N) {
            const float* cr = sC + (tau * R + o) * N;
            part += cr[n0] * hs[j][0] + cr[n0 + 1] * hs[j][1];
          }
        }
        part = group_sum<TPC>(part);
        if (q0 == 0) sY[(tau * R + o) * PBX + pl] = part + Dh * sX[((tau + 1) * R + o) * PBX + pl];
      }
      const int t = t0 + tau;
      if (saved && ((t + 1) % p.save_chunk == 0 || t == L - 1)) save_state(t / p.save_chunk + 1);
    }
    __syncthreads();
    for (int i = tid; i < nt * rout * PBX; i += 256) {
      const int tau = i / (rout * PBX), o = (i / PBX) % rout, c = i % PBX;
      yg[(size_t)(t0 + tau) * tsY + o * P + px * PBX + c] = from_f32<T>(sY[(tau * R + o) * PBX + c]);
    }
  }
  if (seg == p.nseg - 1 && p.h_final) {
    float* hf = p.h_final + (size_t)slice * N * P;
#pragma unroll
    for (int j = 0; j < MAXQ; ++j) {
      const int n0 = 2 * (q0 + TPC * j);
      if (n0 < N) {
        hf[(size_t)n0 * P + col] = hs[j][0];
        hf[(size_t)(n0 + 1) * P + col] = hs[j][1];
      }
    }
  }
}

template <bool BF16, int N, int R>
void launch_fwd_exact(const FwdParams& p, int qtk, hipStream_t stream) {
  const int units = p.batch * p.H * p.nseg;
  if (units <= 0 || !p.wild) return;
  if (p.P % 64 == 0)
    hipLaunchKernelGGL((ssm_fwd_exact<BF16, N, R, 4>), dim3(units * (p.P / 64)), dim3(256), 0,
                       stream, p, qtk);
  else if (p.P % 32 == 0)
    hipLaunchKernelGGL((ssm_fwd_exact<BF16, N, R, 8>), dim3(units * (p.P / 32)), dim3(256), 0,
                       stream, p, qtk);
  else
    hipLaunchKernelGGL((ssm_fwd_exact<BF16, N, R, 16>), dim3(units * (p.P / 16)), dim3(256), 0,
                       stream, p, qtk);
}

// ============================================================== reverse
// Nothing to do unless the chunk-gradient kernel set the "any flagged" word.  Otherwise a
// workgroup walks a contiguous range of items, reads their flags 256 at a time and takes
// the flagged ones whole.  State-shaped values (h_{t-1},
// h_t, g_t) live in LDS as N x P fp32; the rebuilt states come from the saved incoming
// state by the recurrence in registers (thread layout as in the forward, all P columns),
// each reduction over value columns or rows is a plain loop of one thread per output.
template <bool BF16, int N, int P, int R, int QT>
__global__ __launch_bounds__(256) void ssm_bwd_exact(BwdParams p) {
  using T = typename Elem<BF16>::T;
  constexpr int TPC = 256 / P;
  constexpr int MAXQ = (N / 2 + TPC - 1) / TPC;
  static_assert(256 % P == 0 && TPC <= 16, "one workgroup covers every value column");
  __shared__ float sRate[N], sOm[N / 2 + 1];
  __shared__ float sTr[QT + 1][N];                 // transitions of tokens t0 .. t1 + 1
  __shared__ float sDl[QT + 1], sRaw[QT], sGa[QT + 1], sBe[QT + 1];
  __shared__ T sB[(QT + 1) * R * N], sX[(QT + 1) * R * P];  // tokens t0 - 1 .. t1
  __shared__ T sC[QT * R * N], sDY[QT * R * P];             // tokens t0 .. t1
  __shared__ float sH0[N * P], sH1[N * P], sG[N * P];       // h_{t-1}, h_t, g_t
  __shared__ float sV[R * N], sW[R * P];   // V_{t+1}[r][n] = g_{t+1}[n] . X_t[r], W_{t+1} = B_t g_{t+1}
  __shared__ float sE[N][2];               // per row: g_t[n] . h_{t-1}[n], g_t[n] . h_{t-1}[n ^ 1]
  __shared__ float sRed[3][256];
  __shared__ float sPart[2 * N + 2];       // item partials per row / pair, dD
  __shared__ int sFlag[256];

  const int tid = threadIdx.x, q0 = tid % TPC, col = tid / TPC;
  const int L = p.L, H = p.H, G = p.G, nreal = p.n_real, npairs = p.n_pairs;
  const int rin = p.rin, rout = p.rout, nch = p.nchunks;
  const int nitems = p.batch * H * nch;
  const bool te = p.beta != nullptr;
  const bool part = p.dBh != nullptr;
  const int GO = part ? H : G;

  if (*p.wild_any == 0) return;
  const int per = (nitems + gridDim.x - 1) / gridDim.x;
  const int i0 = blockIdx.x * per, i1 = min(nitems, i0 + per);
  for (int base = i0; base < i1; base += 256) {
    __syncthreads();
    sFlag[tid] = base + tid < i1 ? p.wild[base + tid] : 0;
    __syncthreads();
    for (int k = 0; k < 256; ++k) {
      if (!sFlag[k]) continue;
      const int item = base + k;
      const int slice = item / nch, c = item % nch;
      const int b = slice / H, h = slice % H, g = h / (H / G);
      const int t0 = c * QT, t1 = min(t0 + QT, L) - 1, nT = t1 - t0 + 1;
      const bool has_next = t1 + 1 < L;
      __syncthreads();  // the previous item is done with LDS
      for (int n = tid; n < N; n += 256) sRate[n] = row_rate(p.A, h, n, nreal, npairs, p.head_rates);
      for (int q = tid; q < npairs; q += 256) sOm[q] = p.omega[(size_t)h * npairs + q];
      for (int i = tid; i < 2 * N + 2; i += 256) sPart[i] = 0.f;
      if (tid <= nT) {  // token t0 + tid (tid = nT: the next chunk's first token)
        const int t = t0 + tid;
        const bool ok = tid < nT || has_next;
        const size_t idx = ((size_t)b * L + (ok ? t : t0)) * H + h;
        const float raw = ok ? p.dt[idx] : 0.f;
        sDl[tid] = ok ? (p.softplus ? softplus_f32(raw) : raw) : 0.f;
        if (tid < nT) sRaw[tid] = raw;
        sGa[tid] = (te && ok) ? p.gamma[idx] : (ok ? 1.f : 0.f);
        sBe[tid] = (te && ok) ? p.beta[idx] : 0.f;
      }
      for (int i = tid; i < (nT + 1) * R * N; i += 256) {
        const int tau = i / (R * N) - 1, r = (i / N) % R, n = i % N, t = t0 + tau;
        sB[i] = (t >= 0 && r < rin)
                    ? static_cast<const T*>(p.B)[((((size_t)b * L + t) * G + g) * rin + r) * N + n]
                : (t == -1 && r < rin && p.B_prev)
                    ? static_cast<const T*>(p.B_prev)[(((size_t)b * G + g) * rin + r) * N + n]
                    : from_f32<T>(0.f);
      }
      for (int i = tid; i < (nT + 1) * R * P; i += 256) {
        const int tau = i / (R * P) - 1, r = (i / P) % R, q = i % P, t = t0 + tau;
        sX[i] = (t >= 0 && r < rin)
                    ? static_cast<const T*>(p.x)[((((size_t)b * L + t) * H + h) * rin + r) * P + q]
                : (t == -1 && r < rin && p.x_prev)
                    ? static_cast<const T*>(p.x_prev)[(((size_t)b * H + h) * rin + r) * P + q]
                    : from_f32<T>(0.f);
      }
      for (int i = tid; i < nT * R * N; i += 256) {
        const int tau = i / (R * N), o = (i / N) % R, n = i % N, t = t0 + tau;
        sC[i] = o < rout ? static_cast<const T*>(p.C)[((((size_t)b * L + t) * G + g) * rout + o) * N + n]
                         : from_f32<T>(0.f);
      }
      for (int i = tid; i < nT * R * P; i += 256) {
        const int tau = i / (R * P), o = (i / P) % R, q = i % P, t = t0 + tau;
        sDY[i] = o < rout ? static_cast<const T*>(p.dy)[((((size_t)b * L + t) * H + h) * rout + o) * P + q]
                          : from_f32<T>(0.f);
      }
      // the adjoint at the next chunk's first token (after the last chunk: slot nch,
      // dh_final or zero)
      {
        const T* gn = static_cast<const T*>(p.gseg) + ((size_t)slice * (nch + 1) + c + 1) * N * P;
        for (int i = tid; i < N * P; i += 256) sG[i] = to_f32(gn[i]);
      }
      __syncthreads();
      for (int i = tid; i < (nT + 1) * N; i += 256) {
        const int tau = i / N, n = i % N;
        // past the sequence end there is no transition (step 0, and no static rows either)
        transition_entry(sTr[tau], n, sDl[tau], sRate, sOm, nreal, (tau < nT || has_next) ? p.n_static : 0);
      }
      // V_{t1+1} and W_{t1+1} from the next chunk's adjoint and token t1's X and B rows
      for (int i = tid; i < R * N; i += 256) {
        const int r = i / N, n = i % N;
        float v = 0.f;
        for (int q = 0; q < P; ++q) v += sG[n * P + q] * to_f32(sX[(nT * R + r) * P + q]);
        sV[i] = v;
      }
      for (int i = tid; i < R * P; i += 256) {
        const int r = i / P, q = i % P;
        float v = 0.f;
        for (int n = 0; n < N; ++n) v += to_f32(sB[(nT * R + r) * N + n]) * sG[n * P + q];
        sW[i] = v;
      }
      // the incoming state (saved by the forward in the io dtype), in registers
      float s_in[MAXQ][2];
      {
        const T* sv = static_cast<const T*>(p.saved) + ((size_t)slice * (nch + 1) + c) * N * P;
#pragma unroll
        for (int j = 0; j < MAXQ; ++j) {
          const int n0 = 2 * (q0 + TPC * j);
          s_in[j][0] = n0 < N ? to_f32(sv[(size_t)n0 * P + col]) : 0.f;
          s_in[j][1] = n0 < N ? to_f32(sv[(size_t)(n0 + 1) * P + col]) : 0.f;
        }
      }
      float dD = 0.f;
      __syncthreads();

      for (int tau = nT - 1; tau >= 0; --tau) {
        const int t = t0 + tau;
        // h_{t-1} and h_t, rebuilt from the incoming state
        float hs[MAXQ][2];
#pragma unroll
        for (int j = 0; j < MAXQ; ++j) { hs[j][0] = s_in[j][0]; hs[j][1] = s_in[j][1]; }
        for (int u = 0; u <= tau; ++u) {
          if (u == tau) {
#pragma unroll
            for (int j = 0; j < MAXQ; ++j) {
              const int n0 = 2 * (q0 + TPC * j);
              if (n0 < N) {
                sH0[n0 * P + col] = hs[j][0];
                sH0[(n0 + 1) * P + col] = hs[j][1];
              }
            }
          }
          const float ga = sGa[u], be = sBe[u];
#pragma unroll
          for (int j = 0; j < MAXQ; ++j) {
            const int n0 = 2 * (q0 + TPC * j);
            if (n0 < N) {
              float u0 = hs[j][0], u1 = hs[j][1];
              apply_transition(u0, u1, sTr[u], n0, nreal);
#pragma unroll
              for (int r = 0; r < R; ++r) {
                const float xv = ga * to_f32(sX[((u + 1) * R + r) * P + col]);
                const float xq = be * to_f32(sX[(u * R + r) * P + col]);
                u0 += to_f32(sB[((u + 1) * R + r) * N + n0]) * xv +
                      to_f32(sB[(u * R + r) * N + n0]) * xq;
                u1 += to_f32(sB[((u + 1) * R + r) * N + n0 + 1]) * xv +
                      to_f32(sB[(u * R + r) * N + n0 + 1]) * xq;
              }
              hs[j][0] = u0;
              hs[j][1] = u1;
            }
          }
        }
        // g_t = A_{t+1}^T g_{t+1} + C_t dy_t, in place (each thread its own entries)
#pragma unroll
        for (int j = 0; j < MAXQ; ++j) {
          const int n0 = 2 * (q0 + TPC * j);
          if (n0 < N) {
            sH1[n0 * P + col] = hs[j][0];
            sH1[(n0 + 1) * P + col] = hs[j][1];
            float u0 = sG[n0 * P + col], u1 = sG[(n0 + 1) * P + col];
            apply_transition_t(u0, u1, sTr[tau + 1], n0, nreal);
#pragma unroll
            for (int o = 0; o < R; ++o) {
              const float dv = to_f32(sDY[(tau * R + o) * P + col]);
              u0 += to_f32(sC[(tau * R + o) * N + n0]) * dv;
              u1 += to_f32(sC[(tau * R + o) * N + n0 + 1]) * dv;
            }
            sG[n0 * P + col] = u0;
            sG[(n0 + 1) * P + col] = u1;
          }
        }
        __syncthreads();
        const float ga = sGa[tau], ben = sBe[tau + 1];
        // dC_t[o][n] = h_t[n] . dy_t[o]
        for (int i = tid; i < rout * N; i += 256) {
          const int o = i / N, n = i % N;
          float v = 0.f;
          for (int q = 0; q < P; ++q) v += sH1[n * P + q] * to_f32(sDY[(tau * R + o) * P + q]);
          const size_t row = part ? (((size_t)b * L + t) * GO + h) * R + o
                                  : (((size_t)b * L + t) * GO + g) * rout + o;
          static_cast<T*>(part ? p.dCh : p.dC)[row * N + n] = from_f32<T>(v);
        }
        // dB_t = gamma_t g_t X_t^T + beta_{t+1} g_{t+1} X_t^T; the endpoint-weight sums
        float pg = 0.f, pb = 0.f;
        for (int i = tid; i < rin * N; i += 256) {
          const int r = i / N, n = i % N;
          float u = 0.f, v = 0.f;
          for (int q = 0; q < P; ++q) {
            const float gq = sG[n * P + q];
            u += gq * to_f32(sX[((tau + 1) * R + r) * P + q]);
            v += gq * to_f32(sX[(tau * R + r) * P + q]);
          }
          const float db = ga * u + ben * sV[i];
          const size_t row = part ? (((size_t)b * L + t) * GO + h) * R + r
                                  : (((size_t)b * L + t) * GO + g) * rin + r;
          static_cast<T*>(part ? p.dBh : p.dB)[row * N + n] = from_f32<T>(db);
          pg += to_f32(sB[((tau + 1) * R + r) * N + n]) * u;
          pb += to_f32(sB[(tau * R + r) * N + n]) * v;
          sV[i] = v;  // V_t for token t - 1 (read above as V_{t+1} by this same thread)
        }
        // dX_t = D dy_t + gamma_t B_t^T g_t + beta_{t+1} W_{t+1};  W_t = B_{t-1}^T g_t
        const float Dh = p.has_D ? p.D[h] : 0.f;
        for (int i = tid; i < rin * P; i += 256) {
          const int r = i / P, q = i % P;
          float u = 0.f, w = 0.f;
          for (int n = 0; n < N; ++n) {
            const float gq = sG[n * P + q];
            u += to_f32(sB[((tau + 1) * R + r) * N + n]) * gq;
            w += to_f32(sB[(tau * R + r) * N + n]) * gq;
          }
          const float dyv = p.has_D ? to_f32(sDY[(tau * R + r) * P + q]) : 0.f;
          const float dx = Dh * dyv + ga * u + ben * sW[i];
          static_cast<T*>(p.dx)[((((size_t)b * L + t) * H + h) * rin + r) * P + q] = from_f32<T>(dx);
          sW[i] = w;
          if (p.has_D) dD += dyv * to_f32(sX[((tau + 1) * R + r) * P + q]);
        }
        // per row: g_t[n] . h_{t-1}[n] and g_t[n] . h_{t-1}[n ^ 1]
        for (int n = tid; n < N; n += 256) {
          float e = 0.f, x = 0.f;
          for (int q = 0; q < P; ++q) {
            e += sG[n * P + q] * sH0[n * P + q];
            x += sG[n * P + q] * sH0[(n ^ 1) * P + q];
          }
          sE[n][0] = e;
          sE[n][1] = x;
        }
        sRed[0][tid] = pg;
        sRed[1][tid] = pb;
        __syncthreads();
        // step gradient: one thread per real row or pair adds its terms (row order)
        float ddl = 0.f;
        const float dl = sDl[tau];
        if (tid < N) {
          const int n = tid;
          if (n < nreal) {
            // a static row takes a unit step whatever Delta is: no step gradient
            const float a = sTr[tau][n], e = sE[n][0];
            const bool st = n < p.n_static;
            ddl = st ? 0.f : -sRate[n] * a * e;
            sPart[n] += -(st ? 1.f : dl) * a * e;
          } else if (((n - nreal) & 1) == 0) {
            const int k2 = (n - nreal) >> 1;
            const float cr = sTr[tau][n], sr = sTr[tau][n + 1];  // rho cos, rho sin
            // G[i][j] = g[row i] . h_{t-1}[row j] on the pair's rows (n, n + 1)
            const float g00 = sE[n][0], g01 = sE[n][1], g10 = sE[n + 1][1], g11 = sE[n + 1][0];
            // rho drho = <G, rho R>, dtheta = <G, rho R'>
            const float rdrho = g00 * cr - g01 * sr + g10 * sr + g11 * cr;
            const float dth = -g00 * sr - g01 * cr + g10 * cr - g11 * sr;
            ddl = -sRate[n] * rdrho + sOm[k2] * dth;
            sPart[n] += -dl * rdrho;
            sPart[N + k2] += dl * dth;
          }
        }
        sRed[2][tid] = ddl;
        __syncthreads();
        if (tid == 0) {
          float d = 0.f, dg = 0.f, db = 0.f;
          for (int i = 0; i < N; ++i) d += sRed[2][i];
          for (int i = 0; i < 256; ++i) { dg += sRed[0][i]; db += sRed[1][i]; }
          const size_t idx = ((size_t)b * L + t) * H + h;
          p.ddt[idx] = p.softplus ? d * sigmoid_f32(sRaw[tau]) : d;
          if (te && p.dgamma) p.dgamma[idx] = dg;
          if (te && p.dbeta) p.dbeta[idx] = db;
        }
      }
      // the item's parameter partials, in the layout of the chunk kernel's (thread 0 is
      // done reading the last token's sums first)
      __syncthreads();
      sRed[0][tid] = dD;
      __syncthreads();
      if (p.part && tid == 0) {
        const int na = p.head_rates ? 1 : nreal + npairs;
        float* dst = p.part + (size_t)item * p.npart;
        if (p.head_rates) {
          float v = 0.f;
          for (int n = 0; n < N; ++n) v += sPart[n];
          dst[0] = v;
        } else {
          for (int n = 0; n < nreal; ++n) dst[n] = sPart[n];
          for (int k2 = 0; k2 < npairs; ++k2) dst[nreal + k2] = sPart[nreal + 2 * k2];
        }
        for (int k2 = 0; k2 < npairs; ++k2) dst[na + k2] = sPart[N + k2];
        float d = 0.f;
        for (int i = 0; i < 256; ++i) d += sRed[0][i];
        dst[na + npairs] = d;
      }
    }
  }
}

template <bool BF16, int N, int P, int R, int QT>
void launch_bwd_exact(const BwdParams& p, int grid, hipStream_t stream) {
  const int items = p.batch * p.H * p.nchunks;
  if (items <= 0 || !p.wild) return;
  grid = std::max(1, std::min(grid, items));
  hipLaunchKernelGGL((ssm_bwd_exact<BF16, N, P, R, QT>), dim3(grid), dim3(256), 0, stream, p);
}

}  // namespace ssm
