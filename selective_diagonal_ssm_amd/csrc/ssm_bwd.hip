// ssm_bwd.hip -- reverse-mode pass of the state-mediated selective SSM kernel (gfx950).
//
// The adjoint of  h_t = A_t h_{t-1} + W_t,  y_t = C_t^T h_t + D X_t  is
//   g_t = C_t dy_t + A_{t+1}^T g_{t+1}    (g_t = dL/dh_t),
// and every gradient of a chunk depends only on the state entering it (saved by
// the forward) and on g at the first token of the next chunk.  Three kernels:
//
//  ssm_bwd_adjoint  (reverse sweep, one workgroup per (slice, P-block)): the chunk
//      boundary adjoints Gpre[c] = g_{t0(c)} from
//        Gpre[c] = sum_{t in c} Phi_{t,t0}^T C_t dy_t + Phi_{t0',t0}^T Gpre[c+1],
//      Phi_{t,t0} = A_t ... A_{t0+1}; chunk-local folding as in the forward.
//  ssm_bwd_chunk    (persistent: each workgroup walks (slice, chunk) items, the
//      next item's reads in flight while the current one computes): dX, dB, dC,
//      dDelta, dbeta, dgamma and per-chunk parameter partials from the chunked
//      adjoint (transposed masked products on MFMA):
//        dV  = (S o M)^T dY + Ke G~,   dK~ = (Z o M)^T Q + e^{L_end-L_s} (G~ V^T),
//        dC~ = (Z o M) K + e^{L_t} dY S_in^T,   Z = dY V^T,
//      with G~ the folded adjoint of the chunk's final state.  The step gradient
//      uses the exact telescoping identity
//        d(log-decay)_r = sum_{t >= r} [C~_t . dC~_t - K~_t . dK~_t] (+ final-state term)
//      (row sum minus column sum of Z o S o M for the intra-chunk part), and the
//      pair angles the matching C~^T J dC~ + K~^T J dK~ terms (J = 90-degree
//      rotation).  The fp32 state operands (S_in, G~) enter the MFMAs rounded to the
//      io dtype, like the forward's readout copy of the state (a hi + lo split
//      measured 1.3e-4 against 2.6e-4 relative error on the step gradient at SSD SISO
//      shapes, for a third more products).
//  ssm_bwd_params   deterministic fixed-order sum of the per-chunk partials of
//      dA, domega, dD.
//
// Sources: "When a Diagonal State Is Not Enough" (sungsoo.github.io), Part 01 and
// Part 03 (recurrence, Theorem 24 masked-attention form, Theorem 8 pairs), Part 04
// (verification compares outputs, input gradients and parameter gradients).
#include <algorithm>
#include <atomic>

#include <type_traits>

#include "ssm_device.hpp"
#include "ssm_exact.hpp"
#include "ssm_kernels.hpp"
#include "ssm_local.hpp"

namespace ssm {

// ============================================================== boundary adjoints
template <bool BF16, int N, int PB, int R, int QT, bool COORD, int NTHREADS>
struct AdjShape {
  using T = typename Elem<BF16>::T;
  static constexpr int VEC = Elem<BF16>::kVec;
  static constexpr int PAD = 16 / static_cast<int>(sizeof(T));
  static constexpr int QO = QT * R;
  static constexpr int QOC = (QO + 31) / 32 * 32;  // contraction rows, zero padded
  static constexpr int NS = N + PAD;
  static constexpr int VS = PB + PAD;
  static constexpr int NTH = NTHREADS;
  static constexpr int NW = NTHREADS / 64;
  static constexpr int C_VECS = QO * (N / VEC);
  static constexpr int Y_VECS = QO * (PB / VEC);
  static constexpr int C_PER = (C_VECS + NTH - 1) / NTH;
  static constexpr int Y_PER = (Y_VECS + NTH - 1) / NTH;
  static constexpr int TN = N / 16, TP = PB / 16;
  static constexpr int ST_TILES = TN * TP;
  static constexpr int ST_PER_WAVE = (ST_TILES + NW - 1) / NW;
  // per-row decay: the dy vectors go to the threads after the C vectors' waves when both
  // fit once, so that the folding of C (exponentials, pair rotations) and the copy of dy run
  // on different waves (HybridMamba backward 0.564 -> 0.545 ms; with head decay both
  // stagings are light, and SSD-MIMO lost 2%)
  static constexpr int Y_T0 =
      (COORD && C_PER == 1 && Y_PER == 1 && (C_VECS + 63) / 64 * 64 + Y_VECS <= NTH)
          ? (C_VECS + 63) / 64 * 64 : 0;
};

template <bool BF16, int N, int PB, int R, int QT, bool COORD, int NTHREADS>
__global__ __launch_bounds__(NTHREADS) void ssm_bwd_adjoint(BwdParams p) {
  using S = AdjShape<BF16, N, PB, R, QT, COORD, NTHREADS>;
  constexpr int NW = S::NW;
  using T = typename S::T;
  constexpr int NS = S::NS, VS = S::VS, VEC = S::VEC;
  __shared__ __align__(16) T sQ[S::QOC * NS];  // folded, decayed C rows
  __shared__ __align__(16) T sY[S::QOC * VS];  // dy rows (head mode: decayed)
  // per-row rates: a dynamic row's in sRate (exponent rate x summed step), a static row's
  // in sRateS (exponent rate x token count)
  __shared__ float sRate[N], sRateS[N], sOmega[N / 2 + 1];
  // per-token scalars of chunk c in slot c & 1, formed by the last wave a chunk ahead: the
  // summed step over (t0, t] of each token, and over (t0, t0'] (to the next chunk's first
  // token) with the static rows' transition count
  __shared__ float sCdx[2][64], sCend[2][2];
  // per-row decay: the fold of chunk c's C rows, [token][n]: e^{-A_n d'_t} on real rows,
  // e^{-A d'_t} (cos, sin)(omega d'_t) on the rows of a pair; built by the upper half of
  // the workgroup during chunk c + 1's products
  __shared__ __align__(16) float sTC[COORD ? QT * N : 4];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // the chunk-gradient kernel that follows sets this word when a chunk is too steep for
  // its fold
  if (p.wild_any && blockIdx.x == 0 && tid == 0) *p.wild_any = 0;
  const int npblk = p.P / PB;
  const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const int slice = lid / (npblk * p.nseg), seg = (lid / npblk) % p.nseg, pblk = lid % npblk;
  const int c0 = seg * p.chunks_per_seg, c1 = min(p.nchunks, c0 + p.chunks_per_seg);
  const int b = slice / p.H, h = slice % p.H, g = h / (p.H / p.G);
  const int p0 = pblk * PB;
  const int L = p.L, H = p.H, G = p.G, P = p.P, nreal = p.n_real;

  if (COORD) {
    const int na = p.n_real + p.n_pairs;
    for (int n = tid; n < N; n += S::NTH) {
      float r;
      if (p.head_rates) r = p.A[h];
      else if (n < nreal) r = p.A[(size_t)h * na + n];
      else r = p.A[(size_t)h * na + nreal + ((n - nreal) >> 1)];
      const bool st = n < p.n_static;
      sRate[n] = st ? 0.f : r;
      sRateS[n] = st ? r : 0.f;
    }
    for (int k = tid; k < p.n_pairs; k += S::NTH) sOmega[k] = p.omega[(size_t)h * p.n_pairs + k];
  }
  for (int i = tid; i < (S::QOC - S::QO) * NS; i += S::NTH) sQ[S::QO * NS + i] = T(0);
  for (int i = tid; i < (S::QOC - S::QO) * VS; i += S::NTH) sY[S::QO * VS + i] = T(0);
  const float Ah = COORD ? 0.f : p.A[h];
  const T* Cg = static_cast<const T*>(p.C);
  const T* dyg = static_cast<const T*>(p.dy);

  // carried adjoint: zero past the sequence end, else (full pass of a segment) the
  // adjoint flowing in from the segments on the right
  // (the last segment: dh_final, the adjoint after the last token, or zero)
  const float* g_in = seg + 1 < p.nseg ? p.gin + ((size_t)slice * p.nseg + seg) * N * p.P + p0
                      : (p.dh_final ? p.dh_final + (size_t)slice * N * p.P + p0 : nullptr);
  // adjoint tiles, transposed: st[k][i] = G[n = 16 tn + (lane & 15)][p = 16 tp + 4 (lane >> 4) + i]
  // (one state row per lane, so each lane stores a 4-column piece; a pair's two rows
  // sit in lanes l, l ^ 1)
  f32x4 st[S::ST_PER_WAVE];
#pragma unroll
  for (int k = 0; k < S::ST_PER_WAVE; ++k) {
    st[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int tile = wave + NW * k;
    if (g_in && tile < S::ST_TILES) {
      const int n = 16 * (tile / S::TP) + (lane & 15), pl = 16 * (tile % S::TP) + 4 * (lane >> 4);
      const float4 v = *reinterpret_cast<const float4*>(g_in + (size_t)n * p.P + pl);
      st[k] = f32x4{v.x, v.y, v.z, v.w};
    }
  }
  // take these loads here: left pending into the chunk loop, they would make the
  // compiler wait on every outstanding memory operation inside it
#pragma unroll
  for (int k = 0; k < S::ST_PER_WAVE; ++k) asm volatile("" : "+v"(st[k]));

  const int nch = p.nchunks;
  if (seg == p.nseg - 1) {
    // boundary slot nch: the adjoint after the last token, read by the last chunk's gradients
#pragma unroll
    for (int k = 0; k < S::ST_PER_WAVE; ++k) {
      const int tile = wave + NW * k;
      if (tile < S::ST_TILES) {
        const int n = 16 * (tile / S::TP) + (lane & 15), pl = 16 * (tile % S::TP) + 4 * (lane >> 4);
        const float v4[4] = {st[k][0], st[k][1], st[k][2], st[k][3]};
        store4<BF16>(static_cast<T*>(p.gseg) + (((size_t)slice * (nch + 1) + nch) * N + n) * P + p0 + pl, v4);
      }
    }
  }
  // register prefetch of one chunk's C rows and dy rows
  uint4 pc[S::C_PER], py[S::Y_PER];
  auto prefetch = [&](int c) {
    const int t0 = c * QT;
#pragma unroll
    for (int k = 0; k < S::C_PER; ++k) {
      const int v = tid + S::NTH * k;
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (v < S::C_VECS) {
        const int row = v / (N / VEC), n0 = (v % (N / VEC)) * VEC;
        const int t = t0 + row / R, o = row % R;
        if (t < L && o < p.rout)
          raw = *reinterpret_cast<const uint4*>(Cg + ((((size_t)b * L + t) * G + g) * p.rout + o) * N + n0);
      }
      pc[k] = raw;
    }
#pragma unroll
    for (int k = 0; k < S::Y_PER; ++k) {
      const int v = (tid + S::NTH - S::Y_T0) % S::NTH + S::NTH * k;
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (v < S::Y_VECS) {
        const int row = v / (PB / VEC), pv = v % (PB / VEC);
        const int t = t0 + row / R, o = row % R;
        if (t < L && o < p.rout)
          raw = *reinterpret_cast<const uint4*>(dyg + ((((size_t)b * L + t) * H + h) * p.rout + o) * P + p0 + pv * VEC);
      }
      py[k] = raw;
    }
  };

  // The per-token scalars are formed once, by the last wave (SW), a chunk ahead: for chunk c
  // during chunk c + 1's staging, from steps read a chunk before that (held in sdt).  The
  // other waves only read them (the staging waves need them at once, and every wave used to
  // form them itself, all at the same moment).
  constexpr int SW = NW - 1;
  float dnext = 0.f;  // wave SW: step of the first token of the chunk after the one it forms
  auto load_dt = [&](int c) {
    float r = 0.f;
    if (c >= c0 && lane < QT && c * QT + lane < L) r = p.dt[((size_t)b * L + c * QT + lane) * H + h];
    return r;
  };
  auto form_scalars = [&](int c, float raw) {
    const int t0 = c * QT;
    float dl = 0.f;  // step of this chunk's tokens (lane = token)
    if (lane < QT && t0 + lane < L) dl = p.softplus ? softplus_f32(raw) : raw;
    const float cd = wave_prefix_sum(dl);
    const float cdx = cd - read_lane(dl, 0);               // sum over (t0, t]
    const float cdx_end = read_lane(cdx, QT - 1) + dnext;  // sum over (t0, t0']
    dnext = read_lane(dl, 0);
    if (lane < QT) sCdx[c & 1][lane] = cdx;
    if (lane == 0) {
      sCend[c & 1][0] = cdx_end;
      // static rows count the transitions instead: t - t0 over (t0, t], and over (t0, t0']
      // the chunk's tokens after the first plus the next chunk's first token
      sCend[c & 1][1] = static_cast<float>(min(QT, L - t0) - 1 + (t0 + QT < L ? 1 : 0));
    }
  };
  constexpr int TB0 = NTHREADS / 2;  // first thread of the fold-table builders
  auto build_table = [&](int c) {
    const float* cdxs = sCdx[c & 1];
    for (int i = tid - TB0; i < QT * (N / 2); i += NTHREADS - TB0) {
      const int t = i / (N / 2), n = 2 * (i % (N / 2));
      const float cdr = cdxs[t], cnr = static_cast<float>(t);
      float2 f;
      if (n >= nreal) {
        float sn, cs;
        fast_sincos(sOmega[(n - nreal) >> 1] * cdr, &sn, &cs);
        const float e = __expf(-sRate[n] * cdr);
        f = make_float2(e * cs, e * sn);
      } else {
        f = make_float2(__expf(-sRate[n] * cdr - sRateS[n] * cnr), __expf(-sRate[n + 1] * cdr - sRateS[n + 1] * cnr));
      }
      *reinterpret_cast<float2*>(sTC + t * N + n) = f;
    }
  };
  float sdt = 0.f;  // wave SW: raw steps of the chunk it forms next
  if (wave == SW) {
    if (c1 < nch) {
      const float raw = p.dt[((size_t)b * L + c1 * QT) * H + h];
      dnext = p.softplus ? softplus_f32(raw) : raw;
    }
    form_scalars(c1 - 1, load_dt(c1 - 1));
    sdt = load_dt(c1 - 2);
  }
  if (COORD) {
    __syncthreads();  // the first chunk's scalars (and the rates) before its fold table
    if (tid >= TB0) build_table(c1 - 1);
  }
  prefetch(c1 - 1);
  for (int c = c1 - 1; c >= c0; --c) {
    __syncthreads();  // the previous chunk's products are done with sQ / sY (and this chunk's
                      // scalars are formed)
    if (wave == SW && c > c0) form_scalars(c - 1, sdt);
    const float* cdxs = sCdx[c & 1];
    const float cdx_end = sCend[c & 1][0], cnx_end = sCend[c & 1][1];

    // operands: rows (t, o) of  e^{L'_t} R(-Theta'_t) C_t  and  dy_t
#pragma unroll
    for (int k = 0; k < S::C_PER; ++k) {
      const int v = tid + S::NTH * k;
      const int row = (v < S::C_VECS ? v : 0) / (N / VEC);
      if (v < S::C_VECS) {
        const int nv = v % (N / VEC), n0 = nv * VEC;
        uint4 raw = pc[k];
        if (COORD) {
          // times the fold table: per-row factors, or on a pair (a, b) the product
          // (a u0 + b u1, -b u0 + a u1)
          float vals[VEC], f[VEC];
          unpack<BF16>(raw, vals);
          const float* tab = sTC + (row / R) * N + n0;
#pragma unroll
          for (int i = 0; i < VEC; i += 4) {
            const float4 w = *reinterpret_cast<const float4*>(tab + i);
            f[i] = w.x; f[i + 1] = w.y; f[i + 2] = w.z; f[i + 3] = w.w;
          }
#pragma unroll
          for (int i = 0; i < VEC; i += 2) {
            const float a = vals[i], bb = vals[i + 1];
            if (n0 + i >= nreal) {
              vals[i] = f[i] * a + f[i + 1] * bb;
              vals[i + 1] = -f[i + 1] * a + f[i] * bb;
            } else {
              vals[i] = f[i] * a;
              vals[i + 1] = f[i + 1] * bb;
            }
          }
          raw = pack<BF16>(vals);
        }
        *reinterpret_cast<uint4*>(sQ + row * NS + n0) = raw;
      }
    }
#pragma unroll
    for (int k = 0; k < S::Y_PER; ++k) {
      const int v = (tid + S::NTH - S::Y_T0) % S::NTH + S::NTH * k;
      const int row = (v < S::Y_VECS ? v : 0) / (PB / VEC);
      const float wr = COORD ? 1.f : __expf(-Ah * cdxs[row / R]);
      if (v < S::Y_VECS) {
        const int pv = v % (PB / VEC);
        uint4 raw = py[k];
        if (!COORD) {
          float vals[VEC];
          unpack<BF16>(raw, vals);
#pragma unroll
          for (int i = 0; i < VEC; ++i) vals[i] *= wr;
          raw = pack<BF16>(vals);
        }
        *reinterpret_cast<uint4*>(sY + row * VS + pv * VEC) = raw;
      }
    }
    if (c > c0) prefetch(c - 1);  // in flight during this chunk's products
    if (wave == SW && c > c0) sdt = load_dt(c - 2);

    // carried adjoint: Gpre[c+1] -> Phi_{t0',t0}^T Gpre[c+1]
#pragma unroll
    for (int k = 0; k < S::ST_PER_WAVE; ++k) {
      const int tile = wave + NW * k;
      if (tile < S::ST_TILES) {
        const int n = 16 * (tile / S::TP) + (lane & 15);
        const float dec = COORD ? __expf(-sRate[n] * cdx_end - sRateS[n] * cnx_end) : __expf(-Ah * cdx_end);
#pragma unroll
        for (int i = 0; i < 4; ++i) st[k][i] *= dec;
        if (COORD) {
          // R(-theta) on the pair (n, n ^ 1) held by lanes (l, l ^ 1)
          const bool pair = n >= nreal;
          float sn = 0.f, cs = 1.f;
          if (pair) fast_sincos(sOmega[(n - nreal) >> 1] * cdx_end, &sn, &cs);
          const float sg = (lane & 1) ? -sn : sn;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float other = swap_adjacent_lanes(st[k][i]);
            st[k][i] = pair ? cs * st[k][i] + sg * other : st[k][i];
          }
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < S::ST_PER_WAVE; ++k) {
      const int tile = wave + NW * k;
      if (tile < S::ST_TILES) {
        const int tnn = tile / S::TP, tp = tile % S::TP;
        f32x4 acc = st[k];
#pragma unroll
        for (int kk = 0; kk < S::QOC / 32; ++kk) {
          const auto a = load_frag_tr<BF16>(sQ + (kk * 32) * NS + 16 * tnn, NS);
          const auto bq = load_frag_tr<BF16>(sY + (kk * 32) * VS + 16 * tp, VS);
          mma<BF16>(acc, bq, a);  // transposed: rows p, columns n
        }
        st[k] = acc;
        // the boundary adjoint in the io dtype (it enters the chunk products so)
        const int n = 16 * tnn + (lane & 15), pl = 16 * tp + 4 * (lane >> 4);
        T* dst = static_cast<T*>(p.gseg) + ((size_t)slice * (nch + 1) + c) * N * P;
        const float v4[4] = {acc[0], acc[1], acc[2], acc[3]};
        store4<BF16>(dst + (size_t)n * P + p0 + pl, v4);
      }
    }
    // the next chunk's fold table (its scalars were formed during this chunk's staging)
    if (COORD && c > c0 && tid >= TB0) build_table(c - 1);
  }
  // dLoss/dh0 = A_0^T g_0, with g_0 (the adjoint at token 0) now in st
  if (p.dh0 && seg == 0) {
    const float raw = p.dt[(size_t)b * L * H + h];
    const float d0 = p.softplus ? softplus_f32(raw) : raw;
    float* dst = p.dh0 + (size_t)slice * N * P + p0;
#pragma unroll
    for (int k = 0; k < S::ST_PER_WAVE; ++k) {
      const int tile = wave + NW * k;
      if (tile < S::ST_TILES) {
        const int n = 16 * (tile / S::TP) + (lane & 15), pl = 16 * (tile % S::TP) + 4 * (lane >> 4);
        const float dec = COORD ? __expf(-sRate[n] * d0 - sRateS[n]) : __expf(-Ah * d0);
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = st[k][i] * dec;
        if (COORD) {
          // R(-theta_0) = R(theta_0)^T on the pair held by lanes (l, l ^ 1)
          const bool pair = n >= nreal;
          float sn = 0.f, cs = 1.f;
          if (pair) fast_sincos(sOmega[(n - nreal) >> 1] * d0, &sn, &cs);
          const float sg = (lane & 1) ? -sn : sn;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float other = swap_adjacent_lanes(v[i]);
            v[i] = pair ? cs * v[i] + sg * other : v[i];
          }
        }
        *reinterpret_cast<float4*>(dst + (size_t)n * P + pl) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
  }
}

// ============================================================== adjoint segment combine
// Adjoints flowing into the segments of each slice, from the last one back: starting
// from zero after the sequence end, the local-pass ranges of segments nseg-1 .. 1 are
// chained right to left,
//   E <- rho_u R(-theta_u) E + G_loc[u],
// with rho_u = e^{-A_n D_u}, theta_u = omega_k D_u and D_u the summed step of range u's
// transition (the token-by-token transposed decays and rotations compose to exactly
// these); after the first range of segment s, E is the adjoint flowing into segment
// s - 1.  One thread per (slice, row pair, value column).
__global__ __launch_bounds__(256) void ssm_adj_combine(BwdParams p, int per_row) {
  const int N = p.n_real + 2 * p.n_pairs, P = p.P, nreal = p.n_real, na = p.n_real + p.n_pairs;
  const long total = (long)p.batch * p.H * (N / 2) * P;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
    const int pp = (int)(i % P);
    const long r = i / P;
    const int n = 2 * (int)(r % (N / 2));
    const long slice = r / (N / 2);
    const int h = (int)(slice % p.H);
    auto rate = [&](int m) {
      if (!per_row || p.head_rates) return p.A[h];
      return m < nreal ? p.A[(size_t)h * na + m] : p.A[(size_t)h * na + nreal + ((m - nreal) >> 1)];
    };
    const float ra = rate(n), rb = rate(n + 1);
    // static rows (n_static is even, so both rows of the pair (n, n + 1) are of one kind)
    // decay once per token: over a range, the number of transitions it spans
    const bool stat = per_row && n < p.n_static;
    const bool pair = per_row && n >= nreal;
    const float om = pair ? p.omega[(size_t)h * p.n_pairs + ((n - nreal) >> 1)] : 0.f;
    const size_t sb = (size_t)slice * p.nseg, sl = (size_t)slice * (p.nseg - 1) * p.nsub;
    // the adjoint after the last token: dh_final, or zero
    float a = 0.f, bv = 0.f;
    if (p.dh_final) {
      a = p.dh_final[((size_t)slice * N + n) * P + pp];
      bv = p.dh_final[((size_t)slice * N + n + 1) * P + pp];
    }
    for (int s = p.nseg - 1; s >= 1; --s) {
      // ranges (last first) in blocks of kCombineBlock: a block's reads are issued
      // together, then chained (one memory round trip per block instead of per range)
      for (int u0 = p.nsub - 1; u0 >= 0; u0 -= kCombineBlock) {
        const int cnt = min(kCombineBlock, u0 + 1);
        float ds[kCombineBlock], l0[kCombineBlock], l1[kCombineBlock];
#pragma unroll
        for (int k = 0; k < kCombineBlock; ++k) {
          const size_t unit = sl + (size_t)(s - 1) * p.nsub + u0 - (k < cnt ? k : 0);
          const float* loc = p.gloc + (unit * N + n) * P + pp;
          ds[k] = p.gdel[unit];
          l0[k] = loc[0];
          l1[k] = loc[P];
        }
#pragma unroll
        for (int k = 0; k < kCombineBlock; ++k) {
          if (k >= cnt) break;
          float dsum = ds[k];
          if (stat) {
            // range u0 - k of segment s: the transitions of its tokens after the first and
            // of the token after it (when inside the sequence)
            const int ta = s * p.seg_tokens + (u0 - k) * p.lsub;
            const int tb = min(min(ta + p.lsub, (s + 1) * p.seg_tokens), p.L) - 1;
            dsum = tb >= ta ? static_cast<float>(tb - ta + (tb + 1 < p.L ? 1 : 0)) : 0.f;
          }
          float a2 = a * expf(-ra * dsum), b2 = bv * expf(-rb * dsum);
          if (pair) {
            float sn, cs;
            sincosf(om * dsum, &sn, &cs);
            const float x0 = a2, x1 = b2;
            a2 = cs * x0 + sn * x1;  // R(-theta) = R(theta)^T
            b2 = -sn * x0 + cs * x1;
          }
          a = a2 + l0[k];
          bv = b2 + l1[k];
        }
      }
      float* out = p.gin + ((sb + s - 1) * N + n) * P + pp;
      out[0] = a;
      out[P] = bv;
    }
  }
}

// ============================================================== chunk gradients
// fixed-order sum of per-wave slots
template <int NW, typename A>
__device__ __forceinline__ float wsum(const A& arr, int i) {
  float v = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) v += arr[w][i];
  return v;
}
template <int NW>
__device__ __forceinline__ float wsum1(const float* arr) {
  float v = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) v += arr[w];
  return v;
}

template <bool BF16, int N, int P, int R, int KR, int QT, bool COORD, int NTHREADS>
struct BwdShape {
  using T = typename Elem<BF16>::T;
  static constexpr int VEC = Elem<BF16>::kVec;
  static constexpr int PAD = 16 / static_cast<int>(sizeof(T));
  static constexpr int NC = N < 32 ? 32 : N;
  static constexpr int PC = P < 32 ? 32 : P;
  static constexpr int QO = QT * R;
  static constexpr int QOC = (QO + 31) / 32 * 32;
  static constexpr int QK = QT * KR;
  static constexpr bool TE = KR > R;
  static constexpr int TEH = TE ? 1 : 0;
  static constexpr int NS = NC + PAD;   // [row][n] buffers
  static constexpr int PS = PC + PAD;   // [row][p] buffers
  static constexpr int KS = QK + PAD;   // [row][key] buffers
  static constexpr int BROWS = (QT + TEH) * R;
  static constexpr int NTH = NTHREADS;
  static constexpr int NW = NTHREADS / 64;
  static constexpr int C_VECS = QO * (N / VEC);
  static constexpr int B_VECS = BROWS * (N / VEC);
  static constexpr int X_VECS = BROWS * (P / VEC);
  static constexpr int Y_VECS = QO * (P / VEC);
  static constexpr int TQ = QO / 16, TK = QK / 16, TN = N / 16, TP = P / 16;
  // score tiles (16 query rows ti x 16 keys tj) holding at least one causal entry
  static constexpr int row_tiles(int ti) {
    const int c = (((16 * ti + 15) / R) * KR) / 16 + 1;
    return c < TK ? c : TK;
  }
  // two-endpoint writes: the last key tile too, for every query tile (its last key group
  // holds the halo row, which enters at the chunk's first token)
  static constexpr bool extra_tile(int ti) { return TE && row_tiles(ti) < TK; }
  static constexpr int score_tiles() {
    int n = 0;
    for (int ti = 0; ti < TQ; ++ti) n += row_tiles(ti) + (extra_tile(ti) ? 1 : 0);
    return n;
  }
  static constexpr int SC_TILES = score_tiles();
  // dK~ and dC~ tiles in 2 x 2 blocks per wave where there are at least four tiles
  // per wave anyway
  static constexpr bool KBLK = TN % 2 == 0 && TK % 2 == 0 && TN * TK >= 4 * NW;
  static constexpr bool CBLK = TN % 2 == 0 && TQ % 2 == 0 && TN * TQ >= 4 * NW;
  // exactly two tiles per wave otherwise: a wave takes them as one 1 x 2 block (one
  // n-block, two key / query blocks), so the n-block's fragments serve both
  static constexpr bool KPAIR = !KBLK && TK % 2 == 0 && TN * TK == 2 * NW;
  static constexpr bool CPAIR = !CBLK && TQ % 2 == 0 && TN * TQ == 2 * NW;
  static_assert(QO % 16 == 0 && QK % 32 == 0, "chunk rows must fill MFMA tiles");
  static_assert(N % 16 == 0 && P % 16 == 0 && QT <= 64, "unsupported tile shape");
  static_assert(KR <= 4 && 16 % KR == 0 && 16 % R == 0, "a tile spans whole tokens");
};

// SPLIT: write and readout ranks differ (taken from the parameters; R is the larger);
// otherwise both are R, known at compile time
// (at least two waves per SIMD: 256-thread workgroups must fit two to a compute unit, so the
// kernel keeps within 256 registers per lane)
template <bool BF16, int N, int P, int R, int KR, int QT, bool COORD, int NTHREADS, bool SPLIT>
__global__ __launch_bounds__(NTHREADS, 2) void ssm_bwd_chunk(BwdParams p) {
  using S = BwdShape<BF16, N, P, R, KR, QT, COORD, NTHREADS>;
  constexpr int NW = S::NW;
  using T = typename S::T;
  constexpr int NS = S::NS, PS = S::PS, KS = S::KS, VEC = S::VEC;
  constexpr int QO = S::QO, QK = S::QK;

  __shared__ __align__(16) T sQ[S::QOC * NS];   // q rows (t, o)
  __shared__ __align__(16) T sK[QK * NS];        // k rows j
  
  __shared__ __align__(16) T sV[QK * PS];        // value rows j
  __shared__ __align__(16) T sY[S::QOC * PS];   // dy rows (t, o)
  __shared__ __align__(16) T sSM[S::QOC * KS];  // (S o M) rows (t, o)
  __shared__ __align__(16) T sZM[S::QOC * KS];  // (Z o M) rows (t, o)
  __shared__ __align__(16) T sGh[S::NC * PS];   // folded adjoint G~ (io dtype)
  __shared__ __align__(16) T sSh[N * PS];        // incoming state (io dtype)
  // per-row decay: the rates that multiply the summed step (zero on static rows) and the
  // pair frequencies, by item parity (an item's step gradient reads them while the waves
  // past the first two build the next item's)
  __shared__ float sRate2[COORD ? 2 : 1][COORD ? N : 1], sOmega2[COORD ? 2 : 1][N / 2 + 1];
  __shared__ float sE2[2][N], sEth[N / 2 + 1];   // final-state terms per row (by item parity) / pair
  constexpr int WC = COORD ? NW : 1, WH = COORD ? 1 : NW, WT = S::TE ? NW : 1;
  constexpr int NCO = COORD ? N : 1, PCO = COORD ? N / 2 + 1 : 1;
  __shared__ float sEK[WC][NCO], sEKth[WC][PCO];  // per-wave inter source sums per row / pair
  __shared__ float sPA[WC][NCO], sPW[WC][PCO];    // per-wave parameter partials
  __shared__ float sTok[WC][64];                  // per-wave weighted per-token terms (per-row mode)
  __shared__ float sTT[WH][64], sSrc[WH][64];     // head: target / source inter terms per token
  __shared__ float sRS[WH][64], sCS[WH][64];      // head: row / column sums of Z o S o M
  __shared__ float sDg[WT][64], sDb[WT][64];      // per-wave dgamma / dbeta sums
  __shared__ __align__(16) float sTailX[S::TE ? R * P : 4], sTailB[S::TE ? R * N : 4];
  // two-endpoint tail inputs: the next chunk's raw first adjoint g', B and X of the
  // chunk's last token
  __shared__ __align__(16) T sGraw[S::TE ? N * PS : 8];  // io dtype, rows of PS
  __shared__ __align__(16) T sBt1[S::TE ? R * N : 8], sXt1[S::TE ? R * P : 8];
  // two-endpoint: the item's raw B rows (token t0 - 1 + row / R), for the endpoint-weight
  // gradients
  __shared__ __align__(16) T sBraw[S::TE ? S::BROWS * N : 8];
  // per-token factors of the current item (token = index)
  __shared__ float sTcd[64];                       // cumulative step inside the chunk
  __shared__ float sTw[64], sTel[64], sTlc[64];    // head: e^{L_end - L_t}, e^{L_t}, -A CD log2(e)
  __shared__ float sTga[S::TE ? 64 : 1], sTbe[S::TE ? 64 : 1];
  __shared__ float sMisc[NW];
  __shared__ float sDh;  // the head's skip weight (written with the staging)
  __shared__ float sPartOut[N + N / 2 + 2];  // parameter partials of the item (stored a step later)
  // per-row decay: factor tables of the item (token t, row n), E_t = e^{-A_n (CD_t - CD_end/2)},
  // Theta_t = omega CD_t:  TQ[t] = E_t on real rows, (E_t cos, E_t sin)(Theta_t) on the rows of
  // a pair;  TK[t] = 1 / E_t likewise.  Per row Er = e^{-A_n CD_end / 2} and
  // Fd = e^{-A_n Dnext}; per pair the turn (cos, sin)(omega (CD_end + Dnext)).
  __shared__ __align__(16) float sTQ[COORD ? QT * N : 4], sTK[COORD ? QT * N : 4];
  __shared__ float sEr[COORD ? N : 1], sFd[COORD ? N : 1];
  __shared__ float2 sTurn[COORD ? N / 2 + 1 : 1];
  // per-row decay: the item's per-token scalars, formed with its tables in the previous item's
  // tail: the raw steps (wave 0's step gradient reads them at the item's end) and (CD_end,
  // token count) (wave 1's partials), by item parity; beta of the next chunk's first token
  __shared__ float sRaw2[COORD ? 2 : 1][COORD ? 64 : 1], sCn2[COORD ? 2 : 1][2], sBn;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nch = p.nchunks;
  const int L = p.L, H = p.H, G = p.G, nreal = p.n_real, npairs = p.n_pairs;
  const int nitems = p.batch * H * nch;

  const T* xg = static_cast<const T*>(p.x);
  const T* Bg = static_cast<const T*>(p.B);
  const T* Cg = static_cast<const T*>(p.C);
  const T* dyg = static_cast<const T*>(p.dy);
  T* dxg = static_cast<T*>(p.dx);
  // dB / dC rows go straight to the outputs when every head has its own group; else to
  // per-head partials [batch][L][nheads][R][N], summed over each group by ssm_bwd_group_sum
  const bool part = p.dBh != nullptr;
  T* dBg = static_cast<T*>(part ? p.dBh : p.dB);
  T* dCg = static_cast<T*>(part ? p.dCh : p.dC);
  const int GO = part ? H : G;  // rows per token of those buffers
  // rows per token: the side's own rank in the outputs, R in the partials
  const int rin = SPLIT ? p.rin : R, rout = SPLIT ? p.rout : R;
  // dB / dC row r of token t0 + tl of batch bb.  Head decay: a 64-bit base at the item's
  // first token and a 32-bit offset from it (|tl| <= QT); per-row decay forms the whole
  // 64-bit index (held across the item, the bases cost that kernel registers it lacks)
  auto store_bc = [&](T* out, int rows, int bb, int t0_, int tl, int go, int r, int n, const float* v) {
    const int rs = part ? R : rows;
    if constexpr (COORD) {
      store4<BF16>(out + ((((size_t)bb * L + t0_ + tl) * GO + go) * rs + r) * N + n, v);
    } else {
      T* const base = out + (((size_t)bb * L + t0_) * GO + go) * rs * N;
      store4<BF16>(base + ((tl * GO * rs + r) * N + n), v);
    }
  };

  // zero padding rows / columns (the staging never writes them)
  for (int i = tid; i < (S::NC - N) * PS; i += S::NTH) sGh[N * PS + i] = T(0);
  for (int i = tid; i < (S::QOC - QO) * NS; i += S::NTH) sQ[QO * NS + i] = T(0);
  for (int i = tid; i < (S::QOC - QO) * PS; i += S::NTH) sY[QO * PS + i] = T(0);
  // score entries above the causal diagonal (and padding rows) stay zero for good
  for (int i = tid; i < S::QOC * KS; i += S::NTH) { sSM[i] = T(0); sZM[i] = T(0); }
  if (S::NC > N) {
    for (int i = tid; i < S::QOC * (S::NC - N); i += S::NTH) sQ[(i / (S::NC - N)) * NS + N + i % (S::NC - N)] = T(0);
    for (int i = tid; i < QK * (S::NC - N); i += S::NTH) {
      sK[(i / (S::NC - N)) * NS + N + i % (S::NC - N)] = T(0);
    }
  }
  if (S::PC > P) {
    for (int i = tid; i < QK * (S::PC - P); i += S::NTH) sV[(i / (S::PC - P)) * PS + P + i % (S::PC - P)] = T(0);
    for (int i = tid; i < S::QOC * (S::PC - P); i += S::NTH) sY[(i / (S::PC - P)) * PS + P + i % (S::PC - P)] = T(0);
    for (int i = tid; i < N * (S::PC - P); i += S::NTH) {
      const int r = i / (S::PC - P), cc = P + i % (S::PC - P);
      sGh[r * PS + cc] = T(0); sSh[r * PS + cc] = T(0);
    }
  }

  // ---------------------------------------------------------------- prefetch
  // The workgroup walks the (slice, chunk) items item = blockIdx.x + k gridDim.x.
  // The global reads of the next item go into registers while the current item
  // computes, so the loads overlap the MFMA / VALU work.
  constexpr int PV = P / 4;  // fp32 vectors per state row
  constexpr int CP = (S::C_VECS + S::NTH - 1) / S::NTH, BP = (S::B_VECS + S::NTH - 1) / S::NTH;
  constexpr int XP = (S::X_VECS + S::NTH - 1) / S::NTH, YP = (S::Y_VECS + S::NTH - 1) / S::NTH;
  constexpr int SPV = (N / 2) * PV, SP = (SPV + S::NTH - 1) / S::NTH;
  uint4 pfc[CP], pfb[BP], pfx[XP], pfy[YP];
  // 4-column pieces of the incoming state and the outgoing adjoint rows, as stored (io dtype)
  using Raw4 = typename std::conditional<BF16, uint2, float4>::type;
  Raw4 pfs[SP][2], pfg[SP][2];
  auto raw4_f32 = [](const Raw4& r, float* v) {
    if constexpr (BF16) {
      v[0] = __uint_as_float(r.x << 16);
      v[1] = __uint_as_float(r.x & 0xffff0000u);
      v[2] = __uint_as_float(r.y << 16);
      v[3] = __uint_as_float(r.y & 0xffff0000u);
    } else {
      v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
    }
  };
  Raw4 zr4;
  if constexpr (BF16) zr4 = make_uint2(0, 0); else zr4 = make_float4(0.f, 0.f, 0.f, 0.f);
  float pf_dt = 0.f, pf_be = 0.f, pf_ga = 0.f, pf_dtn = 0.f, pf_bn = 0.f, pf_D = 0.f;
  // per-row decay: the threads past the first two waves build the factor tables, each for
  // one row pair (n, n + 1) = 2 ((tid - TT0) mod N / 2); they hold the item's rates of its
  // two rows (a complex pair: its rate and its frequency)
  constexpr int TT0 = 128, TTN = S::NTH - TT0;
  static_assert(!COORD || (NW >= 4 && TTN % (N / 2) == 0), "table threads cover whole row pairs");
  float pf_ra = 0.f, pf_rb = 0.f;
  const uint4 zero4 = make_uint4(0, 0, 0, 0);

  // The loads of an item, in four parts (C / B rows, X / dy rows and the per-token
  // scalars, incoming states, outgoing adjoints).
  auto prefetch = [&](int item, int part) {
    const int slice = item / nch, c = item % nch;
    const int b = slice / H, h = slice % H, g = h / (H / G);
    const int t0 = c * QT, tn = t0 + QT;
    const bool has_next = tn < L;
    // Rows (token t0 + tl, rank r) of the [batch][L][heads][rank][width] operands, as in
    // store_bc: head decay adds a 32-bit offset to a 64-bit base at the item's first token
    auto row_at = [&](const T* base, int heads, int hh, int rank, int width, int tl, int r, int col) {
      if constexpr (COORD) return base + ((((size_t)b * L + t0 + tl) * heads + hh) * rank + r) * width + col;
      else return base + (((size_t)b * L + t0) * heads + hh) * rank * width + ((tl * heads * rank + r) * width + col);
    };
    if (part == 0) {
#pragma unroll
    for (int k = 0; k < CP; ++k) {
      const int v = tid + S::NTH * k;
      uint4 raw = zero4;
      if (v < S::C_VECS) {
        const int row = v / (N / VEC), n0 = (v % (N / VEC)) * VEC;
        const int t = t0 + row / R, o = row % R;
        if (t < L && o < rout) raw = *reinterpret_cast<const uint4*>(row_at(Cg, G, g, rout, N, row / R, o, n0));
      }
      pfc[k] = raw;
    }
#pragma unroll
    for (int k = 0; k < BP; ++k) {
      const int v = tid + S::NTH * k;
      uint4 raw = zero4;
      if (v < S::B_VECS) {
        const int row = v / (N / VEC), n0 = (v % (N / VEC)) * VEC;
        const int t = t0 + row / R - S::TEH, r = row % R;
        if (t >= 0 && t < L && r < rin) raw = *reinterpret_cast<const uint4*>(row_at(Bg, G, g, rin, N, row / R - S::TEH, r, n0));
        else if (t == -1 && r < rin && p.B_prev)  // the carried token before the sequence
          raw = *reinterpret_cast<const uint4*>(static_cast<const T*>(p.B_prev) + (((size_t)b * G + g) * rin + r) * N + n0);
      }
      pfb[k] = raw;
    }
    }
    if (part == 1) {
#pragma unroll
    for (int k = 0; k < XP; ++k) {
      const int v = tid + S::NTH * k;
      uint4 raw = zero4;
      if (v < S::X_VECS) {
        const int row = v / (P / VEC), p0 = (v % (P / VEC)) * VEC;
        const int t = t0 + row / R - S::TEH, r = row % R;
        if (t >= 0 && t < L && r < rin) raw = *reinterpret_cast<const uint4*>(row_at(xg, H, h, rin, P, row / R - S::TEH, r, p0));
        else if (t == -1 && r < rin && p.x_prev)
          raw = *reinterpret_cast<const uint4*>(static_cast<const T*>(p.x_prev) + (((size_t)b * H + h) * rin + r) * P + p0);
      }
      pfx[k] = raw;
    }
#pragma unroll
    for (int k = 0; k < YP; ++k) {
      const int v = tid + S::NTH * k;
      uint4 raw = zero4;
      if (v < S::Y_VECS) {
        const int row = v / (P / VEC), p0 = (v % (P / VEC)) * VEC;
        const int t = t0 + row / R, o = row % R;
        if (t < L && o < rout) raw = *reinterpret_cast<const uint4*>(row_at(dyg, H, h, rout, P, row / R, o, p0));
      }
      pfy[k] = raw;
    }
    }
    if (part == 2) {
      const T* Sg = static_cast<const T*>(p.saved) + ((size_t)slice * (nch + 1) + c) * N * P;
#pragma unroll
      for (int k = 0; k < SP; ++k) {
        const int v = tid + S::NTH * k;
        Raw4 s0 = zr4, s1 = zr4;
        if (v < SPV) {
          const int n = 2 * (v / PV), q0 = (v % PV) * 4;
          s0 = *reinterpret_cast<const Raw4*>(Sg + (size_t)n * P + q0);
          s1 = *reinterpret_cast<const Raw4*>(Sg + (size_t)(n + 1) * P + q0);
        }
        pfs[k][0] = s0; pfs[k][1] = s1;
      }
      return;
    }
    if (part == 3) {
      // the boundary adjoint of the next chunk (after the last chunk: slot nch, dh_final or
      // zero)
      const T* Gg = static_cast<const T*>(p.gseg) + ((size_t)slice * (nch + 1) + (c + 1)) * N * P;
#pragma unroll
      for (int k = 0; k < SP; ++k) {
        const int v = tid + S::NTH * k;
        Raw4 g0 = zr4, g1 = zr4;
        if (v < SPV) {
          const int n = 2 * (v / PV), q0 = (v % PV) * 4;
          g0 = *reinterpret_cast<const Raw4*>(Gg + (size_t)n * P + q0);
          g1 = *reinterpret_cast<const Raw4*>(Gg + (size_t)(n + 1) * P + q0);
        }
        pfg[k][0] = g0; pfg[k][1] = g1;
      }
      return;
    }
    if (part != 1) return;
    // per-row decay: only the table waves (tid >= TT0) use the per-token scalars
    const bool scal = !COORD || tid >= TT0;
    pf_dt = pf_be = pf_ga = 0.f;
    if (scal && lane < QT && t0 + lane < L) {
      // token t0 + lane of the head (head decay: a 64-bit base and a 32-bit offset)
      const size_t idx = COORD ? ((size_t)b * L + t0 + lane) * H + h
                               : ((size_t)b * L + t0) * H + h + lane * H;
      pf_dt = p.dt[idx];
      if (S::TE) { pf_be = p.beta[idx]; pf_ga = p.gamma[idx]; }
    }
    // the head's skip weight travels with the item's operands: a global value read later,
    // once the next item's loads and this item's stores are in flight, would wait for all
    // of them (one counter covers vector-memory reads and writes)
    pf_D = p.has_D ? p.D[h] : 0.f;
    pf_dtn = pf_bn = 0.f;
    if (scal && has_next) {
      const size_t idx = ((size_t)b * L + tn) * H + h;
      pf_dtn = p.dt[idx];
      if (S::TE) pf_bn = p.beta[idx];
    }
    if (COORD && tid >= TT0) {
      // (the row index is formed per item: hoisted out of the item loop, the addresses
      // derived from it would hold registers the item's phases need)
      int n = 2 * ((tid - TT0) % (N / 2));
      asm volatile("" : "+v"(n));
      const bool pr = n >= nreal;
      const int k = (n - nreal) >> 1;
      const float* ah = p.A + (p.head_rates ? (size_t)h : (size_t)h * (nreal + npairs));
      const int ia = p.head_rates ? 0 : (pr ? nreal + k : n);
      const int ib = p.head_rates ? 0 : n + 1;
      pf_ra = ah[ia];
      pf_rb = pr ? p.omega[(size_t)h * npairs + k] : ah[ib];
    }
  };

  // Per-row decay: the factor tables of item `it` and its rates into buffer `pw`, from its
  // prefetched operands, on the threads tid >= TT0 (whole waves).  The tables have no readers
  // left once an item's dC~ barrier is passed, so the next item's are built during the
  // current item's tail (step gradient and parameter partials on waves 0 and 1).  The item's
  // steep-chunk flag is stored here as well.
  auto make_tables = [&](int it, int pw) {
    const int ct = it % nch, t0t = ct * QT, tnt = t0t + QT;
    float dlt = 0.f;
    if (lane < QT && t0t + lane < L) dlt = p.softplus ? softplus_f32(pf_dt) : pf_dt;
    const float cdt = wave_prefix_sum(dlt);
    const float cde = read_lane(cdt, QT - 1);
    const float nve = static_cast<float>(min(QT, L - t0t));
    const float dnx = tnt < L ? (p.softplus ? softplus_f32(pf_dtn) : pf_dtn) : 0.f;
    const int j = tid - TT0, n = 2 * (j % (N / 2));
    if (j < kWave) {
      // the per-token scalars of the item (its first table wave)
      if (lane < QT) {
        sTcd[lane] = cdt;
        sRaw2[pw][lane] = (t0t + lane < L) ? pf_dt : 0.f;
        if (S::TE) {
          const bool in = t0t + lane < L;
          sTga[lane] = in ? pf_ga : 0.f;
          sTbe[lane] = in ? pf_be : 0.f;
        }
      }
      if (lane == 0) {
        sCn2[pw][0] = cde;
        sCn2[pw][1] = nve;
        if (S::TE) sBn = tnt < L ? pf_bn : 0.f;
      }
    }
    const bool pair = n >= nreal, st0 = n < p.n_static, st1 = n + 1 < p.n_static;
    // exponent rates of rows n, n + 1 per summed step (r) and per token (rs)
    const float r0 = st0 ? 0.f : pf_ra, r0s = st0 ? pf_ra : 0.f;
    const float r1 = pair ? pf_ra : (st1 ? 0.f : pf_rb), r1s = (pair || !st1) ? 0.f : pf_rb;
    const float om = pair ? pf_rb : 0.f;
    const float hc = 0.5f * cde, hn = 0.5f * nve;
    // TQ[t] = E_t (times the pair's turn), TK[t] = 1 / E_t likewise, with
    // E_t = e^{-A_n (CD_t - CD_end / 2)} (static rows: token counts for the summed steps)
    constexpr int TE_N = QT * (N / 2);
#pragma unroll
    for (int i0 = 0; i0 < TE_N; i0 += TTN) {
      // a partial last round goes to the last table threads (the first table wave also forms
      // the per-token scalars and the per-row terms); entries stay TTN apart, so a thread's
      // row pair is the same in every round
      const int cnt = TE_N - i0 < TTN ? TE_N - i0 : TTN;
      const bool ok = j >= TTN - cnt;
      const int i = i0 + j - (TTN - cnt);
      const int t = (ok ? i : 0) / (N / 2);
      const float cd = __shfl(cdt, t, kWave);  // (the shuffle runs on whole waves)
      if (ok) {
        float2 q, k;
        if (pair) {
          const float x = r0 * (cd - hc);
          const float e = __expf(-x), ei = __expf(x);
          float sn, cs;
          fast_sincos(om * cd, &sn, &cs);
          q = make_float2(e * cs, e * sn);
          k = make_float2(ei * cs, ei * sn);
        } else {
          const float cn = static_cast<float>(t + 1) - hn;
          const float x0 = r0 * (cd - hc) + r0s * cn;
          const float x1 = r1 * (cd - hc) + r1s * cn;
          q = make_float2(__expf(-x0), __expf(-x1));
          k = make_float2(__expf(x0), __expf(x1));
        }
        *reinterpret_cast<float2*>(sTQ + t * N + n) = q;
        *reinterpret_cast<float2*>(sTK + t * N + n) = k;
      }
    }
    // per row: Er = e^{-A_n CD_end / 2}, Fd = e^{-A_n Dnext}; per pair the turn
    // (cos, sin)(omega (CD_end + Dnext)); the rates of the item
    if (j < N / 2) {
      const float nx = tnt < L ? 1.f : 0.f;
      sEr[n] = __expf(-r0 * hc - r0s * hn);
      sEr[n + 1] = __expf(-r1 * hc - r1s * hn);
      sFd[n] = __expf(-r0 * dnx - r0s * nx);
      sFd[n + 1] = __expf(-r1 * dnx - r1s * nx);
      sRate2[pw][n] = r0;
      sRate2[pw][n + 1] = r1;
      if (pair) {
        float sn, cs;
        fast_sincos(om * (cde + dnx), &sn, &cs);
        sTurn[(n - nreal) >> 1] = make_float2(cs, sn);
        sOmega2[pw][(n - nreal) >> 1] = om;
      }
    }
    // a chunk too steep for the midpoint fold is redone by the token-by-token reverse pass:
    // the largest |rate| of its dynamic and of its static rows
    if (p.wild && j < kWave) {
      const bool own = j < N / 2;
      const float amax = wave_max(own ? fmaxf(fabsf(r0), fabsf(r1)) : 0.f);
      const float smax = wave_max(own ? fmaxf(fabsf(r0s), fabsf(r1s)) : 0.f);
      const bool steep = amax * cde + smax * nve > kFoldLimit;
      if (j == 0) {
        p.wild[it] = steep ? 1 : 0;
        if (steep) atomicOr(p.wild_any, 1);
      }
    }
  };

  // The per-token scalar gradients and the parameter partials of an item are
  // stored during the next item, after its prefetch: they come from wave 0 at the
  // very end of an item, and storing them at once would make wave 0's wait for its
  // next prefetched loads include them, with every other wave held at the barrier.
  float o_ddt = 0.f, o_dg = 0.f, o_db = 0.f;
  auto flush_scalars = [&](int it) {
    const int slice = it / nch, c = it % nch;
    const int b = slice / H, h = slice % H;
    const int t0 = c * QT;
    if (wave == 0 && lane < QT && t0 + lane < L) {
      const size_t idx = COORD ? ((size_t)b * L + t0 + lane) * H + h
                               : ((size_t)b * L + t0) * H + h + lane * H;
      p.ddt[idx] = o_ddt;
      if (S::TE) {
        if (p.dgamma) p.dgamma[idx] = o_dg;
        if (p.dbeta) p.dbeta[idx] = o_db;
      }
    }
    // (per-row decay: wave 1 stores the partials itself at the end of the item)
    if (p.part && !COORD)
      for (int k = tid; k < p.npart; k += S::NTH) p.part[((size_t)slice * nch + c) * p.npart + k] = sPartOut[k];
  };

  // VEC consecutive rows n0.. of a staged vector times their table entries: per-row
  // factors, or on a pair (a, b) = table entries the product (a u0 + b u1, -b u0 + a u1)
  auto apply_tab = [&](float* v, const float* tab, int n0) {
    float f[VEC];
#pragma unroll
    for (int i = 0; i < VEC; i += 4) {
      const float4 w = *reinterpret_cast<const float4*>(tab + n0 + i);
      f[i] = w.x; f[i + 1] = w.y; f[i + 2] = w.z; f[i + 3] = w.w;
    }
#pragma unroll
    for (int i = 0; i < VEC; i += 2) {
      const float a = v[i], bb = v[i + 1];
      if (n0 + i >= nreal) {
        v[i] = f[i] * a + f[i + 1] * bb;
        v[i + 1] = -f[i + 1] * a + f[i] * bb;
      } else {
        v[i] = f[i] * a;
        v[i + 1] = f[i + 1] * bb;
      }
    }
  };

  // Key rows.  Without two-endpoint writes group u (KR = R rows) holds the keys of token u.
  // With them, group u (KR = 2R rows) holds the two rows that carry source token u's B_u and
  // X_u: the gamma row gamma_u B_u, entering at u (rows r < R), and the beta row
  // beta_{u+1} B_u, entering at u + 1 (rows R + r), so the gradients of B_u and X_u add
  // lanes r and R + r of one group.  The last source's beta row enters the next chunk and
  // is not formed here; its place holds the halo row beta_0 B_{t0-1} (source -1, entering
  // at the chunk's first token).
  auto key_entry = [](int j) {
    const int u = j / KR;
    return (!S::TE || j % KR < R) ? u : (u == QT - 1 ? 0 : u + 1);
  };
  auto key_src = [](int j) {
    const int u = j / KR;
    return (!S::TE || j % KR < R) ? u : (u == QT - 1 ? -1 : u);
  };
  // value of v in lane l ^ R (the other row of the same source inside a key group)
  auto partner = [](float v) { return R == 1 ? dpp_f32<0xB1>(v) : dpp_f32<0x4E>(v); };

  int prev = -1;
  int item = blockIdx.x;
  if (item < nitems) {
#pragma unroll
    for (int part = 0; part < 4; ++part) prefetch(item, part);
    if (COORD && tid >= TT0) make_tables(item, 0);
  }
  // Plain head decay: wave 0's step-gradient tail of an item reads only per-wave sums
  // (zeroed by their own wave after the staging barrier) and the final-state terms
  // (double-buffered by item parity), so the other waves go on with the next item's
  // staging while it runs; the staging barrier then waits for wave 0.
  constexpr bool RELAXED = !COORD && !S::TE;
  int par = 0;
  for (; item < nitems; item += gridDim.x, par ^= 1) {
    const int slice = item / nch, c = item % nch;
    const int b = slice / H, h = slice % H, g = h / (H / G);
    const int t0 = c * QT, tn = t0 + QT;
    const bool has_next = tn < L;
    float* sE = sE2[par];
    // row (token t0 + s, rank kr) of dx, addressed like the dB / dC rows (store_bc)
    auto dx_row = [&](int s, int kr, int col) {
      if constexpr (COORD) return dxg + ((((size_t)b * L + t0 + s) * H + h) * rin + kr) * P + col;
      else return dxg + (((size_t)b * L + t0) * H + h) * rin * P + ((s * H * rin + kr) * P + col);
    };

    // the previous item is done with every shared buffer (and, per-row decay, its tail has
    // built this item's factor tables and rates)
    if (!RELAXED) __syncthreads();
    const float* sRate = sRate2[COORD ? par : 0];
    const float* sOmega = sOmega2[COORD ? par : 0];
    const float Ah = COORD ? 0.f : p.A[h];

    // ---------------------------------------------------------------- scalars
    // per-row decay: formed with the tables in the previous item's tail (sTcd, sTga, sTbe,
    // sRaw2, sCn2, sBn); head decay: formed here by every wave
    float raw_l = 0.f, dl = 0.f;
    float dnext = 0.f;
    float cdend = 0.f;
    if constexpr (!COORD) {
      if (lane < QT && t0 + lane < L) {
        raw_l = pf_dt;
        dl = p.softplus ? softplus_f32(raw_l) : raw_l;
      }
      if (has_next) dnext = p.softplus ? softplus_f32(pf_dtn) : pf_dtn;
      // scalars read again after the next item's loads are issued are materialised here:
      // left to the compiler, they are copied out of the prefetch registers at the end of
      // the item, and that copy waits for every load and store in flight
      asm volatile("" : "+v"(raw_l), "+v"(dl));
      const float cd_l = wave_prefix_sum(dl);
      cdend = read_lane(cd_l, QT - 1);
      const float w_l = __expf(-Ah * (cdend - cd_l));   // e^{L_end - L_t}
      const float el_l = __expf(-Ah * cd_l);            // e^{L_t}
      if (wave == 0 && lane < QT) {
        sTcd[lane] = cd_l;
        sTw[lane] = w_l;
        sTel[lane] = el_l;
        sTlc[lane] = -Ah * 1.4426950408889634f * cd_l;
      }
    }
    // ---------------------------------------------------------------- staging
    // queries (t, o)
  #pragma unroll
    for (int k = 0; k < CP; ++k) {
      const int v = tid + S::NTH * k;
      const int vv = v < S::C_VECS ? v : 0;
      const int row = vv / (N / VEC), n0 = (vv % (N / VEC)) * VEC;
      const int tl = row / R;
      if (v >= S::C_VECS) continue;
      uint4 raw = pfc[k];
      if (COORD) {
        // q = R(-Theta_t) C_t E_t
        float vals[VEC];
        unpack<BF16>(raw, vals);
        apply_tab(vals, sTQ + tl * N, n0);
        raw = pack<BF16>(vals);
      }
      *reinterpret_cast<uint4*>(sQ + row * NS + n0) = raw;
    }
    // keys: gamma_s B_s in group s, beta_{s+1} B_s in group s (row R + r), the halo's beta
    // row in the last group
  #pragma unroll
    for (int k = 0; k < BP; ++k) {
      const int v = tid + S::NTH * k;
      const int vv = v < S::B_VECS ? v : 0;
      const int row = vv / (N / VEC), n0 = (vv % (N / VEC)) * VEC;
      const int sl = row / R - S::TEH, r = row % R;
      const int ta = sl < 0 ? 0 : sl, tb = sl + 1 < QT ? sl + 1 : QT - 1;
      const float wv[2] = {S::TE ? sTga[ta] : 1.f, S::TE ? sTbe[tb] : 0.f};
      if (v >= S::B_VECS) continue;
      if (S::TE && sl == QT - 1) *reinterpret_cast<uint4*>(sBt1 + r * N + n0) = pfb[k];
      if (S::TE) *reinterpret_cast<uint4*>(sBraw + row * N + n0) = pfb[k];
      float vals[VEC];
      unpack<BF16>(pfb[k], vals);
  #pragma unroll
      for (int e = 0; e < 2; ++e) {
        if (e == 1 && !S::TE) break;
        const int tau = sl + e;
        if (tau < 0 || tau >= QT || (e == 0 && sl < 0)) continue;
        const int j = e == 0 ? sl * KR + r : (sl < 0 ? QT - 1 : sl) * KR + R + r;
        float u[VEC], kk[VEC];
  #pragma unroll
        for (int i = 0; i < VEC; ++i) u[i] = vals[i] * wv[e];
        if (COORD) {
          // k = R(-Theta_tau) u / E_tau,  ke = k e^{-A CD_end / 2}
          apply_tab(u, sTK + tau * N, n0);
  #pragma unroll
          for (int i = 0; i < VEC; ++i) kk[i] = u[i];
        } else {
  #pragma unroll
          for (int i = 0; i < VEC; ++i) kk[i] = u[i];
        }
        *reinterpret_cast<uint4*>(sK + j * NS + n0) = pack<BF16>(kk);
      }
    }
    // values j and dy rows (and the head's skip weight, from the prefetched operands: kept in
    // a register across the item, its copy would wait for the next item's loads)
    if (tid == 0) sDh = pf_D;
    float dDp = 0.f;
  #pragma unroll
    for (int k = 0; k < XP; ++k) {
      const int v = tid + S::NTH * k;
      if (v >= S::X_VECS) continue;
      const int row = v / (P / VEC), p0 = (v % (P / VEC)) * VEC;
      const int sl = row / R - S::TEH, r = row % R;
      if (sl >= 0) *reinterpret_cast<uint4*>(sV + (sl * KR + r) * PS + p0) = pfx[k];
      if (S::TE && sl == QT - 1) *reinterpret_cast<uint4*>(sXt1 + r * P + p0) = pfx[k];
      if (S::TE && sl + 1 < QT)
        *reinterpret_cast<uint4*>(sV + ((sl < 0 ? QT - 1 : sl) * KR + R + r) * PS + p0) = pfx[k];
    }
  #pragma unroll
    for (int k = 0; k < YP; ++k) {
      const int v = tid + S::NTH * k;
      if (v >= S::Y_VECS) continue;
      const int row = v / (P / VEC), p0 = (v % (P / VEC)) * VEC;
      *reinterpret_cast<uint4*>(sY + row * PS + p0) = pfy[k];
    }
    // incoming state S_in and folded adjoint G~ = e^{-A Dnext} R(-omega (cd_end + Dnext)) g'
    // (per-row decay: also times e^{-A CD_end / 2}, the factor that turns the folded keys
    // into the keys seen from the chunk end, so the keys need no second scaled copy)
    // (rounded to the io dtype as MFMA operands), final-state terms per row / pair
    {
      const float lend_h = COORD ? 0.f : __expf(-Ah * cdend);
      const float gdec_h = COORD ? 0.f : __expf(-Ah * dnext);
  #pragma unroll
      for (int k = 0; k < SP; ++k) {
        const int v = tid + S::NTH * k;
        if (v >= SPV) continue;
        const int rp = v / PV, pc = v % PV;
        const int n = 2 * rp, q0 = pc * 4;
        float sa[4], sb[4], ga[4], gb[4];
        raw4_f32(pfs[k][0], sa);
        raw4_f32(pfs[k][1], sb);
        raw4_f32(pfg[k][0], ga);
        raw4_f32(pfg[k][1], gb);
        if (S::TE) {
          store4<BF16>(sGraw + n * PS + q0, ga);
          store4<BF16>(sGraw + (n + 1) * PS + q0, gb);
        }
        float fa, fb, lea, leb;
        if (COORD) {
          fa = sFd[n] * sEr[n]; fb = sFd[n + 1] * sEr[n + 1];
          lea = sEr[n]; leb = sEr[n + 1];
        } else {
          fa = fb = gdec_h; lea = leb = lend_h;
        }
  #pragma unroll
        for (int i = 0; i < 4; ++i) { ga[i] *= fa; gb[i] *= fb; }
        const bool pair = COORD && n >= nreal;
        if (pair) {
          const float2 tr = sTurn[(n - nreal) >> 1];
          const float sn = tr.y, cs = tr.x;
  #pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float a0 = ga[i], a1 = gb[i];
            ga[i] = cs * a0 + sn * a1;
            gb[i] = -sn * a0 + cs * a1;
          }
        }
        float ea = 0.f, eb = 0.f, eth = 0.f;
  #pragma unroll
        for (int i = 0; i < 4; ++i) {
          ea += ga[i] * sa[i];
          eb += gb[i] * sb[i];
          eth += -ga[i] * sb[i] + gb[i] * sa[i];  // <G~, J S>
        }
        ea *= lea; eb *= leb; eth *= lea;
        // reduce over the PV p-vectors of this row pair (an aligned group of lanes)
        ea = group_sum<PV>(ea);
        eb = group_sum<PV>(eb);
        if (COORD) eth = group_sum<PV>(eth);
        if (pc == 0) {
          sE[n] = ea; sE[n + 1] = eb;
          if (pair) sEth[(n - nreal) >> 1] = eth;
        }
        store4<BF16>(sSh + n * PS + q0, sa);
        store4<BF16>(sSh + (n + 1) * PS + q0, sb);
        store4<BF16>(sGh + n * PS + q0, ga);
        store4<BF16>(sGh + (n + 1) * PS + q0, gb);
      }
    }
    // the next item's loads go out now and land while this one computes
    const int nxt = item + static_cast<int>(gridDim.x);
    if (nxt < nitems)
#pragma unroll
      for (int part = 0; part < 4; ++part) prefetch(nxt, part);
    if (prev >= 0) flush_scalars(prev);
    __syncthreads();
    // this wave's own slots of the per-wave sums (only it accumulates into them; the previous
    // item's tail, which reads every wave's, ended before the staging barrier)
    if (RELAXED) {
      sTT[wave][lane] = 0.f; sSrc[wave][lane] = 0.f; sRS[wave][lane] = 0.f; sCS[wave][lane] = 0.f;
    }
    if (COORD) {
      sTok[wave][lane] = 0.f;
      for (int n = lane; n < NCO; n += kWave) { sEK[wave][n] = 0.f; sPA[wave][n] = 0.f; }
      for (int k = lane; k < PCO; k += kWave) { sEKth[wave][k] = 0.f; sPW[wave][k] = 0.f; }
      if (S::TE) { sDg[wave][lane] = 0.f; sDb[wave][lane] = 0.f; }
    }
    // two-endpoint tails of the last token from the staged rows: beta_{t0'} B_{t1}^T g'
    // and g' X_{t1}^T (zero without a next chunk, where g' and beta_{t0'} are zero),
    // as MFMA products in the io dtype (g' rounded to it, as the folded G~ is) with the
    // R rows padded to 16:
    //   tail X (R x P) = B_{t1} (R x N) g' (N x P),   tail B^T (N x R) = g' (N x P) X_{t1}^T (P x R),
    // one 16-column output tile per wave (P / 16 tiles of tail X, then N / 16 of tail B)
    if constexpr (S::TE && N % 32 == 0 && P % 32 == 0) {
      static_assert(R <= 16, "tail products with the rows padded to 16");
      // 8 consecutive elements of row m of a staged R-row buffer (zero for m >= R)
      auto rows8 = [&](const T* buf, int ld, int m, int k0) {
        Frag<BF16> f;
        if (m < R) {
          f = load_frag<BF16>(buf + m * ld + k0);
        } else {
          if constexpr (BF16) {
            f.v = bf16x8{};
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) f.v[i] = 0.f;
          }
        }
        return f;
      };
      for (int u = wave; u < P / 16 + N / 16; u += NW) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (u < P / 16) {
          const int tp = u;
#pragma unroll
          for (int kk = 0; kk < N / 32; ++kk) {
            const auto fa = rows8(sBt1, N, lane & 15, kk * 32 + 8 * (lane >> 4));
            const auto fb = load_frag_tr<BF16>(sGraw + (kk * 32) * PS + 16 * tp, PS);
            mma<BF16>(acc, fa, fb);
          }
          // lane l: rows r = 4 (l >> 4) + i, column p = 16 tp + (l & 15)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * (lane >> 4) + i;
            if (r < R) sTailX[r * P + 16 * tp + (lane & 15)] = sBn * acc[i];
          }
        } else {
          const int tn = u - P / 16;
#pragma unroll
          for (int kk = 0; kk < P / 32; ++kk) {
            const auto fa = load_frag<BF16>(sGraw + (16 * tn + (lane & 15)) * PS + kk * 32 + 8 * (lane >> 4));
            const auto fb = rows8(sXt1, P, lane & 15, kk * 32 + 8 * (lane >> 4));
            mma<BF16>(acc, fa, fb);
          }
          // lane l: rows n = 16 tn + 4 (l >> 4) + i, column r = l & 15
          if ((lane & 15) < R) {
#pragma unroll
            for (int i = 0; i < 4; ++i) sTailB[(lane & 15) * N + 16 * tn + 4 * (lane >> 4) + i] = sBn * acc[i];
          }
        }
      }
    } else if constexpr (S::TE) {
      // narrow states: each of the R P + R N outputs is a dot product of length N or P
      // split over TT adjacent lanes, summed by a fixed butterfly
      constexpr int O1 = R * P, OT = R * P + R * N;
      constexpr int TQ = S::NTH / OT;
      constexpr int TT = TQ >= 16 ? 16 : TQ >= 8 ? 8 : TQ >= 4 ? 4 : TQ >= 2 ? 2 : 1;
      static_assert(N % TT == 0 && P % TT == 0, "tail dot products split evenly");
      for (int base = 0; base < OT * TT; base += S::NTH) {
        const int u = base + tid, o = u / TT, part = u % TT;
        float acc = 0.f;
        if (o < O1) {
          const int r = o / P, pp = o % P;
#pragma unroll 2
          for (int n = part * (N / TT); n < (part + 1) * (N / TT); ++n)
            acc += to_f32(sBt1[r * N + n]) * to_f32(sGraw[n * PS + pp]);
        } else if (o < OT) {
          const int r = (o - O1) / N, n = (o - O1) % N;
#pragma unroll 2
          for (int pp = part * (P / TT); pp < (part + 1) * (P / TT); ++pp)
            acc += to_f32(sGraw[n * PS + pp]) * to_f32(sXt1[r * P + pp]);
        }
        acc = group_sum<TT>(acc);
        if (part == 0 && o < O1) sTailX[o] = sBn * acc;
        else if (part == 0 && o < OT) sTailB[o - O1] = sBn * acc;
      }
    }
    if (p.has_D) {
      // sum of dy . x over the item, one 16-byte vector of each per step
      for (int v = tid; v < QO * (P / VEC); v += S::NTH) {
        const int row = v / (P / VEC), p0 = (v % (P / VEC)) * VEC, tl = row / R, o = row % R;
        float yv[VEC], xv[VEC];
        unpack<BF16>(*reinterpret_cast<const uint4*>(sY + row * PS + p0), yv);
        unpack<BF16>(*reinterpret_cast<const uint4*>(sV + (tl * KR + o) * PS + p0), xv);
#pragma unroll
        for (int e = 0; e < VEC; ++e) dDp += yv[e] * xv[e];
      }
    }
    dDp = wave_sum(dDp);
    if (lane == 0) sMisc[wave] = dDp;

    // ---------------------------------------------------------------- scores
    // S^T = K Q^T and Z^T = V dY^T, computed transposed: lane l holds query row
    // 16 ti + (l & 15) against keys 16 tj + 4 (l >> 4) + i.  Only tiles with a causal
    // entry are formed; the others stay zero from the start.
    for (int tile = wave; tile < S::SC_TILES; tile += NW) {
      int ti = 0, tj = tile;
#pragma unroll
      for (int a = 0; a < S::TQ - 1; ++a) {
        const int rt = S::row_tiles(ti) + (S::extra_tile(ti) ? 1 : 0);
        if (tj >= rt) {
          tj -= rt;
          ++ti;
        }
      }
      if (tj == S::row_tiles(ti)) tj = S::TK - 1;  // the halo's tile
      f32x4 sc = {0.f, 0.f, 0.f, 0.f}, z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < S::NC / 32; ++kk) {
        const auto fk = load_frag<BF16>(sK + (16 * tj + (lane & 15)) * NS + kk * 32 + 8 * (lane >> 4));
        const auto fq = load_frag<BF16>(sQ + (16 * ti + (lane & 15)) * NS + kk * 32 + 8 * (lane >> 4));
        mma<BF16>(sc, fk, fq);
      }
#pragma unroll
      for (int kk = 0; kk < S::PC / 32; ++kk) {
        const auto fv = load_frag<BF16>(sV + (16 * tj + (lane & 15)) * PS + kk * 32 + 8 * (lane >> 4));
        const auto fy = load_frag<BF16>(sY + (16 * ti + (lane & 15)) * PS + kk * 32 + 8 * (lane >> 4));
        mma<BF16>(z, fv, fy);
      }
      const int row = 16 * ti + (lane & 15), t = row / R;
      const int j0 = 16 * tj + 4 * (lane >> 4);
      const float lt = COORD ? 0.f : sTlc[t];
      float smv[4], zmv[4], wv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = key_entry(j0 + i);
        // masked by selection: with per-row decay the folded product of a masked entry
        // (s > t) can overflow, and inf * 0 would be NaN
        const bool causal = s <= t;
        const float m = COORD ? 1.f : __builtin_amdgcn_exp2f(lt - sTlc[causal ? s : t]);
        smv[i] = causal ? sc[i] * m : 0.f;
        zmv[i] = causal ? z[i] * m : 0.f;
        // same-token entries (mask 1 whatever the decay) add equally to the row and the
        // column sum of a token, whose difference the step gradient takes: left out of
        // both, so steep decay (tiny differences) does not meet fp32 rounding of them
        wv[i] = s < t ? z[i] * smv[i] : 0.f;
      }
      store4<BF16>(sSM + row * KS + j0, smv);
      store4<BF16>(sZM + row * KS + j0, zmv);
      if (!COORD) {
        // W = Z o S o M: row sums per query token (the four lane groups hold disjoint
        // keys of one row), column sums per key token (the 16 lanes of a group hold
        // the 16 rows of each key)
        float rs = (wv[0] + wv[1]) + (wv[2] + wv[3]);
        rs = add_xor16(rs);
        rs = add_xor32(rs);
        rs = group_sum<R>(rs);
        if (lane < 16 && (lane % R) == 0) sRS[wave][t] += rs;
        float cs[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) cs[i] = group_sum<16>(wv[i]);
        if ((lane & 15) == 0) {
#pragma unroll
          for (int i = 0; i < 4; i += KR) {
            float v = 0.f;
#pragma unroll
            for (int e = 0; e < KR; ++e) v += cs[i + e];
            sCS[wave][(j0 + i) / KR] += v;
          }
        }
      }
    }
    __syncthreads();

    // ---------------------------------------------------------------- dV -> dX
    // dV^T = dY^T (S o M) + G~^T K^T, computed transposed: lane l holds key
    // 16 tj + (l & 15) and value columns 16 tp + 4 (l >> 4) + i.  When NW is a multiple
    // of the column tiles, a wave takes two tiles of one column block (tiles t and
    // t + NW), and their dY and G~ fragments are read once.
    auto dv_tile = [&](const int tj, const int tp, const f32x4& ai, const f32x4& ae) {
      const int j = 16 * tj + (lane & 15), s = j / KR, kr = j % KR;
      const int pl = 16 * tp + 4 * (lane >> 4);
      const float wj = COORD ? 1.f : sTw[s];
      float dv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) dv[i] = ai[i] + wj * ae[i];
      if (!S::TE) {
        if (p.has_D) {
          float yv[4];
          load4<BF16>(sY + (s * R + kr) * PS + pl, yv);
#pragma unroll
          for (int i = 0; i < 4; ++i) dv[i] += sDh * yv[i];
        }
        const int t = t0 + s;
        if (t < L && kr < rin) store4<BF16>(dx_row(s, kr, pl), dv);
      } else {
        // dX_s = (gamma row) + (beta row) of group s, lanes kr and kr + R; the last
        // source's beta term comes from the next chunk's boundary adjoint (the tail), and
        // the halo row in its place belongs to the chunk before
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = partner(dv[i]);
        if (kr < R) {
          if (s == QT - 1) {
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = sTailX[kr * P + pl + i];
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) dv[i] += o[i];
          if (p.has_D) {
            float yv[4];
            load4<BF16>(sY + (s * R + kr) * PS + pl, yv);
#pragma unroll
            for (int i = 0; i < 4; ++i) dv[i] += sDh * yv[i];
          }
          const int t = t0 + s;
          if (t < L && kr < rin) store4<BF16>(dx_row(s, kr, pl), dv);
        }
      }
    };
    {
      constexpr int NT_DV = S::TK * S::TP;
      constexpr int DVB = (NW % S::TP == 0 && NT_DV % (2 * NW) == 0) ? 2 : 1;
      for (int tile = wave; tile < NT_DV; tile += NW * DVB) {
        const int tp = tile % S::TP;
        int tjs[DVB];
#pragma unroll
        for (int x = 0; x < DVB; ++x) tjs[x] = (tile + x * NW) / S::TP;
        f32x4 ai[DVB], ae[DVB];
#pragma unroll
        for (int x = 0; x < DVB; ++x) ai[x] = ae[x] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < S::QOC / 32; ++kk) {
          const auto fy = load_frag_tr<BF16>(sY + (kk * 32) * PS + 16 * tp, PS);
#pragma unroll
          for (int x = 0; x < DVB; ++x) {
            const auto fs = load_frag_tr<BF16>(sSM + (kk * 32) * KS + 16 * tjs[x], KS);
            mma<BF16>(ai[x], fy, fs);
          }
        }
#pragma unroll
        for (int kk = 0; kk < S::NC / 32; ++kk) {
          if (kk * 32 < N) {
            const auto fgh = load_frag_tr<BF16>(sGh + (kk * 32) * PS + 16 * tp, PS);
#pragma unroll
            for (int x = 0; x < DVB; ++x) {
              const auto fk = load_frag<BF16>(sK + (16 * tjs[x] + (lane & 15)) * NS + kk * 32 + 8 * (lane >> 4));
              mma<BF16>(ae[x], fgh, fk);
            }
          }
        }
#pragma unroll
        for (int x = 0; x < DVB; ++x) dv_tile(tjs[x], tp, ai[x], ae[x]);
      }
    }

    // ---------------------------------------------------------------- dK~ -> dB, dbeta, dgamma
    // lane l holds key 16 tj + (l & 15) and state rows 16 tnn + 4 (l >> 4) + i.  Tiles
    // go in BN x BJ blocks per wave: a block's fragments are read once for all of its
    // tiles, and its tiles are independent MFMA chains.
    // per-row decay: the tile's per-row partial sums (over its 16 key columns, one per
    // lane) are added into xpa / xek / xpw / xekt; flush_rows reduces them over the lanes
    // and adds them to this wave's slots
    auto dk_tile = [&](const int tnn, const int tj, const f32x4& ai, const f32x4& ae, float* xpa,
                       float* xek, float* xpw, float* xekt) {
      const int j = 16 * tj + (lane & 15), kr = j % KR;
      const int s = key_entry(j), src = key_src(j);  // entry token, token of the B row carried
      const int n0 = 16 * tnn + 4 * (lane >> 4);
      const float cds = sTcd[s];
      const float wj = COORD ? 1.f : sTw[s];
      const bool brow = S::TE && kr >= R;
      const int rr = brow ? kr - R : kr;
      const int tb = t0 + src;
      float tokacc = 0.f;
      float dk[4], kv[4], rpa[4], rek[4], rpw[2] = {0.f, 0.f}, rekt[2] = {0.f, 0.f};
      load4<BF16>(sK + j * NS + n0, kv);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = n0 + i;
        rpa[i] = 0.f; rek[i] = 0.f;
        if (COORD) {
          const float ck = ai[i] + ae[i];
          dk[i] = ck;  // scaled by e^{r - L_s} (with the pair's turn) below
          // source terms: -k o cK  (rows); the inter part also feeds the final-state term
          const float dr = -kv[i] * ck;
          tokacc += -sRate[n] * dr;                          // zero on static rows
          rpa[i] = -(n < p.n_static ? static_cast<float>(s + 1) : cds) * dr;
          rek[i] = kv[i] * ae[i];
        } else {
          dk[i] = ai[i] + wj * ae[i];
          tokacc += kv[i] * wj * ae[i];  // K~ o dK~ (inter part)
        }
      }
      if (COORD) {
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const int n = n0 + i;
          if (n >= nreal) {
            const int kp = (n - nreal) >> 1;
            const float ca = ai[i] + ae[i], cb = ai[i + 1] + ae[i + 1];
            // K~^T J dK~ in scaled form: -k_a cK_b + k_b cK_a
            const float dth = -kv[i] * cb + kv[i + 1] * ca;
            tokacc += sOmega[kp] * dth;
            rpw[i >> 1] = cds * dth;
            rekt[i >> 1] = -(-kv[i] * ae[i + 1] + kv[i + 1] * ae[i]);
          }
        }
        // dK~ = e^{r - L_s} cK, and unfold the key's rotation: u = R(+Theta_s) dK~
        // (table entries (a, b) = (cos, sin) / E_s on a pair)
        const float4 tk = *reinterpret_cast<const float4*>(sTK + s * N + n0);
        const float f[4] = {tk.x, tk.y, tk.z, tk.w};
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const float a0 = dk[i], a1 = dk[i + 1];
          if (n0 + i >= nreal) {
            dk[i] = f[i] * a0 - f[i + 1] * a1;
            dk[i + 1] = f[i + 1] * a0 + f[i] * a1;
          } else {
            dk[i] = f[i] * a0;
            dk[i + 1] = f[i + 1] * a1;
          }
        }
      }
      // gradient w.r.t. the stored B row and the endpoint weights
      float dgb = 0.f;
      if (S::TE) {
        const float wgt = brow ? sTbe[s] : sTga[s];
        {
          // the staged raw row (zero outside the sequence and for rows >= rank_in)
          float braw[4];
          load4<BF16>(sBraw + ((src + 1) * R + rr) * N + n0, braw);
#pragma unroll
          for (int i = 0; i < 4; ++i) dgb += dk[i] * braw[i];
        }
        // dB_u = gamma_u (gamma row's dK~) + beta_{u+1} (beta row's dK~), lanes kr and kr + R
        // of group u (the last source's beta term: the tail)
        float db[4], o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          db[i] = wgt * dk[i];
          o[i] = partner(db[i]);
        }
        if (!brow) {
          const int u = j / KR;
          if (u == QT - 1) {
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = sTailB[rr * N + n0 + i];
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) db[i] += o[i];
          if (t0 + u < L && rr < rin) store_bc(dBg, rin, b, t0, u, part ? h : g, rr, n0, db);
        }
      } else if (tb < L && rr < rin) {
        store_bc(dBg, rin, b, t0, src, part ? h : g, rr, n0, dk);
      }
      if (COORD) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xpa[i] += rpa[i];
          xek[i] += rek[i];
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          xpw[q] += rpw[q];
          xekt[q] += rekt[q];
        }
      }
      // per-key sums over the 4 row groups, then over the keys of one entry token: a group's
      // R gamma rows; with two-endpoint writes the beta rows of the group before (R lanes
      // down) enter at the same token and are added there, except for the tile's last
      // group, whose beta rows (entering at the next group's token, or the halo's at 0)
      // are stored on their own
      tokacc = add_xor16(tokacc);
      tokacc = add_xor32(tokacc);
      bool tok_store = false;
      if constexpr (S::TE) {
        tokacc = group_sum<R>(tokacc);
        const float prevb = dpp_f32<0x110 + R>(tokacc);  // lane - R inside the row
        const int l16 = lane & 15;
        if (kr == 0 && l16 >= KR) tokacc += prevb;
        tok_store = kr == 0 || (kr == R && l16 == 16 - R);
      } else {
        tokacc = group_sum<KR>(tokacc);
        tok_store = (lane % KR) == 0;
      }
      if (S::TE) {
        dgb = add_xor16(dgb);
        dgb = add_xor32(dgb);
        dgb = group_sum<R>(dgb);
      }
      if (lane < 16) {
        if (tok_store) {
          if (COORD) sTok[wave][s] += tokacc;  // weighted source contribution
          else sSrc[wave][s] += tokacc;        // K~ o dK~ (inter), unweighted
        }
        if (S::TE && (lane % R) == 0) {
          if (brow) sDb[wave][s] += dgb;
          else sDg[wave][s] += dgb;
        }
      }
    };
    {
      constexpr int BN = S::KBLK ? 2 : 1, BJ = (S::KBLK || S::KPAIR) ? 2 : 1, NBJ = S::TK / BJ, NBN = S::TN / BN;
      // per-row decay: blocks go n-block fastest, so when NW is a multiple of the n-blocks
      // all blocks of a wave share its n-block and their per-row sums are reduced once,
      // after the loop
      constexpr bool SHARE_N = NW % NBN == 0;
      float apa[BN][4], aek[BN][4], apw[BN][2], aekt[BN][2];
      auto zero_rows = [&]() {
#pragma unroll
        for (int x = 0; x < BN; ++x) {
#pragma unroll
          for (int i = 0; i < 4; ++i) apa[x][i] = aek[x][i] = 0.f;
          apw[x][0] = apw[x][1] = aekt[x][0] = aekt[x][1] = 0.f;
        }
      };
      auto flush_rows = [&](int tn0) {
#pragma unroll
        for (int x = 0; x < BN; ++x) {
          const int n0 = 16 * (tn0 + x) + 4 * (lane >> 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            apa[x][i] = group_sum<16>(apa[x][i]);
            aek[x][i] = group_sum<16>(aek[x][i]);
          }
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            apw[x][q] = group_sum<16>(apw[x][q]);
            aekt[x][q] = group_sum<16>(aekt[x][q]);
          }
          if ((lane & 15) == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int n = n0 + i;
              sPA[wave][n] += apa[x][i];
              sEK[wave][n] += aek[x][i];
              if ((i & 1) == 0 && n >= nreal) {
                sPW[wave][(n - nreal) >> 1] += apw[x][i >> 1];
                sEKth[wave][(n - nreal) >> 1] += aekt[x][i >> 1];
              }
            }
          }
        }
      };
      if (COORD) zero_rows();
      for (int blk = wave; blk < NBN * NBJ; blk += NW) {
        const int tn0 = (COORD ? blk % NBN : blk / NBJ) * BN, tj0 = (COORD ? blk / NBN : blk % NBJ) * BJ;
        // key tiles of the block: per-row decay takes tiles NBJ apart, so that a wave holds
        // an early and a late key tile (the late ones carry the tails: more work)
        auto ktile = [&](int y) { return COORD ? blk / NBN + y * NBJ : tj0 + y; };
        f32x4 ai[BN][BJ], ae[BN][BJ];
#pragma unroll
        for (int x = 0; x < BN; ++x)
#pragma unroll
          for (int y = 0; y < BJ; ++y) ai[x][y] = ae[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < S::QOC / 32; ++kk) {
          Frag<BF16> a[BN], bz[BJ];
#pragma unroll
          for (int x = 0; x < BN; ++x) a[x] = load_frag_tr<BF16>(sQ + (kk * 32) * NS + 16 * (tn0 + x), NS);
#pragma unroll
          for (int y = 0; y < BJ; ++y) bz[y] = load_frag_tr<BF16>(sZM + (kk * 32) * KS + 16 * ktile(y), KS);
#pragma unroll
          for (int x = 0; x < BN; ++x)
#pragma unroll
            for (int y = 0; y < BJ; ++y) mma<BF16>(ai[x][y], a[x], bz[y]);
        }
#pragma unroll
        for (int kk = 0; kk < S::PC / 32; ++kk) {
          Frag<BF16> bv[BJ], ah[BN];
#pragma unroll
          for (int y = 0; y < BJ; ++y)
            bv[y] = load_frag<BF16>(sV + (16 * ktile(y) + (lane & 15)) * PS + kk * 32 + 8 * (lane >> 4));
#pragma unroll
          for (int x = 0; x < BN; ++x) {
            ah[x] = load_frag<BF16>(sGh + (16 * (tn0 + x) + (lane & 15)) * PS + kk * 32 + 8 * (lane >> 4));
          }
#pragma unroll
          for (int x = 0; x < BN; ++x)
#pragma unroll
            for (int y = 0; y < BJ; ++y) {
              mma<BF16>(ae[x][y], ah[x], bv[y]);
            }
        }
#pragma unroll
        for (int x = 0; x < BN; ++x)
#pragma unroll
          for (int y = 0; y < BJ; ++y) dk_tile(tn0 + x, ktile(y), ai[x][y], ae[x][y], apa[x], aek[x], apw[x], aekt[x]);
        if (COORD && !SHARE_N) {
          flush_rows(tn0);
          zero_rows();
        }
      }
      if (COORD && SHARE_N && wave < NBN * NBJ) flush_rows((wave % NBN) * BN);
    }

    // ---------------------------------------------------------------- dC~ -> dC
    // lane l holds query row 16 tq + (l & 15) and state rows 16 tnn + 4 (l >> 4) + i
    // (blocked like dK~)
    auto dc_tile = [&](const int tnn, const int tq, const f32x4& ai, const f32x4& ae) {
      const int row = 16 * tq + (lane & 15), t = row / R, o = row % R, tg = t0 + t;
      const int n0 = 16 * tnn + 4 * (lane >> 4);
      const float cdt = sTcd[t];
      const float elt = COORD ? 0.f : sTel[t];
      float tokacc = 0.f, dc[4], qv[4], rpa[4], rpw[2] = {0.f, 0.f};
      load4<BF16>(sQ + row * NS + n0, qv);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = n0 + i;
        rpa[i] = 0.f;
        if (COORD) {
          const float er = sEr[n];
          const float cc = ai[i] + er * ae[i];
          dc[i] = cc;  // scaled by E_t (with the pair's turn) below
          const float dr = qv[i] * cc;
          tokacc += -sRate[n] * dr;                          // zero on static rows
          rpa[i] = -(n < p.n_static ? static_cast<float>(t + 1) : cdt) * dr;
        } else {
          dc[i] = ai[i] + elt * ae[i];
          tokacc += qv[i] * elt * ae[i];  // C~ o dC~ (inter part)
        }
      }
      if (COORD) {
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const int n = n0 + i;
          if (n >= nreal) {
            const int kp = (n - nreal) >> 1;
            const float er = sEr[n];
            const float ca = ai[i] + er * ae[i], cb = ai[i + 1] + er * ae[i + 1];
            const float dth = -qv[i] * cb + qv[i + 1] * ca;  // C~^T J dC~ (scaled form)
            tokacc += sOmega[kp] * dth;
            rpw[i >> 1] = cdt * dth;
          }
        }
        // dC~ = E_t cC, unfolded by R(+Theta_t) (table entries (a, b) = E_t (cos, sin))
        const float4 tq = *reinterpret_cast<const float4*>(sTQ + t * N + n0);
        const float f[4] = {tq.x, tq.y, tq.z, tq.w};
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const float a0 = dc[i], a1 = dc[i + 1];
          if (n0 + i >= nreal) {
            dc[i] = f[i] * a0 - f[i + 1] * a1;
            dc[i + 1] = f[i + 1] * a0 + f[i] * a1;
          } else {
            dc[i] = f[i] * a0;
            dc[i + 1] = f[i + 1] * a1;
          }
        }
      }
      if (tg < L && o < rout) store_bc(dCg, rout, b, t0, t, part ? h : g, o, n0, dc);
      if (COORD) {
#pragma unroll
        for (int i = 0; i < 4; ++i) rpa[i] = group_sum<16>(rpa[i]);
#pragma unroll
        for (int q = 0; q < 2; ++q) rpw[q] = group_sum<16>(rpw[q]);
        if ((lane & 15) == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int n = n0 + i;
            sPA[wave][n] += rpa[i];
            if ((i & 1) == 0 && n >= nreal) sPW[wave][(n - nreal) >> 1] += rpw[i >> 1];
          }
        }
      }
      tokacc = add_xor16(tokacc);
      tokacc = add_xor32(tokacc);
      tokacc = group_sum<R>(tokacc);
      if (lane < 16 && (lane % R) == 0) {
        if (COORD) sTok[wave][t] += tokacc;
        else sTT[wave][t] += tokacc;
      }
    };
    {
      constexpr int BN = S::CBLK ? 2 : 1, BQ = (S::CBLK || S::CPAIR) ? 2 : 1, NBQ = S::TQ / BQ;
      for (int blk = wave; blk < (S::TN / BN) * NBQ; blk += NW) {
        // per-row decay: n-blocks interleaved from the middle (pair rows, usually the upper
        // ones, cost more), so that the waves whose dK~ block holds real rows take pair rows
        // here and the other way round
        constexpr int NBC = S::TN / BN;
        const int ib = blk / NBQ;
        const int tn0 = (COORD && NBC % 2 == 0 ? (ib % 2 == 0 ? NBC / 2 + ib / 2 : ib / 2) : ib) * BN;
        const int tq0 = (blk % NBQ) * BQ;
        f32x4 ai[BN][BQ], ae[BN][BQ];
#pragma unroll
        for (int x = 0; x < BN; ++x)
#pragma unroll
          for (int y = 0; y < BQ; ++y) ai[x][y] = ae[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < QK / 32; ++kk) {
          Frag<BF16> a[BN], bz[BQ];
#pragma unroll
          for (int x = 0; x < BN; ++x) a[x] = load_frag_tr<BF16>(sK + (kk * 32) * NS + 16 * (tn0 + x), NS);
#pragma unroll
          for (int y = 0; y < BQ; ++y)
            bz[y] = load_frag<BF16>(sZM + (16 * (tq0 + y) + (lane & 15)) * KS + kk * 32 + 8 * (lane >> 4));
#pragma unroll
          for (int x = 0; x < BN; ++x)
#pragma unroll
            for (int y = 0; y < BQ; ++y) mma<BF16>(ai[x][y], a[x], bz[y]);
        }
#pragma unroll
        for (int kk = 0; kk < S::PC / 32; ++kk) {
          Frag<BF16> by[BQ], ah[BN];
#pragma unroll
          for (int y = 0; y < BQ; ++y)
            by[y] = load_frag<BF16>(sY + (16 * (tq0 + y) + (lane & 15)) * PS + kk * 32 + 8 * (lane >> 4));
#pragma unroll
          for (int x = 0; x < BN; ++x) {
            ah[x] = load_frag<BF16>(sSh + (16 * (tn0 + x) + (lane & 15)) * PS + kk * 32 + 8 * (lane >> 4));
          }
#pragma unroll
          for (int x = 0; x < BN; ++x)
#pragma unroll
            for (int y = 0; y < BQ; ++y) {
              mma<BF16>(ae[x][y], ah[x], by[y]);
            }
        }
#pragma unroll
        for (int x = 0; x < BN; ++x)
#pragma unroll
          for (int y = 0; y < BQ; ++y) dc_tile(tn0 + x, tq0 + y, ai[x][y], ae[x][y]);
      }
    }
    __syncthreads();

    // ---------------------------------------------------------------- step gradient
    // per-token d(loss)/d(L_t) contributions; the final-state term sits on the last
    // position of the chunk; dDelta_r = sum_{t >= r} dcd_t (reverse cumsum).
    if (wave == 0) {
      float tok = 0.f, dunw = 0.f;  // weighted dcd_t, and (head) the unweighted D_t
      float srcsum = 0.f, e = 0.f;
      if (COORD) {
        if (lane < QT) tok = wsum<WC>(sTok, lane);
        float eterm = 0.f;
        for (int n = lane; n < N; n += kWave) {
          const float en = sE[n] + wsum<WC>(sEK, n);
          eterm += -sRate[n] * en;
        }
        for (int k = lane; k < npairs; k += kWave) {
          const float et = sEth[k] + wsum<WC>(sEKth, k);
          eterm += sOmega[k] * et;
        }
        eterm = wave_sum(eterm);
        if (lane == QT - 1) tok += eterm;
      } else {
        // d(loss)/d(L_t) = rs_t - cs_t + tt_t - src_t, plus the final-state term e and
        // the sum of the source terms on the last position.  Summed over t >= r (the step
        // gradient of token r) the source terms of t >= r cancel; taking the sum as
        // suffix(rs - cs + tt) + prefix_{s < r}(src) + e keeps that cancellation (and the
        // same-token scores left out of rs and cs) out of fp32
        float src = 0.f;
        if (lane < QT) {
          const float rs = wsum<WH>(sRS, lane);
          const float cs = wsum<WH>(sCS, lane);
          const float tt = wsum<WH>(sTT, lane);
          src = wsum<WH>(sSrc, lane);
          dunw = rs - cs + tt;
        }
        for (int n = lane; n < N; n += kWave) e += sE[n];
        e = wave_sum(e);
        srcsum = wave_prefix_sum(src) - src;  // sources of the tokens before this one
      }
      // sum over t >= r, lane r, as a prefix sum of the lanes in reverse token order
      auto suffix_sum = [&](float v) {
        const float r = __shfl(lane < QT ? v : 0.f, lane < QT ? QT - 1 - lane : lane, kWave);
        const float pr = wave_prefix_sum(r);
        return __shfl(pr, lane < QT ? QT - 1 - lane : lane, kWave);
      };
      float rev;
      if (COORD) {
        rev = suffix_sum(tok);
      } else {
        dunw = suffix_sum(dunw) + srcsum + e;  // d(loss)/d(cumulative log-decay at r) summed over t >= r
        rev = -Ah * dunw;
      }
      const int t = t0 + lane;
      if (lane < QT && t < L) {
        const float raw = COORD ? sRaw2[COORD ? par : 0][lane] : raw_l;
        o_ddt = p.softplus ? rev * sigmoid_f32(raw) : rev;
        if (S::TE) {
          o_dg = wsum<WT>(sDg, lane);
          o_db = wsum<WT>(sDb, lane);
        }
      }
      if (!COORD && p.part) {
        // dA_h partial = sum_t (-cd_t) D_t = -sum_r Delta_r sum_{t >= r} D_t
        const float v = wave_sum(lane < QT ? -dl * dunw : 0.f);
        if (lane == 0) sPartOut[0] = v;
      }
    }
    // parameter partials of this chunk: with per-row decay on wave 1, beside wave 0's step
    // gradient (both read only the per-wave sums that the dC~ barrier published, and the
    // next item's first barrier waits for both), stored straight to the workspace
    if (p.part) {
      const int na = (COORD && !p.head_rates) ? nreal + npairs : 1;
      if (COORD) {
        float* dst = p.part + ((size_t)slice * nch + c) * p.npart;
        if (wave == 1) {
          // row n = n0 + lane; a pair's two rows sit in lanes (l, l ^ 1) (n_real is even)
          float hsum = 0.f;
          for (int n0 = 0; n0 < N; n0 += kWave) {
            const int n = n0 + lane;
            float v = 0.f;
            if (n < N) {
              const float en = sE[n] + wsum<WC>(sEK, n);
              v = wsum<WC>(sPA, n) - (n < p.n_static ? sCn2[par][1] : sCn2[par][0]) * en;
            }
            const float other = swap_adjacent_lanes(v);
            // slot of row n (a pair's first row: the pair's); formed here each item (hoisted
            // out of the item loop, the compiler keeps it in a spilled register)
            int slot = n < nreal ? n : nreal + ((n - nreal) >> 1);
            asm volatile("" : "+v"(slot));
            if (p.head_rates) hsum += v;
            else if (n < nreal) dst[slot] = v;
            else if (n < N && ((n - nreal) & 1) == 0) dst[slot] = v + other;
          }
          if (p.head_rates) {
            hsum = wave_sum(hsum);
            if (lane == 0) dst[0] = hsum;
          } else {
            for (int k = lane; k < npairs; k += kWave) {
              const float et = sEth[k] + wsum<WC>(sEKth, k);
              dst[na + k] = wsum<WC>(sPW, k) + sCn2[par][0] * et;
            }
          }
          if (lane == 0) dst[na + npairs] = wsum1<NW>(sMisc);
        }
      } else if (tid == 0) {
        sPartOut[na + npairs] = wsum1<NW>(sMisc);
      }
    }
    if (COORD && tid >= TT0 && nxt < nitems) make_tables(nxt, par ^ 1);
    prev = item;
  }  // items
  __syncthreads();
  if (prev >= 0) flush_scalars(prev);
}

// ============================================================== group sums of dB / dC
// dB and dC of a head group are the sums of its heads' partials (io dtype), added in head
// order in fp32 (deterministic).  One thread per 4-element piece of a (batch, token, group,
// row).
template <bool BF16>
__global__ __launch_bounds__(256) void ssm_bwd_group_sum(BwdParams p, int R) {
  using T = typename Elem<BF16>::T;
  const int N = p.n_real + 2 * p.n_pairs, H = p.H, G = p.G, hpg = H / G;
  const long total = (long)p.batch * p.L * G * R * (N / 4);
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
    const int n4 = (int)(i % (N / 4)) * 4;
    long r = i / (N / 4);
    const int rr = (int)(r % R);
    r /= R;
    const int g = (int)(r % G);
    const long bt = r / G;  // batch * L + token
#pragma unroll 1
    for (int which = 0; which < 2; ++which) {
      // partials hold R rows per token; dB has rank_in rows, dC rank_out
      const int rows = which ? p.rout : p.rin;
      if (rr >= rows) continue;
      const T* part = static_cast<const T*>(which ? p.dCh : p.dBh);
      T* out = static_cast<T*>(which ? p.dC : p.dB);
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      for (int k = 0; k < hpg; ++k) {
        float a[4];
        load4<BF16>(part + ((bt * H + g * hpg + k) * R + rr) * N + n4, a);
        v[0] += a[0]; v[1] += a[1]; v[2] += a[2]; v[3] += a[3];
      }
      store4<BF16>(out + ((bt * G + g) * rows + rr) * N + n4, v);
    }
  }
}

// ============================================================== carried token
// Gradients of the token before the sequence, whose write beta_0 B_prev X_prev enters at
// token 0:  dX_prev = beta_0 B_prev^T g_0  and  dB_prev = beta_0 g_0 X_prev^T, with g_0 the
// boundary adjoint of chunk 0 (the adjoint at token 0).  One workgroup per (batch, group):
// dB_prev is the sum over the group's heads, added in head order.
constexpr int kPrevMaxNP = 128 * 64;  // N x P of the largest variant
template <bool BF16>
__global__ __launch_bounds__(256) void ssm_bwd_prev(BwdParams p) {
  using T = typename Elem<BF16>::T;
  __shared__ float sG[kPrevMaxNP];
  const int N = p.n_real + 2 * p.n_pairs, P = p.P, R = p.rin, H = p.H, G = p.G, hpg = H / G;
  const int b = blockIdx.x / G, g = blockIdx.x % G, tid = threadIdx.x;
  const T* Bp = static_cast<const T*>(p.B_prev) + ((size_t)b * G + g) * R * N;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};  // dB_prev entries tid + 256 j (R N <= 1024)
  for (int k = 0; k < hpg; ++k) {
    const int h = g * hpg + k, slice = b * H + h;
    const T* g0 = static_cast<const T*>(p.gseg) + (size_t)slice * (p.nchunks + 1) * N * P;
    const T* xp = static_cast<const T*>(p.x_prev) + (size_t)slice * R * P;
    const float beta0 = p.beta[(size_t)b * p.L * H + h];
    __syncthreads();
    for (int i = tid; i < N * P; i += 256) sG[i] = to_f32(g0[i]);
    __syncthreads();
    if (p.dx_prev)
      for (int i = tid; i < R * P; i += 256) {
        const int r = i / P, q = i % P;
        float v = 0.f;
        for (int n = 0; n < N; ++n) v += to_f32(Bp[r * N + n]) * sG[n * P + q];
        static_cast<T*>(p.dx_prev)[(size_t)slice * R * P + i] = from_f32<T>(beta0 * v);
      }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid + 256 * j;
      if (i < R * N) {
        const int r = i / N, n = i % N;
        float v = 0.f;
        for (int q = 0; q < P; ++q) v += sG[n * P + q] * to_f32(xp[r * P + q]);
        acc[j] += beta0 * v;
      }
    }
  }
  if (p.dB_prev)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid + 256 * j;
      if (i < R * N) static_cast<T*>(p.dB_prev)[((size_t)b * G + g) * R * N + i] = from_f32<T>(acc[j]);
    }
}

// ============================================================== parameter sums
// One wave per output: lane l sums the partials j = l, l + 64, ... of the (batch,
// chunk) items in order, then a fixed butterfly combines the lanes, so the result
// does not depend on timing.
__global__ __launch_bounds__(256) void ssm_bwd_params(BwdParams p, int nA) {
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int per_head = p.npart;
  if (i >= p.H * per_head) return;
  const int h = i / per_head, k = i % per_head;
  const int nch = p.nchunks, items = p.batch * nch;
  float acc = 0.f;
  for (int j = lane; j < items; j += kWave) {
    const int b = j / nch, c = j % nch;
    acc += p.part[((size_t)(b * p.H + h) * nch + c) * per_head + k];
  }
  acc = wave_sum(acc);
  if (lane != 0) return;
  if (k < nA) {
    if (p.dA) p.dA[(size_t)h * nA + k] = acc;
  } else if (k < nA + p.n_pairs) {
    if (p.domega) p.domega[(size_t)h * p.n_pairs + (k - nA)] = acc;
  } else {
    if (p.dD) p.dD[h] = acc;
  }
}

// ------------------------------------------------------------------ dispatch
// (io bf16?, N, P, R, keys per token, tokens per chunk, per-row decay, ranks differ)
#define SSM_BWD_VARIANTS(X)            \
  X(false, 16, 16, 1, 1, 64, false, false)    \
  X(false, 32, 16, 1, 1, 64, false, false)    \
  X(false, 32, 16, 2, 2, 32, false, false)    \
  X(false, 16, 16, 1, 2, 16, true, false)     \
  X(false, 32, 16, 1, 2, 16, true, false)     \
  X(false, 32, 16, 2, 4, 16, true, false)     \
  X(false, 32, 16, 1, 1, 32, true, false)     \
  X(false, 32, 16, 2, 2, 16, true, false)     \
  X(true, 64, 64, 1, 1, 64, false, false)     \
  X(true, 128, 64, 1, 1, 64, false, false)    \
  X(true, 64, 64, 4, 4, 16, false, false)     \
  X(true, 64, 64, 1, 2, 16, true, false)      \
  X(true, 64, 64, 2, 4, 16, true, false)     \
  /* per-row decay with plain writes */     \
  X(true, 64, 64, 1, 1, 32, true, false)     \
  X(true, 64, 64, 2, 2, 16, true, false)     \
  /* write and readout ranks that differ */ \
  X(false, 32, 16, 2, 2, 32, false, true)    \
  X(false, 32, 16, 2, 4, 16, true, true)     \
  X(true, 64, 64, 4, 4, 16, false, true)     \
  X(true, 64, 64, 2, 4, 16, true, true)

bool bwd_variant_exists(const BwdKey& k) {
#define SSM_BWD_MATCH(BF, NN, PP, RR, KRR, QTT, CO, SP)                                      \
  if (k.bf16 == BF && k.N == NN && k.P == PP && k.R == RR && k.KR == KRR && k.QT == QTT &&   \
      k.coord == CO && k.split == SP)                                                        \
    return true;
  SSM_BWD_VARIANTS(SSM_BWD_MATCH)
#undef SSM_BWD_MATCH
  return false;
}

#ifndef ADJ_NT
#define ADJ_NT 1024
#endif
// Chunk-gradient workgroup size: 512 threads, or 256 for head decay with narrow states
// (N <= 64), where two workgroups of 256 share a compute unit (LDS and registers allow
// it) and hide each other's latencies (SSD-MIMO 0.78 -> 0.67 ms; SSD SISO with N = 128
// and the per-row variants run best at 512)
#define CHUNK_NT(NN, CO) ((!(CO) && (NN) <= 64) ? 256 : 512)
#define ADJ_PB(PP) (PP)

// compute units of the current device (cached per device)
static int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// workgroups of `kernel` resident per compute unit (cached by the caller)
static int blocks_per_cu(const void* kernel, int nthreads, std::atomic<int>& cache) {
  int v = cache.load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, kernel, nthreads, 0) != hipSuccess || v <= 0)
      v = 1;
    cache.store(v, std::memory_order_relaxed);
  }
  return v;
}

// the boundary-adjoint sweep's local pass: C keys and dy values over the ranges of
// segments 1 .. nseg-1
static LocalParams adj_local_params(const BwdParams& p) {
  LocalParams l{};
  l.key = p.C; l.val = p.dy; l.dt = p.dt; l.A = p.A; l.omega = p.omega;
  l.out = p.gloc; l.delta = p.gdel; l.rk = p.rout;
  l.batch = p.batch; l.L = p.L; l.H = p.H; l.G = p.G; l.P = p.P; l.n_real = p.n_real;
  l.n_static = p.n_static;
  l.n_pairs = p.n_pairs; l.softplus = p.softplus; l.head_rates = p.head_rates;
  l.nseg = p.nseg; l.seg_tokens = p.seg_tokens; l.nsub = p.nsub; l.lsub = p.lsub;
  return l;
}

hipError_t launch_bwd(const BwdKey& k, const BwdParams& p, hipStream_t stream,
                      void* const* events) {
  const int slices = p.batch * p.H;
  if (slices == 0 || p.nchunks == 0) return hipSuccess;
  auto mark = [&](int i) {
    if (events && events[i]) (void)hipEventRecord(static_cast<hipEvent_t>(events[i]), stream);
  };
  const int nA = k.coord && !p.head_rates ? p.n_real + p.n_pairs : 1;
#define SSM_BWD_LAUNCH(BF, NN, PP, RR, KRR, QTT, CO, SP)                                      \
  if (k.bf16 == BF && k.N == NN && k.P == PP && k.R == RR && k.KR == KRR && k.QT == QTT &&    \
      k.coord == CO && k.split == SP) {                                                       \
    constexpr int PB = ADJ_PB(PP);                                                            \
    mark(0);                                                                                  \
    const int agrid = slices * (PP / PB) * p.nseg;                                            \
    if (p.nseg > 1) {                                                                         \
      launch_local<BF, NN, RR, false, CO, true>(adj_local_params(p), stream);                 \
      const long total = (long)slices * (NN / 2) * PP;                                        \
      const int cb = (int)std::min<long>((total + 255) / 256, 2048);                          \
      hipLaunchKernelGGL(ssm_adj_combine, dim3(cb), dim3(256), 0, stream, p, CO ? 1 : 0);     \
    }                                                                                         \
    hipLaunchKernelGGL((ssm_bwd_adjoint<BF, NN, PB, RR, QTT, CO, ADJ_NT>), dim3(agrid),       \
                       dim3(ADJ_NT), 0, stream, p);                                           \
    if (p.dx_prev || p.dB_prev)                                                               \
      hipLaunchKernelGGL(ssm_bwd_prev<BF>, dim3(p.batch * p.G), dim3(256), 0, stream, p);     \
    mark(1);                                                                                  \
    {                                                                                         \
      static std::atomic<int> occ{0};                                                         \
      const void* kfn = reinterpret_cast<const void*>(                                        \
          &ssm_bwd_chunk<BF, NN, PP, RR, KRR, QTT, CO, CHUNK_NT(NN, CO), SP>);                \
      const int items = slices * p.nchunks;                                                   \
      int grid = std::min(items, device_cus() * blocks_per_cu(kfn, CHUNK_NT(NN, CO), occ));   \
      if (p.chunk_grid_cap > 0) grid = std::min(grid, p.chunk_grid_cap);                      \
      hipLaunchKernelGGL((ssm_bwd_chunk<BF, NN, PP, RR, KRR, QTT, CO, CHUNK_NT(NN, CO), SP>),     \
                         dim3(grid), dim3(CHUNK_NT(NN, CO)), 0, stream, p);                   \
    }                                                                                         \
    if constexpr (CO) launch_bwd_exact<BF, NN, PP, RR, QTT>(p, device_cus(), stream);         \
    if (p.dBh) {                                                                              \
      const long total = (long)p.batch * p.L * p.G * RR * (NN / 4);                          \
      const int gb = (int)std::min<long>((total + 255) / 256, 4096);                         \
      hipLaunchKernelGGL(ssm_bwd_group_sum<BF>, dim3(gb), dim3(256), 0, stream, p, RR);      \
    }                                                                                         \
    mark(2);                                                                                  \
    hipLaunchKernelGGL(ssm_bwd_params, dim3((p.H * p.npart + 3) / 4), dim3(256), 0,          \
                       stream, p, nA);                                                        \
    mark(3);                                                                                  \
    return hipGetLastError();                                                                 \
  }
  SSM_BWD_VARIANTS(SSM_BWD_LAUNCH)
#undef SSM_BWD_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace ssm
