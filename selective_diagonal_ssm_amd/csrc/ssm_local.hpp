// ssm_local.hpp -- local pass of the sequence segments (gfx950), shared by the forward
// scan and the boundary-adjoint sweep of the reverse pass.
//
// Forward: the state at the end of a token range [ta, tb] from a zero start,
//   S = sum_{tau in [ta, tb]} Phi(tb, tau) W_tau,
//   W_tau = gamma_tau B_tau X_tau + beta_tau B_{tau-1} X_{tau-1}   (plain write: B_tau X_tau),
// where Phi(tb, tau) scales row n by e^{-A_n d_tau} and turns pair k by R(omega_k d_tau),
// d_tau = sum_{r = tau+1 .. tb} Delta_r.  The two writes of X_tau (the gamma term at tau,
// the beta term at tau + 1) fold into one key row per (token, rank):
//   K_tau = [tau >= ta] gamma_tau Phi(tb, tau) B_tau + [tau < tb] beta_{tau+1} Phi(tb, tau+1) B_tau,
// so S = sum_{tau = ta-1 .. tb} K_tau^T X_tau (token ta - 1 carries only its beta term).
//
// Adjoint (g_t = C_t dy_t + A_{t+1}^T g_{t+1}): the adjoint at ta from a zero adjoint
// after tb,
//   G = sum_{t in [ta, tb]} Phi(t, ta)^T C_t dy_t,
// Phi(t, ta)^T scaling row n by e^{-A_n d'_t} and turning pair k by R(-omega_k d'_t),
// d'_t = sum_{r = ta+1 .. t} Delta_r: keys e^{-A d'} R(-omega d') C_t, values dy_t.
//
// Either way the range is one contraction over its tokens, with no sequential
// dependence.  Each wave takes steps of 32 key rows on its own (wave-private LDS, no
// workgroup barrier inside the loop; the next step's loads are in flight while a step
// is staged), and the four waves' partial states are added in a fixed order at the
// end.  The range's summed step goes out with it for the segment chain: forward
// sum_{r = ta..tb} Delta_r, adjoint sum_{r = ta+1..tb+1} Delta_r (the transition from
// ta to the next range's first token).
//
// Sources: "When a Diagonal State Is Not Enough" (sungsoo.github.io), Part 01 and
// Part 03 (recurrence, Theorem 8 rotating pairs, two-endpoint writes).
#pragma once
#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

namespace ssm {

template <bool BF16, int N, int PBL, int R, bool TE, bool COORD>
struct LocalShape {
  using T = typename Elem<BF16>::T;
  static constexpr int VEC = Elem<BF16>::kVec;
  static constexpr int PAD = 16 / static_cast<int>(sizeof(T));
  static constexpr int QL = 32 / R;  // tokens per step (32 key rows)
  static constexpr int KS = N + PAD, VS = PBL + PAD;
  static constexpr int NV = N / VEC, PV = PBL / VEC;
  static constexpr int TN = N / 16, TP = PBL / 16;
  static constexpr int BI = QL * NV;      // key items per step: (token, n-vector), all ranks
  static constexpr int XI = QL * R * PV;  // value vectors per step
  static constexpr int BI_PER = (BI + 63) / 64, XI_PER = (XI + 63) / 64;
  static constexpr int STAGE_BYTES = 4 * 32 * (KS + VS) * static_cast<int>(sizeof(T));
  static constexpr int RED_BYTES = 3 * N * PBL * 4;  // partial states of waves 1..3
  static constexpr int SMEM = STAGE_BYTES > RED_BYTES ? STAGE_BYTES : RED_BYTES;
  static_assert(32 % R == 0 && N % 16 == 0 && PBL % 16 == 0, "unsupported local shape");
};

template <bool BF16, int N, int PBL, int R, bool TE, bool COORD, bool ADJ>
__global__ __launch_bounds__(256) void ssm_local(LocalParams p) {
  static_assert(!(ADJ && TE), "the adjoint has no two-endpoint term");
  using S = LocalShape<BF16, N, PBL, R, TE, COORD>;
  using T = typename S::T;
  constexpr int VEC = S::VEC, QL = S::QL, KS = S::KS, VS = S::VS, NV = S::NV, PV = S::PV;
  constexpr int LM = kLocalMaxTokens;
  constexpr float kLog2e = 1.4426950408889634f;
  __shared__ __align__(16) unsigned char smem[S::SMEM];
  __shared__ float sD[LM];                                   // Delta, then d (or d')
  __shared__ float sGa[TE ? LM : 1], sBe[TE ? LM : 1];
  __shared__ float sBlk[LM / 64];
  // per-row rates (log2 e scaled): dynamic rows in sRate (exponent rate x summed step),
  // static rows in sRateS (exponent rate x token count); each row has one of them nonzero
  __shared__ float sRate[COORD ? N : 1], sRateS[COORD ? N : 1], sOm[COORD ? N / 2 + 1 : 1];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nlp = p.P / PBL, nsegl = p.nseg - 1;
  const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const int pblk = lid % nlp;
  int rest = lid / nlp;
  const int sub = rest % p.nsub;
  rest /= p.nsub;
  const int segi = rest % nsegl, slice = rest / nsegl;
  const int seg = segi + (ADJ ? 1 : 0);  // the adjoint needs segments 1.., the forward 0..nseg-2
  const int b = slice / p.H, h = slice % p.H, g = h / (p.H / p.G);
  const int L = p.L, H = p.H, G = p.G, P = p.P, p0 = pblk * PBL;
  const int s0 = seg * p.seg_tokens;
  const int ta = s0 + sub * p.lsub;
  const int tb = min(min(ta + p.lsub, s0 + p.seg_tokens), L) - 1;
  const int len = max(tb - ta + 1, 0);  // ranges past the sequence end are empty
  const size_t unit = ((size_t)slice * nsegl + segi) * p.nsub + sub;

  if (COORD) {
    const int na = p.n_real + p.n_pairs, nreal = p.n_real;
    for (int n = tid; n < N; n += 256) {
      float r;
      if (p.head_rates) r = p.A[h];
      else if (n < nreal) r = p.A[(size_t)h * na + n];
      else r = p.A[(size_t)h * na + nreal + ((n - nreal) >> 1)];
      const bool st = n < p.n_static;
      sRate[n] = st ? 0.f : r * kLog2e;
      sRateS[n] = st ? r * kLog2e : 0.f;
    }
    for (int k = tid; k < p.n_pairs; k += 256) sOm[k] = p.omega[(size_t)h * p.n_pairs + k];
  }
  const float* dtg = p.dt + (size_t)b * L * H + h;
  for (int i = tid; i < len; i += 256) {
    const float raw = dtg[(size_t)(ta + i) * H];
    // the adjoint's decays run over (ta, t]: the range's first step is left out
    sD[i] = (ADJ && i == 0) ? 0.f : (p.softplus ? softplus_f32(raw) : raw);
    if (TE) {
      sGa[i] = p.gamma[((size_t)b * L + ta + i) * H + h];
      sBe[i] = p.beta[((size_t)b * L + ta + i) * H + h];
    }
  }
  __syncthreads();
  // forward: d_i = sum of Delta over the tokens after i (exclusive suffix sums in blocks
  // of 64 tokens, lanes in reverse token order, plus the later blocks' totals);
  // adjoint: d'_i = sum over the tokens up to i (inclusive prefix sums, plus the
  // earlier blocks' totals)
  const int nblk = (len + 63) / 64;
  for (int blk = wave; blk < nblk; blk += 4) {
    const int i = ADJ ? blk * 64 + lane : blk * 64 + 63 - lane;
    const float v = i < len ? sD[i] : 0.f;
    const float incl = wave_prefix_sum(v);
    if (lane == 63) sBlk[blk] = incl;
    if (i < len) sD[i] = ADJ ? incl : incl - v;
  }
  __syncthreads();
  for (int i = tid; i < len; i += 256) {
    float other = 0.f;
    if (ADJ)
      for (int k = 0; k < i / 64; ++k) other += sBlk[k];
    else
      for (int k = i / 64 + 1; k < nblk; ++k) other += sBlk[k];
    sD[i] += other;
  }
  if (tid == 0 && pblk == 0) {
    float tot = 0.f;
    for (int k = 0; k < nblk; ++k) tot += sBlk[k];
    if (ADJ && len > 0 && tb + 1 < L) {
      const float raw = dtg[(size_t)(tb + 1) * H];
      tot += p.softplus ? softplus_f32(raw) : raw;
    }
    p.delta[unit] = tot;
  }
  __syncthreads();

  // key / value rows per token: rk <= R (rows rk .. R-1 load as zero)
  const int rk = p.rk;
  const T* Kg = static_cast<const T*>(p.key) + ((size_t)b * L * G + g) * rk * N;
  const T* Vg = static_cast<const T*>(p.val) + ((size_t)b * L * H + h) * rk * P + p0;
  const int tsG = G * rk * N, tsH = H * rk * P;
  const T* Kp = (!ADJ && p.key_prev) ? static_cast<const T*>(p.key_prev) + ((size_t)b * G + g) * rk * N : nullptr;
  const T* Vp = (!ADJ && p.val_prev) ? static_cast<const T*>(p.val_prev) + ((size_t)b * H + h) * rk * P + p0 : nullptr;
  T* kw = reinterpret_cast<T*>(smem) + wave * 32 * KS;
  T* vw = reinterpret_cast<T*>(smem) + 4 * 32 * KS + wave * 32 * VS;
  const float ah = COORD ? 0.f : p.A[h] * kLog2e;
  const int i_first = TE ? -1 : 0;  // relative token of the first key row
  const int nsteps = len > 0 ? (len - i_first + QL - 1) / QL : 0;
  const float rsg = ADJ ? -1.f : 1.f;  // rotation sense: R(+phi) forward, R(-phi) adjoint
  // a loaded vector, or zero (selected per component: a whole-struct select can be
  // lowered through scratch memory)
  auto keep = [](bool ok, const uint4& v) {
    return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
  };

  f32x4 acc[S::TN][S::TP];
#pragma unroll
  for (int a = 0; a < S::TN; ++a)
#pragma unroll
    for (int c = 0; c < S::TP; ++c) acc[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // raw key vectors (all ranks of a (token, n-vector) item) and value vectors of one
  // step; loads are branch-free (clamped token, zero for rows outside the range)
  uint4 rb[S::BI_PER][R], rx[S::XI_PER];
  auto load = [&](int k) {
    const int i0 = i_first + k * QL;
#pragma unroll
    for (int q = 0; q < S::BI_PER; ++q) {
      const int u = lane + 64 * q;
      const int j = u / NV, v = u % NV;
      const int t = ta + i0 + j;
      const bool ok = u < S::BI && i0 + j < len && t >= 0;
      // the carried token before the sequence (forward, two-endpoint writes)
      const bool okp = !ADJ && u < S::BI && t == -1 && Kp != nullptr;
      const int tc = ok ? t : ta;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int rc = r < rk ? r : 0;
        const uint4 val = *reinterpret_cast<const uint4*>(
            (okp ? Kp : Kg + (size_t)tc * tsG) + rc * N + v * VEC);
        rb[q][r] = keep((ok || okp) && r < rk, val);
      }
    }
#pragma unroll
    for (int q = 0; q < S::XI_PER; ++q) {
      const int u = lane + 64 * q;
      const int jr = u / PV, pv = u % PV;
      const int j = jr / R, r = jr % R;
      const int t = ta + i0 + j;
      const bool ok = u < S::XI && i0 + j < len && t >= 0 && r < rk;
      const bool okp = !ADJ && u < S::XI && t == -1 && r < rk && Vp != nullptr;
      const int tc = ok ? t : ta, rc = (ok || okp) ? r : 0;
      const uint4 val = *reinterpret_cast<const uint4*>((okp ? Vp : Vg + (size_t)tc * tsH) + rc * P + pv * VEC);
      rx[q] = keep(ok || okp, val);
    }
  };

  // key rows of one step into the wave's LDS: K_tau = coefficient (x) key vector
  auto stage = [&](int k) {
    const int i0 = i_first + k * QL;
#pragma unroll
    for (int q = 0; q < S::BI_PER; ++q) {
      const int u = lane + 64 * q;
      if (u >= S::BI) break;
      const int j = u / NV, v = u % NV, n0 = v * VEC;
      const int i = i0 + j;
      // the gamma term (write at token i) and the beta term (write at token i + 1)
      const bool h0 = i >= 0 && i < len;
      const bool h1 = TE && i + 1 < len;
      const float d0 = h0 ? sD[i] : 0.f, d1 = h1 ? sD[i + 1] : 0.f;
      // the token counts that go with d0, d1 (static rows): tokens after i in the range
      // (forward), tokens in (ta, ta + i] (adjoint)
      const float n0c = h0 ? static_cast<float>(ADJ ? i : len - 1 - i) : 0.f;
      const float n1c = h1 ? static_cast<float>(ADJ ? i + 1 : len - 2 - i) : 0.f;
      const float g0 = h0 ? (TE ? sGa[i] : 1.f) : 0.f, g1 = h1 ? sBe[i + 1] : 0.f;
      float cf[VEC], sf[VEC];  // per-row factor; pairs: (cos-part, sin-part) on both rows
      if (!COORD) {
        float c = g0 * __builtin_amdgcn_exp2f(-ah * d0);
        if (TE) c += g1 * __builtin_amdgcn_exp2f(-ah * d1);
#pragma unroll
        for (int e = 0; e < VEC; ++e) { cf[e] = c; sf[e] = 0.f; }
      } else {
#pragma unroll
        for (int e = 0; e < VEC; e += 2) {
          const int n = n0 + e;
          if (n >= p.n_real) {
            const float a = sRate[n], om = sOm[(n - p.n_real) >> 1];
            float s0v, c0v, s1v = 0.f, c1v = 0.f;
            fast_sincos(om * d0, &s0v, &c0v);
            const float w0 = g0 * __builtin_amdgcn_exp2f(-a * d0);
            float cc = w0 * c0v, ss = w0 * s0v;
            if (TE) {
              fast_sincos(om * d1, &s1v, &c1v);
              const float w1 = g1 * __builtin_amdgcn_exp2f(-a * d1);
              cc += w1 * c1v;
              ss += w1 * s1v;
            }
            cf[e] = cc; sf[e] = rsg * ss; cf[e + 1] = cc; sf[e + 1] = rsg * ss;
          } else {
#pragma unroll
            for (int f = 0; f < 2; ++f) {
              const float a = sRate[n + f], as = sRateS[n + f];
              float c = g0 * __builtin_amdgcn_exp2f(-a * d0 - as * n0c);
              if (TE) c += g1 * __builtin_amdgcn_exp2f(-a * d1 - as * n1c);
              cf[e + f] = c; sf[e + f] = 0.f;
            }
          }
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float bv[VEC], kv[VEC];
        unpack<BF16>(rb[q][r], bv);
#pragma unroll
        for (int e = 0; e < VEC; e += 2) {
          // [[c, -s], [s, c]] on a pair (s = 0 on real rows)
          kv[e] = cf[e] * bv[e] - sf[e] * bv[e + 1];
          kv[e + 1] = sf[e] * bv[e] + cf[e + 1] * bv[e + 1];
        }
        *reinterpret_cast<uint4*>(kw + (j * R + r) * KS + n0) = pack<BF16>(kv);
      }
    }
#pragma unroll
    for (int q = 0; q < S::XI_PER; ++q) {
      const int u = lane + 64 * q;
      if (u >= S::XI) break;
      const int jr = u / PV, pv = u % PV;
      *reinterpret_cast<uint4*>(vw + jr * VS + pv * VEC) = rx[q];
    }
  };

  int k = wave;
  if (k < nsteps) load(k);
  for (; k < nsteps; k += 4) {
    stage(k);
    if (k + 4 < nsteps) load(k + 4);
    // the wave's own LDS writes before its transposed reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
    for (int tn = 0; tn < S::TN; ++tn) {
      const auto fk = load_frag_tr<BF16>(kw + 16 * tn, KS);
#pragma unroll
      for (int tp = 0; tp < S::TP; ++tp) {
        const auto fv = load_frag_tr<BF16>(vw + 16 * tp, VS);
        mma<BF16>(acc[tn][tp], fv, fk);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  }

  // partial states of waves 1..3 through LDS, added to wave 0's in order;
  // acc[tn][tp][i] = S[n = 16 tn + (lane & 15)][p = 16 tp + 4 (lane >> 4) + i]
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
  if (wave > 0) {
#pragma unroll
    for (int tn = 0; tn < S::TN; ++tn)
#pragma unroll
      for (int tp = 0; tp < S::TP; ++tp) {
        const int n = 16 * tn + (lane & 15), pl = 16 * tp + 4 * (lane >> 4);
        *reinterpret_cast<float4*>(red + ((wave - 1) * N + n) * PBL + pl) =
            make_float4(acc[tn][tp][0], acc[tn][tp][1], acc[tn][tp][2], acc[tn][tp][3]);
      }
  }
  __syncthreads();
  if (wave == 0) {
    float* dst = p.out + unit * N * P + p0;
#pragma unroll
    for (int tn = 0; tn < S::TN; ++tn)
#pragma unroll
      for (int tp = 0; tp < S::TP; ++tp) {
        const int n = 16 * tn + (lane & 15), pl = 16 * tp + 4 * (lane >> 4);
        float4 s = make_float4(acc[tn][tp][0], acc[tn][tp][1], acc[tn][tp][2], acc[tn][tp][3]);
#pragma unroll
        for (int w = 0; w < 3; ++w) {
          const float4 o = *reinterpret_cast<const float4*>(red + (w * N + n) * PBL + pl);
          s.x += o.x; s.y += o.y; s.z += o.z; s.w += o.w;
        }
        *reinterpret_cast<float4*>(dst + (size_t)n * P + pl) = s;
      }
  }
}

// launch over every (slice, segment, range, value block): 64-column value blocks when
// the state has at most 64 rows, else 32 (or 16)
template <bool BF16, int N, int R, bool TE, bool COORD, bool ADJ>
void launch_local(const LocalParams& p, hipStream_t stream) {
  const int units = p.batch * p.H * (p.nseg - 1) * p.nsub;
  if (units <= 0) return;
  if (N <= 64 && p.P % 64 == 0)
    hipLaunchKernelGGL((ssm_local<BF16, N, 64, R, TE, COORD, ADJ>), dim3(units * (p.P / 64)),
                       dim3(256), 0, stream, p);
  else if (p.P % 32 == 0)
    hipLaunchKernelGGL((ssm_local<BF16, N, 32, R, TE, COORD, ADJ>), dim3(units * (p.P / 32)),
                       dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((ssm_local<BF16, N, 16, R, TE, COORD, ADJ>), dim3(units * (p.P / 16)),
                       dim3(256), 0, stream, p);
}

}  // namespace ssm
