// ssm_decode.hip -- single-token recurrent step of the state-mediated selective SSM
// kernel for gfx950 (the step-by-step inference mode of the same recurrence):
//
//   h <- A_t h + gamma_t B_t X_t + beta_t B_{t-1} X_{t-1},     y_t = C_t^T h + D_h X_t
//
// with A_t block diagonal (real rows exp(-Delta A_n), rotating pairs
// rho R(Delta omega)).  The step streams the N x P fp32 state of every (batch, head)
// slice once in and once out; everything else (x, B, C, the scalars) is a few
// hundred bytes per slice.  One workgroup per slice: each thread owns 4 adjacent
// value columns (16-byte state accesses, P/4 threads cover a row) of whole row pairs
// (a rotating pair needs both of its rows), the row pairs are spread over the
// 256/(P/4) thread groups, the state of several pairs is loaded before any is
// updated (memory-level parallelism), and y is summed over the groups in a fixed
// order through LDS, so the result is bitwise reproducible.
//
// Sources: "When a Diagonal State Is Not Enough" (sungsoo.github.io), Part 01 (the
// recurrence h_t = A_t h_{t-1} + B_t u_t, y_t = C_t h_t + D_t u_t, run one token at a
// time with constant state at inference) and Part 03 (rotating pairs, two-endpoint
// writes of the HybridMamba rows).
#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

namespace ssm {

namespace {

template <bool BF16>
__device__ __forceinline__ void load_cols4(const typename Elem<BF16>::T* p, float* v) {
  if constexpr (BF16) {
    const uint2 r = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(r.x << 16);
    v[1] = __uint_as_float(r.x & 0xffff0000u);
    v[2] = __uint_as_float(r.y << 16);
    v[3] = __uint_as_float(r.y & 0xffff0000u);
  } else {
    const float4 r = *reinterpret_cast<const float4*>(p);
    v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
  }
}

template <bool BF16>
__device__ __forceinline__ void store_cols4(typename Elem<BF16>::T* p, const float* v) {
  if constexpr (BF16) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// two adjacent elements (a row pair's entries of one B or C row) as floats
template <bool BF16>
__device__ __forceinline__ float2 load_pair(const typename Elem<BF16>::T* p) {
  if constexpr (BF16) {
    const uint32_t r = *reinterpret_cast<const uint32_t*>(p);
    return make_float2(__uint_as_float(r << 16), __uint_as_float(r & 0xffff0000u));
  } else {
    return *reinterpret_cast<const float2*>(p);
  }
}

}  // namespace

// Workgroup barrier for data exchanged through LDS only: the global stores in
// flight (the updated state) need not complete before the workgroup proceeds.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// RMAX: bound on rank_in and rank_out of the variant (the per-thread x and y
// registers scale with it).  Global reads are written without branches (clamped
// indices; the surplus values are never used) so that they are all in flight
// together: a read inside a divergent branch is waited for before the branch ends.
// PREV: the previous token's write is given (two-endpoint, not the first token).
template <bool BF16, int RMAX, bool PREV>
__global__ __launch_bounds__(256) void ssm_decode_kernel(DecodeParams p) {
  using T = typename Elem<BF16>::T;
  constexpr int MP = kDecodePairs;  // row pairs whose state is loaded together
  extern __shared__ float lds[];

  // 256 / tps slices per workgroup, tps threads each
  const int NT = p.tps;
  const int sub = threadIdx.x / NT;
  const int slice = blockIdx.x * (256 / NT) + sub;
  const int nslices = p.batch * p.H;
  const bool live = slice < nslices;  // a tail workgroup may hold fewer slices
  const int sl = live ? slice : 0;
  const int b = sl / p.H, h = sl % p.H, g = h / (p.H / p.G);
  const int N = p.n_real + 2 * p.n_pairs, P = p.P, R = p.R, O = p.O, nreal = p.n_real;
  const int na = p.n_real + p.n_pairs;
  const int npair = N / 2;
  const int cpr = P / 4;         // threads per state row (host: 4 | P, P / 4 <= tps)
  const int groups = NT / cpr;   // row-pair groups; threads beyond cpr * groups idle
  const int tid = threadIdx.x % NT;
  const int c4 = (tid % cpr) * 4, grp = tid / cpr;
  const bool active = live && grp < groups;

  float* sTab = lds + sub * decode_lds_floats(N, R, O, P, NT);  // [N] row decay; pairs: rho cos, rho sin
  float* sB = sTab + N;            // [R][N] gamma_t B_t
  float* sBp = sB + R * N;         // [R][N] beta_t B_{t-1}
  float* sC = sBp + R * N;         // [O][N] C_t
  float* sY = sC + O * N;          // [O][groups][P]

  const T* x = static_cast<const T*>(p.x) + (size_t)sl * R * P;
  const T* Bm = static_cast<const T*>(p.B) + ((size_t)b * p.G + g) * R * N;
  const T* Cm = static_cast<const T*>(p.C) + ((size_t)b * p.G + g) * O * N;
  const T* xp = static_cast<const T*>(p.x_prev) + (size_t)sl * R * P;    // used iff PREV
  const T* Bp = static_cast<const T*>(p.B_prev) + ((size_t)b * p.G + g) * R * N;
  float* st = p.state + (size_t)sl * N * P;

  // ---- every global read, issued before the first wait (optional inputs are read
  // through a valid stand-in pointer and their value discarded)
  const float raw = p.dt[sl];
  const float ga_raw = (p.gamma ? p.gamma : p.dt)[sl];
  const float be_raw = (p.beta ? p.beta : p.dt)[sl];
  // this thread's columns of X_t and X_{t-1} (rows past R read row R-1, then zeroed)
  float xr[RMAX][4], xpr[PREV ? RMAX : 1][4];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    const int rr = r < R ? r : R - 1;
    load_cols4<BF16>(x + rr * P + c4, xr[r]);
    if constexpr (PREV) load_cols4<BF16>(xp + rr * P + c4, xpr[r]);
  }
  // B / C rows for the LDS tables, two elements per item (N is even), one item of
  // each table per thread here (clamped), the rest below
  const int rn2 = R * N / 2, on2 = O * N / 2;
  const int ib = tid < rn2 ? tid : 0, ic = tid < on2 ? tid : 0;
  const float2 eb = load_pair<BF16>(Bm + 2 * ib);
  const float2 ec = load_pair<BF16>(Cm + 2 * ic);
  const float2 ep = PREV ? load_pair<BF16>(Bp + 2 * ib) : make_float2(0.f, 0.f);
  // the rates of this thread's row pair of the transition table
  const int q = tid < npair ? tid : 0;
  const int nq = 2 * q;
  const bool qpair = nq >= nreal;
  const int jq = qpair ? (nq - nreal) >> 1 : 0;
  const int ia0 = p.head_rates ? h : h * na + (qpair ? nreal + jq : nq);
  const int ia1 = p.head_rates ? h : h * na + (qpair ? nreal + jq : nq + 1);
  const float ra0 = p.A[ia0], ra1 = p.A[ia1];
  const float om = (qpair ? p.omega + h * p.n_pairs + jq : p.A + ia0)[0];
  // the state of the first MP row pairs (rows past N read row pair 0)
  float4 s0[MP], s1[MP];
  auto load_batch = [&](int base) {
#pragma unroll
    for (int k = 0; k < MP; ++k) {
      const int n = 2 * (base + k * groups);
      const int nc = (n < N && active) ? n : 0;
      s0[k] = *reinterpret_cast<const float4*>(st + (size_t)nc * P + c4);
      s1[k] = *reinterpret_cast<const float4*>(st + (size_t)(nc + 1) * P + c4);
    }
  };
  load_batch(grp);

  // ---- LDS tables
  const float dl = p.softplus ? softplus_f32(raw) : raw;
  const float ga = p.gamma ? ga_raw : 1.f;
  const float be = p.beta ? be_raw : 0.f;
  if (live && tid < rn2) {
    sB[2 * tid] = ga * eb.x;
    sB[2 * tid + 1] = ga * eb.y;
    if constexpr (PREV) {
      sBp[2 * tid] = be * ep.x;
      sBp[2 * tid + 1] = be * ep.y;
    }
  }
  if (live && tid < on2) {
    sC[2 * tid] = ec.x;
    sC[2 * tid + 1] = ec.y;
  }
  for (int it = tid + NT; live && it < rn2; it += NT) {  // rare: R N / 2 > threads per slice
    const float2 e = load_pair<BF16>(Bm + 2 * it);
    sB[2 * it] = ga * e.x;
    sB[2 * it + 1] = ga * e.y;
    if constexpr (PREV) {
      const float2 f = load_pair<BF16>(Bp + 2 * it);
      sBp[2 * it] = be * f.x;
      sBp[2 * it + 1] = be * f.y;
    }
  }
  for (int it = tid + NT; live && it < on2; it += NT) {
    const float2 e = load_pair<BF16>(Cm + 2 * it);
    sC[2 * it] = e.x;
    sC[2 * it + 1] = e.y;
  }
  if (live && tid < npair) {
    // a static row pair (n_static is even) takes a unit step whatever Delta is
    const float dq = nq < p.n_static ? 1.f : dl;
    const float d0 = __expf(-ra0 * dq), d1 = __expf(-ra1 * dq);
    if (qpair) {
      float sn, cs;
      fast_sincos(om * dl, &sn, &cs);
      sTab[nq] = d0 * cs;
      sTab[nq + 1] = d0 * sn;
    } else {
      sTab[nq] = d0;
      sTab[nq + 1] = d1;
    }
  }
  for (int qq = tid + NT; live && qq < npair; qq += NT) {  // rare: N / 2 > threads per slice
    const int n = 2 * qq;
    if (n >= nreal) {
      const int j = (n - nreal) >> 1;
      const float d = __expf(-p.A[h * na + nreal + j] * dl);
      float sn, cs;
      fast_sincos(p.omega[h * p.n_pairs + j] * dl, &sn, &cs);
      sTab[n] = d * cs;
      sTab[n + 1] = d * sn;
    } else {
      const float dq = n < p.n_static ? 1.f : dl;
      sTab[n] = __expf(-p.A[p.head_rates ? h : h * na + n] * dq);
      sTab[n + 1] = __expf(-p.A[p.head_rates ? h : h * na + n + 1] * dq);
    }
  }
  lds_barrier();

  // ---- state update and readout partials
#pragma unroll
  for (int r = 0; r < RMAX; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xr[r][i] = r < R ? xr[r][i] : 0.f;
      if constexpr (PREV) xpr[r][i] = r < R ? xpr[r][i] : 0.f;
    }
  float yacc[RMAX][4];
#pragma unroll
  for (int o = 0; o < RMAX; ++o)
#pragma unroll
    for (int i = 0; i < 4; ++i) yacc[o][i] = 0.f;

  if (active) {
    for (int base = grp; base < npair; base += MP * groups) {
      if (base != grp) load_batch(base);
#pragma unroll
      for (int k = 0; k < MP; ++k) {
        const int n = 2 * (base + k * groups);
        if (n >= N) break;
        float v0[4] = {s0[k].x, s0[k].y, s0[k].z, s0[k].w};
        float v1[4] = {s1[k].x, s1[k].y, s1[k].z, s1[k].w};
        // transition: decay of each row, or the pair's decayed rotation
        const float t0 = sTab[n], t1 = sTab[n + 1];
        if (n >= nreal) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float u0 = v0[i], u1 = v1[i];
            v0[i] = t0 * u0 - t1 * u1;
            v1[i] = t1 * u0 + t0 * u1;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v0[i] *= t0;
            v1[i] *= t1;
          }
        }
        // writes: gamma B_t X_t + beta B_{t-1} X_{t-1} (rows past R: x is zero and the
        // table row is clamped to a written one)
#pragma unroll
        for (int r = 0; r < RMAX; ++r) {
          const int rr = r < R ? r : R - 1;
          const float b0 = sB[rr * N + n], b1 = sB[rr * N + n + 1];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v0[i] += b0 * xr[r][i];
            v1[i] += b1 * xr[r][i];
          }
          if constexpr (PREV) {
            const float q0 = sBp[rr * N + n], q1 = sBp[rr * N + n + 1];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              v0[i] += q0 * xpr[r][i];
              v1[i] += q1 * xpr[r][i];
            }
          }
        }
        *reinterpret_cast<float4*>(st + (size_t)n * P + c4) =
            make_float4(v0[0], v0[1], v0[2], v0[3]);
        *reinterpret_cast<float4*>(st + (size_t)(n + 1) * P + c4) =
            make_float4(v1[0], v1[1], v1[2], v1[3]);
        // readout partials (rows past O accumulate a copy of row O-1, never stored)
#pragma unroll
        for (int o = 0; o < RMAX; ++o) {
          const int oo = o < O ? o : O - 1;
          const float f0 = sC[oo * N + n], f1 = sC[oo * N + n + 1];
#pragma unroll
          for (int i = 0; i < 4; ++i) yacc[o][i] += f0 * v0[i] + f1 * v1[i];
        }
      }
    }
    // the feedthrough D_h X_t joins the partials of group 0 (D implies O == R)
    if (p.D && grp == 0) {
      const float Dh = p.D[h];
#pragma unroll
      for (int o = 0; o < RMAX; ++o)
#pragma unroll
        for (int i = 0; i < 4; ++i) yacc[o][i] += Dh * xr[o][i];
    }
#pragma unroll
    for (int o = 0; o < RMAX; ++o)
      if (o < O)
        *reinterpret_cast<float4*>(&sY[(o * groups + grp) * P + c4]) =
            make_float4(yacc[o][0], yacc[o][1], yacc[o][2], yacc[o][3]);
  }
  lds_barrier();
  // y[o][c..c+3] = sum of the partials over the groups in order
  T* y = static_cast<T*>(p.y) + (size_t)sl * O * P;
  for (int item = tid; item < (live ? O * cpr : 0); item += NT) {
    const int o = item / cpr, c = (item % cpr) * 4;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < groups; ++k) {
      const float4 f = *reinterpret_cast<const float4*>(&sY[(o * groups + k) * P + c]);
      v[0] += f.x; v[1] += f.y; v[2] += f.z; v[3] += f.w;
    }
    store_cols4<BF16>(y + o * P + c, v);
  }
}

hipError_t launch_decode(bool bf16, const DecodeParams& p, hipStream_t stream) {
  const long slices = (long)p.batch * p.H;
  if (slices == 0) return hipSuccess;
  const int spw = 256 / p.tps;
  const long wgs = (slices + spw - 1) / spw;
  const size_t lds = (size_t)spw * decode_lds_floats(p.n_real + 2 * p.n_pairs, p.R, p.O, p.P, p.tps) * 4;
  const int rank = p.R > p.O ? p.R : p.O;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)wgs), dim3(256), lds, stream, p);
  };
  const bool prev = p.x_prev != nullptr;
#define SSM_DECODE_GO(BF)                                                                   \
  if (prev) {                                                                               \
    if (rank <= 1) go(ssm_decode_kernel<BF, 1, true>);                                      \
    else if (rank <= 2) go(ssm_decode_kernel<BF, 2, true>);                                 \
    else if (rank <= 4) go(ssm_decode_kernel<BF, 4, true>);                                 \
    else go(ssm_decode_kernel<BF, kDecodeMaxRank, true>);                                   \
  } else {                                                                                  \
    if (rank <= 1) go(ssm_decode_kernel<BF, 1, false>);                                     \
    else if (rank <= 2) go(ssm_decode_kernel<BF, 2, false>);                                \
    else if (rank <= 4) go(ssm_decode_kernel<BF, 4, false>);                                \
    else go(ssm_decode_kernel<BF, kDecodeMaxRank, false>);                                  \
  }
  if (bf16) {
    SSM_DECODE_GO(true)
  } else {
    SSM_DECODE_GO(false)
  }
#undef SSM_DECODE_GO
  return hipGetLastError();
}

}  // namespace ssm
