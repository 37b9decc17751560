// ssm_decode.hip -- single-token recurrent step of the state-mediated selective SSM
// kernel for gfx950 (the step-by-step inference mode of the same recurrence):
//
//   h <- A_t h + gamma_t B_t X_t + beta_t B_{t-1} X_{t-1},     y_t = C_t^T h + D_h X_t
//
// with A_t block diagonal (real rows exp(-Delta A_n), rotating pairs
// rho R(Delta omega)).  The step streams the N x P fp32 state of every (batch, head)
// slice once in and once out; everything else (x, B, C, the scalars) is a few
// hundred bytes per slice.  One workgroup per slice: each thread owns 4 adjacent
// value columns (16-byte state accesses, P/4 threads cover a row) of one row pair
// at a time (a rotating pair needs both of its rows), the row pairs are spread over
// the 256/(P/4) thread groups, and y is summed over the groups in a fixed order
// through LDS, so the result is bitwise reproducible.
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

}  // namespace

template <bool BF16>
__global__ __launch_bounds__(256) void ssm_decode_kernel(DecodeParams p) {
  using T = typename Elem<BF16>::T;
  constexpr int NT = 256;
  constexpr int RMAX = kDecodeMaxRank;
  __shared__ float sY[RMAX * NT * 4];  // [o][group][P] readout partials

  const int slice = blockIdx.x;
  const int b = slice / p.H, h = slice % p.H, g = h / (p.H / p.G);
  const int N = p.n_real + 2 * p.n_pairs, P = p.P, R = p.R, O = p.O, nreal = p.n_real;
  const int na = p.n_real + p.n_pairs;
  const int cpr = P / 4;         // threads per state row (host: 4 | P, P <= 1024)
  const int groups = NT / cpr;   // row-pair groups; threads beyond cpr * groups idle
  const int tid = threadIdx.x;
  const int c4 = (tid % cpr) * 4, grp = tid / cpr;
  const bool active = grp < groups;

  const T* x = static_cast<const T*>(p.x) + (size_t)slice * R * P;
  const T* Bm = static_cast<const T*>(p.B) + ((size_t)b * p.G + g) * R * N;
  const T* Cm = static_cast<const T*>(p.C) + ((size_t)b * p.G + g) * O * N;
  const bool prev = p.x_prev != nullptr;
  const T* xp = prev ? static_cast<const T*>(p.x_prev) + (size_t)slice * R * P : nullptr;
  const T* Bp = prev ? static_cast<const T*>(p.B_prev) + ((size_t)b * p.G + g) * R * N : nullptr;
  float* st = p.state + (size_t)slice * N * P;

  const float raw = p.dt[slice];
  const float dl = p.softplus ? softplus_f32(raw) : raw;
  const float ga = p.gamma ? p.gamma[slice] : 1.f;
  const float be = p.beta ? p.beta[slice] : 0.f;

  // this thread's columns of X_t (scaled by gamma) and X_{t-1} (scaled by beta)
  float xv[RMAX][4], xpv[RMAX][4], yacc[RMAX][4];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    float t[4] = {0.f, 0.f, 0.f, 0.f}, u[4] = {0.f, 0.f, 0.f, 0.f};
    if (r < R && active) {
      load_cols4<BF16>(x + r * P + c4, t);
      if (prev) load_cols4<BF16>(xp + r * P + c4, u);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xv[r][i] = ga * t[i];
      xpv[r][i] = be * u[i];
      yacc[r][i] = 0.f;
    }
  }

  if (active) {
    for (int n = 2 * grp; n < N; n += 2 * groups) {
      float4 s0 = *reinterpret_cast<const float4*>(st + (size_t)n * P + c4);
      float4 s1 = *reinterpret_cast<const float4*>(st + (size_t)(n + 1) * P + c4);
      float v0[4] = {s0.x, s0.y, s0.z, s0.w}, v1[4] = {s1.x, s1.y, s1.z, s1.w};
      // transition: decay of each row, then the pair's rotation
      float d0, d1;
      if (p.head_rates) {
        d0 = d1 = __expf(-p.A[h] * dl);
      } else if (n < nreal) {
        d0 = __expf(-p.A[(size_t)h * na + n] * dl);
        d1 = __expf(-p.A[(size_t)h * na + n + 1] * dl);
      } else {
        d0 = d1 = __expf(-p.A[(size_t)h * na + nreal + ((n - nreal) >> 1)] * dl);
      }
      if (n >= nreal) {
        float sn, cs;
        fast_sincos(p.omega[(size_t)h * p.n_pairs + ((n - nreal) >> 1)] * dl, &sn, &cs);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float u0 = d0 * v0[i], u1 = d0 * v1[i];
          v0[i] = cs * u0 - sn * u1;
          v1[i] = sn * u0 + cs * u1;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v0[i] *= d0;
          v1[i] *= d1;
        }
      }
      // writes: gamma B_t X_t (+ beta B_{t-1} X_{t-1})
#pragma unroll
      for (int r = 0; r < RMAX; ++r) {
        if (r < R) {
          const float b0 = to_f32(Bm[r * N + n]), b1 = to_f32(Bm[r * N + n + 1]);
          float q0 = 0.f, q1 = 0.f;
          if (prev) {
            q0 = to_f32(Bp[r * N + n]);
            q1 = to_f32(Bp[r * N + n + 1]);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v0[i] += b0 * xv[r][i] + q0 * xpv[r][i];
            v1[i] += b1 * xv[r][i] + q1 * xpv[r][i];
          }
        }
      }
      *reinterpret_cast<float4*>(st + (size_t)n * P + c4) = make_float4(v0[0], v0[1], v0[2], v0[3]);
      *reinterpret_cast<float4*>(st + (size_t)(n + 1) * P + c4) =
          make_float4(v1[0], v1[1], v1[2], v1[3]);
      // readout partials
#pragma unroll
      for (int o = 0; o < RMAX; ++o) {
        if (o < O) {
          const float e0 = to_f32(Cm[o * N + n]), e1 = to_f32(Cm[o * N + n + 1]);
#pragma unroll
          for (int i = 0; i < 4; ++i) yacc[o][i] += e0 * v0[i] + e1 * v1[i];
        }
      }
    }
#pragma unroll
    for (int o = 0; o < RMAX; ++o)
      if (o < O)
        *reinterpret_cast<float4*>(&sY[(o * groups + grp) * P + c4]) =
            make_float4(yacc[o][0], yacc[o][1], yacc[o][2], yacc[o][3]);
  }
  __syncthreads();
  // y[o][c4..c4+3] = sum over the groups in order, plus the feedthrough
  T* y = static_cast<T*>(p.y) + (size_t)slice * O * P;
  const float Dh = p.D ? p.D[h] : 0.f;
  for (int item = tid; item < O * cpr; item += NT) {
    const int o = item / cpr, c = (item % cpr) * 4;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < groups; ++k) {
      const float4 q = *reinterpret_cast<const float4*>(&sY[(o * groups + k) * P + c]);
      v[0] += q.x; v[1] += q.y; v[2] += q.z; v[3] += q.w;
    }
    if (p.D) {
      float t[4];
      load_cols4<BF16>(x + o * P + c, t);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] += Dh * t[i];
    }
    store_cols4<BF16>(y + o * P + c, v);
  }
}

hipError_t launch_decode(bool bf16, const DecodeParams& p, hipStream_t stream) {
  const long slices = (long)p.batch * p.H;
  if (slices == 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(ssm_decode_kernel<true>, dim3((unsigned)slices), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(ssm_decode_kernel<false>, dim3((unsigned)slices), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace ssm
