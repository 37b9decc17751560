// ssm_device.hpp -- gfx950 device helpers shared by the forward and reverse kernels:
// element storage (bf16 bits or fp32), 16x16 MFMA tiles, wave-wide prefix sums.
//
// MFMA tile conventions (v_mfma_f32_16x16x32_bf16 and its fp32 counterpart):
//   A fragment (16 x 32): lane l holds A[l & 15][8 * (l >> 4) + i], i = 0..7
//   B fragment (32 x 16): lane l holds B[8 * (l >> 4) + i][l & 15], i = 0..7
//   D tile     (16 x 16): lane l holds D[4 * (l >> 4) + i][l & 15], i = 0..3
// An operand stored row-major with the contraction index contiguous therefore
// loads as one 16-byte LDS read per lane (bf16).  The fp32 path keeps the same
// fragment layout (8 floats per lane) and issues eight 16x16x4 fp32 MFMAs, so the
// two element types share every kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- element storage
template <bool BF16> struct Elem;
template <> struct Elem<true> {
  using T = uint16_t;
  static constexpr int kVec = 8;  // elements per 16-byte vector
};
template <> struct Elem<false> {
  using T = float;
  static constexpr int kVec = 4;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// round to nearest even (gfx950 v_cvt_pk_bf16_f32); NaN stays NaN
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// two floats -> packed bf16 pair (low half = a)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float to_f32(uint16_t v) { return bf16_to_f32(v); }
__device__ __forceinline__ float to_f32(float v) { return v; }

template <typename T> __device__ __forceinline__ T from_f32(float f);
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float f) { return f32_to_bf16(f); }
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }

template <bool BF16>
__device__ __forceinline__ void unpack(const uint4& r, float* v) {
  if constexpr (BF16) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    v[0] = __uint_as_float(r.x);
    v[1] = __uint_as_float(r.y);
    v[2] = __uint_as_float(r.z);
    v[3] = __uint_as_float(r.w);
  }
}

template <bool BF16>
__device__ __forceinline__ uint4 pack(const float* v) {
  uint4 r;
  if constexpr (BF16) {
    r.x = pack_bf16x2(v[0], v[1]);
    r.y = pack_bf16x2(v[2], v[3]);
    r.z = pack_bf16x2(v[4], v[5]);
    r.w = pack_bf16x2(v[6], v[7]);
  } else {
    r.x = __float_as_uint(v[0]);
    r.y = __float_as_uint(v[1]);
    r.z = __float_as_uint(v[2]);
    r.w = __float_as_uint(v[3]);
  }
  return r;
}

// the raw stored elements of a 16-byte vector
template <bool BF16>
__device__ __forceinline__ void unpack_raw(const uint4& r, typename Elem<BF16>::T* e) {
  if constexpr (BF16) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e[2 * i] = static_cast<uint16_t>(w[i] & 0xffffu);
      e[2 * i + 1] = static_cast<uint16_t>(w[i] >> 16);
    }
  } else {
    e[0] = __uint_as_float(r.x);
    e[1] = __uint_as_float(r.y);
    e[2] = __uint_as_float(r.z);
    e[3] = __uint_as_float(r.w);
  }
}

// ---------------------------------------------------------------- MFMA fragments
template <bool BF16> struct Frag;
template <> struct Frag<true> { bf16x8 v; };
template <> struct Frag<false> { float v[8]; };

// 8 consecutive elements starting at p (16-byte aligned for bf16, 32 for fp32)
template <bool BF16>
__device__ __forceinline__ Frag<BF16> load_frag(const typename Elem<BF16>::T* p) {
  Frag<BF16> f;
  if constexpr (BF16) {
    f.v = *reinterpret_cast<const bf16x8*>(p);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
  }
  return f;
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Fragment whose contraction index runs along the ROWS of a row-major buffer:
// lane l receives buf[8 * (l >> 4) + i][l & 15] (i = 0..7) of the 32 x 16 block at
// `base` (row stride `ld` elements).  Serves as a B operand stored [k][n] or an A
// operand stored transposed [k][m].  bf16 uses the gfx950 LDS transpose read
// (ds_read_b64_tr_b16): inside each 16-lane group, lanes 4r..4r+3 supply the four
// 4-element pieces of row r of a 4 x 16 block and lane i receives its column i.
template <bool BF16>
__device__ __forceinline__ Frag<BF16> load_frag_tr(const typename Elem<BF16>::T* base, int ld) {
  const int l = threadIdx.x & 63;
  Frag<BF16> f;
  if constexpr (BF16) {
    const int row = 8 * (l >> 4) + ((l >> 2) & 3);
    const int col = 4 * (l & 3);
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(base + row * ld + col));
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(base + (row + 4) * ld + col));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 c = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    f.v = __builtin_bit_cast(bf16x8, c);
  } else {
    const int col = l & 15, row0 = 8 * (l >> 4);
#pragma unroll
    for (int i = 0; i < 8; ++i) f.v[i] = base[(row0 + i) * ld + col];
  }
  return f;
}

// four consecutive elements <-> floats (8 bytes bf16, 16 bytes fp32; aligned to that)
template <bool BF16>
__device__ __forceinline__ void store4(typename Elem<BF16>::T* dst, const float* v) {
  if constexpr (BF16) {
    uint2 w;
    w.x = pack_bf16x2(v[0], v[1]);
    w.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(dst) = w;
  } else {
    *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

template <bool BF16>
__device__ __forceinline__ void load4(const typename Elem<BF16>::T* src, float* v) {
  if constexpr (BF16) {
    const uint2 w = *reinterpret_cast<const uint2*>(src);
    v[0] = __uint_as_float(w.x << 16);
    v[1] = __uint_as_float(w.x & 0xffff0000u);
    v[2] = __uint_as_float(w.y << 16);
    v[3] = __uint_as_float(w.y & 0xffff0000u);
  } else {
    const float4 w = *reinterpret_cast<const float4*>(src);
    v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
  }
}

// acc += A(16x32) * B(32x16)
template <bool BF16>
__device__ __forceinline__ void mma(f32x4& acc, const Frag<BF16>& a, const Frag<BF16>& b) {
  if constexpr (BF16) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
  } else {
    // lane l supplies k = 8*(l>>4) + i to instruction i, seen by the 16x16x4
    // instruction as its k = l >> 4; the eight instructions cover all 32 k.
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], acc, 0, 0, 0);
  }
}

// ---------------------------------------------------------------- wave primitives
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// inclusive prefix sum across the 64 lanes of a wave: a Hillis-Steele scan inside
// each 16-lane row by DPP row shifts (lanes shifted in from outside the row add 0),
// then the totals of the earlier rows (lanes 15, 31, 47) are added in
__device__ __forceinline__ float wave_prefix_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xF, 0xF, false));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 47));
  const int row = lane_id() >> 4;
  const float carry = row == 0 ? 0.f : row == 1 ? r0 : row == 2 ? r0 + r1 : (r0 + r1) + r2;
  return v + carry;
}

// value of the neighbouring lane (l ^ 1), by a DPP quad permutation [1, 0, 3, 2]
__device__ __forceinline__ float swap_adjacent_lanes(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}


template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of K consecutive lanes (K = 1, 2, 4, 8, 16), by DPP lane
// permutations inside 16-lane rows: every lane of a group receives the group's
// sum, added in the same order on every call.
template <int K>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(K == 1 || K == 2 || K == 4 || K == 8 || K == 16, "group of 1..16 lanes");
  if constexpr (K >= 2) v += dpp_f32<0xB1>(v);   // quad permutation [1, 0, 3, 2]
  if constexpr (K >= 4) v += dpp_f32<0x4E>(v);   // quad permutation [2, 3, 0, 1]
  if constexpr (K >= 8) v += dpp_f32<0x141>(v);  // mirror inside each half row
  if constexpr (K >= 16) v += dpp_f32<0x140>(v); // mirror inside the row
  return v;
}

// value of v in lane `src` (src must be the same for the whole wave)
__device__ __forceinline__ float read_lane(float v, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

// v + (v of lane l ^ 16) and v + (v of lane l ^ 32), by the gfx950 VALU row swaps
// v_permlane16_swap / v_permlane32_swap applied to two copies of v (both lanes of a
// pair add their two values in the same order)
__device__ __forceinline__ float add_xor16(float v) {
  const unsigned u = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float v) {
  const unsigned u = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// sum over the 64 lanes of a wave (every lane receives the same value): DPP sums
// inside the four 16-lane rows, then the row totals read from lanes 0, 16, 32, 48
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<16>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// largest value over the 64 lanes of a wave (every lane receives it)
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// softplus(v) = log(1 + e^v) with hardware exp/log: log1p(u) is evaluated as
// log(w) * u / (w - 1), w = 1 + u, which keeps full relative accuracy for tiny u.
__device__ __forceinline__ float softplus_f32(float v) {
  if (v > 20.f) return v;
  const float u = __builtin_amdgcn_exp2f(v * 1.4426950408889634f);
  const float w = 1.f + u;
  // w >= 1 is a normal number, so the raw hardware log2 is exact to its ulp bound
  return (w == 1.f) ? u
                    : __builtin_amdgcn_logf(w) * 0.6931471805599453f * u *
                          __builtin_amdgcn_rcpf(w - 1.f);
}

// sin and cos of an angle in radians: reduce to revolutions in [-1/2, 1/2], then
// the hardware sin / cos (which take revolutions)
__device__ __forceinline__ void fast_sincos(float x, float* sn, float* cs) {
  float r = x * 0.15915494309189535f;  // 1 / (2 pi)
  r -= rintf(r);
  *sn = __builtin_amdgcn_sinf(r);
  *cs = __builtin_amdgcn_cosf(r);
}

__device__ __forceinline__ float sigmoid_f32(float v) { return 1.f / (1.f + expf(-v)); }

// Workgroup -> work item mapping that keeps consecutive logical ids on one XCD
// (the dispatcher places workgroup i on XCD i % 8), so the P-blocks of one slice
// share that XCD's L2 for their common B and C reads.
__device__ __forceinline__ int xcd_logical_id(int wg, int nwg) {
  if (nwg % 8) return wg;
  return (wg % 8) * (nwg / 8) + wg / 8;
}

}  // namespace ssm
