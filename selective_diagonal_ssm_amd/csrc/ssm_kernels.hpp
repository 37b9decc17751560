// ssm_kernels.hpp -- launch parameters and host-side launch entry points of the
// HIP kernels (internal to libssmscan; the public boundary is include/ssm_scan.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

struct FwdParams {
  const void* x;
  const void* B;
  const void* C;
  const float* dt;
  const float* A;
  const float* omega;
  const float* beta;
  const float* gamma;
  const float* D;
  void* y;
  void* saved;   // [batch][nheads][save_nchunks + 1][N][P] in the io dtype, or null
  const float* h0;  // [batch][nheads][N][P] fp32 state before token 0, or null
  float* h_final;   // [batch][nheads][N][P] fp32 state after the last token, or null
  // the token before the sequence (two-endpoint carry), or null: x [batch][nheads][rin][P],
  // B [batch][ngroups][rin][N]
  const void* x_prev;
  const void* B_prev;
  int batch, L, H, G, P, n_real, n_pairs, nchunks, npblk;
  // the saved states are those of chunks of save_chunk tokens (the kernel's chunk, or half of
  // it), save_nchunks of them
  int save_chunk, save_nchunks;
  int n_static;  // the first n_static real rows decay by e^{-A} per token, whatever the step
  // ranks of the write (B, x) and of the readout (C, y); the kernel's rank R is the
  // larger, rows past a side's own rank are zero on load and dropped on store
  int rin, rout;
  int softplus, has_D;
  int head_rates;  // A holds one rate per head even though the per-row kernel runs
  // sequence segments (nseg = 1: one workgroup walks the whole sequence)
  int nseg, cps;     // segments per slice, chunks per segment
  // local pass: every segment but the last is cut into nsub ranges of lsub tokens
  // (the last range may be shorter); each range's final state from a zero start
  int seg_tokens, nsub, lsub;
  float* seg_local;  // [slice][nseg - 1][nsub][N][P] range final states (local pass output)
  float* seg_in;     // [slice][nseg][N][P] states entering the segments (combine output)
  float* seg_delta;  // [slice][nseg - 1][nsub] sum of Delta over each range (local pass output)
  // per-row kernel: one flag per workgroup (logical id), set when its range holds a chunk
  // too steep for the fold (workspace); null for the head-decay kernel
  int* wild;
};

// Largest chunk exponent the per-row kernels fold: a chunk whose summed step times the
// largest |rate| of the head's rows exceeds it is flagged and redone by the token-by-token
// kernels (ssm_exact.hpp).  The folded factors then stay below e^{kFoldLimit / 2} = e^60.
constexpr float kFoldLimit = 120.f;
// tokens the token-by-token forward stages per block
constexpr int kExactTokens = 16;

// tokens of one local-pass range (bounds the kernel's per-token LDS tables)
constexpr int kLocalMaxTokens = 512;
// ranges whose boundary states a combine thread reads in one batch
constexpr int kCombineBlock = 8;

// operands of a segment local pass: forward ranges (states from a zero start) or
// boundary-adjoint ranges (adjoints from a zero adjoint after the range)
struct LocalParams {
  const void* key;  // B (forward) or C (adjoint): [batch][L][G][R][N], io dtype
  const void* val;  // x (forward) or dy (adjoint): [batch][L][H][R][P], io dtype
  // forward: the token before the sequence (two-endpoint carry), or null
  const void* key_prev;  // [batch][G][R][N]
  const void* val_prev;  // [batch][H][R][P]
  const float* dt;
  const float* A;
  const float* omega;
  const float* beta;
  const float* gamma;
  float* out;    // [slice][nseg - 1][nsub][N][P] range states
  float* delta;  // [slice][nseg - 1][nsub] range summed steps
  int rk;        // rows per token of key and value (rank_in forward, rank_out adjoint)
  int batch, L, H, G, P, n_real, n_pairs, softplus, head_rates;
  int n_static;  // static real rows (decay e^{-A} per token)
  int nseg, seg_tokens, nsub, lsub;
};

struct BwdParams {
  const void* x;
  const void* B;
  const void* C;
  const void* dy;
  const float* dt;
  const float* A;
  const float* omega;
  const float* beta;
  const float* gamma;
  const float* D;
  const void* saved;  // forward's chunk-boundary states (io dtype)
  // two-endpoint carry (or null): the token before the sequence, its gradients, and the
  // upstream gradient of the final state
  const void* x_prev;
  const void* B_prev;
  const float* dh_final;  // [batch][nheads][N][P] fp32
  void* dx_prev;
  void* dB_prev;
  void* dx;
  void* dB;
  void* dC;
  float* ddt;
  float* dbeta;
  float* dgamma;
  float* part;     // per-(slice, segment) parameter-gradient partials (workspace)
  void* gseg;      // chunk-boundary adjoint states, [slice][nchunks + 1][N][P] io dtype
                   // (workspace); slot nchunks holds dh_final (zero without it)
  float* dA;
  float* domega;
  float* dD;
  float* dh0;  // [batch][nheads][N][P] fp32, or null
  // head groups shared by several heads: per-head dB / dC partials in the io dtype,
  // [batch][L][nheads][R][N] (workspace), summed over each group's heads afterwards;
  // null when every head has its own group
  void* dBh;
  void* dCh;
  int batch, L, H, G, P, n_real, n_pairs, nchunks;
  int n_static;  // static real rows (decay e^{-A} per token)
  // ranks of the write (B, x, dB, dx) and of the readout (C, dy, dC); the kernels' rank
  // R is the larger, rows past a side's own rank are zero on load and dropped on store
  int rin, rout;
  int nseg, chunks_per_seg;  // sequence segments of the boundary-adjoint sweep
  int softplus, has_D, npart;
  int head_rates;
  // upper bound on the persistent chunk-gradient grid (0 = one workgroup per resident
  // slot); a smaller grid makes each workgroup walk more items, with the same results
  int chunk_grid_cap;
  // local pass: every segment but the first is cut into nsub ranges of lsub tokens
  int seg_tokens, nsub, lsub;
  float* gloc;     // [slice][nseg - 1][nsub][N][P] range adjoints at the ranges' first tokens
  float* gin;      // [slice][nseg][N][P] adjoints flowing into the segments from the right
  float* gdel;     // [slice][nseg - 1][nsub] summed step of each range's transition
  // per-row kernel: one flag per (slice, chunk) item, set when the chunk is too steep for
  // the fold, and one word set when any item is (workspace; zeroed by the boundary-adjoint
  // sweep, which runs first); null for the head-decay kernel
  int* wild;
  int* wild_any;
};

// Single-token recurrent step (one token per slice, state updated in place).
constexpr int kDecodeMaxRank = 8;  // rank_in and rank_out limit of the step kernel
struct DecodeParams {
  const void* x;       // [batch][nheads][R][P]
  const void* B;       // [batch][ngroups][R][N]
  const void* C;       // [batch][ngroups][O][N]
  const float* dt;     // [batch][nheads]
  const float* A;
  const float* omega;
  const float* beta;
  const float* gamma;
  const float* D;
  const void* x_prev;  // previous token's x and B (two-endpoint writes), or null
  const void* B_prev;
  float* state;        // [batch][nheads][N][P] fp32, read and overwritten
  void* y;             // [batch][nheads][O][P]
  int batch, H, G, P, R, O, n_real, n_pairs;
  int n_static;  // static real rows (decay e^{-A} per token)
  int softplus, head_rates;
  int tps;  // threads per slice (64, 128 or 256); 256 / tps slices per workgroup
};
hipError_t launch_decode(bool bf16, const DecodeParams& p, hipStream_t stream);
// LDS of one slice of the step kernel (tps threads), in floats: the transition
// table, the staged gamma B_t, beta B_{t-1} and C_t rows, and the readout partials
// [O][groups][P].
__host__ __device__ inline int decode_lds_floats(int N, int R, int O, int P, int tps) {
  const int groups = tps / (P / 4);
  return N + (2 * R + O) * N + O * groups * P;
}
// Threads per slice: the fewest (down to one wave) that still give each thread
// kDecodePairs row pairs of 4 columns, so that small states share a workgroup.
constexpr int kDecodePairs = 4;
inline int decode_tps(int N, int P) {
  const long units = (long)(N / 2) * (P / 4);  // (row pair, 4 columns) units
  int tps = 256;
  while (tps > 64 && units < (long)tps * kDecodePairs && tps / 2 >= P / 4) tps /= 2;
  return tps;
}
constexpr long kDecodeMaxLdsBytes = 65536;

// Kernel variant key: io dtype, state size, P-block, rank, keys per token, tokens
// per chunk, decay mode.
struct FwdKey {
  bool bf16;
  int N, PB, R, KR, QT;
  bool coord;
  int nthreads;
};

// Returns hipSuccess, or hipErrorInvalidValue when no variant matches.
hipError_t launch_fwd(const FwdKey& key, const FwdParams& p, hipStream_t stream,
                      void* const* events);
bool fwd_variant_exists(const FwdKey& key);

struct BwdKey {
  bool bf16;
  int N, P, R, KR, QT;
  bool coord;
  bool split;  // rank_in != rank_out (the chunk kernel then takes both ranks at run time)
};
hipError_t launch_bwd(const BwdKey& key, const BwdParams& p, hipStream_t stream,
                      void* const* events);
bool bwd_variant_exists(const BwdKey& key);

}  // namespace ssm
