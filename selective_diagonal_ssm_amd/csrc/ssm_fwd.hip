// ssm_fwd.hip -- forward chunked scan of the state-mediated selective SSM kernel
// for gfx950 (MI355X).
//
// One workgroup owns one (batch, head) slice and one block of PB value columns,
// and walks the sequence chunk by chunk with the N x PB state held in MFMA
// accumulator registers (fp32).  Score, output and state tiles are computed
// transposed (operands swapped), so that each lane holds four consecutive keys or
// value columns: one decay factor per lane, 8-byte LDS and global writes.  One
// wave forms the next chunk's per-token factors while the others compute scores.
// Per chunk of QT tokens:
//
//  a1  chunk-local cumulative step CD_t = sum_{r<=t} Delta_r by a wave prefix sum
//      (Delta = softplus(dt) when flagged); the log-decay of row n is
//      L_t[n] = -A_n CD_t and the pair angle Theta_t[k] = omega_k CD_t.
//  a2  write prologue: rotation folding C~_t = R(-Theta_t) C_t, K~_s = R(-Theta_s) K_s
//      (exact because a pair's rotation commutes with its scalar decay), and the
//      two-endpoint write as rank-2R keys per token: K_s = [gamma_s B_s | beta_s B_{s-1}]
//      with values [X_s ; X_{s-1}] (one halo token per chunk).
//  a3  intra-chunk masked product Y = (Q K^T o M) V on bf16 MFMA (fp32 accumulate).
//      Head decay: M_ts = exp(L_t - L_s) [s <= t] applied per element in fp32.
//      Per-row decay: the decay is folded into the operands around the chunk
//      midpoint, q_t = C~_t e^{L_t - L_end/2}, k_s = K~_s e^{L_end/2 - L_s}, so that no
//      factor exceeds e^{|L_end|/2}; the mask is then the causal indicator.
//  a4/a5  chunk state and state passing: S <- Lambda o S + (K~ o e^{L_end - L_s})^T V,
//      then the chunk-total rotation of the pairs; S never leaves the registers
//      (a bf16 copy in LDS feeds the next chunk's readout).
//  a6  readout C~_t e^{L_t} S_in + Y + D X_t, stored as the io dtype.
//
// Sources: "When a Diagonal State Is Not Enough" (sungsoo.github.io), Part 01 and
// Part 03 (recurrence; Theorem 24 masked linear attention form; Theorem 8 rotating
// pairs), Parts 03 / 08.3 (SSD-MIMO rank-R writes, HybridMamba rows and
// two-endpoint writes).
#include <algorithm>

#include "ssm_device.hpp"
#include "ssm_exact.hpp"
#include "ssm_kernels.hpp"
#include "ssm_local.hpp"

namespace ssm {

template <bool BF16, int N, int PB, int R, int KR, int QT, bool COORD, int NTHREADS>
struct FwdShape {
  using T = typename Elem<BF16>::T;
  static constexpr int VEC = Elem<BF16>::kVec;
  static constexpr int PAD = 16 / static_cast<int>(sizeof(T));
  static constexpr int NC = N < 32 ? 32 : N;  // contraction width over n (zero padded)
  static constexpr int QO = QT * R;
  static constexpr bool TE = KR > R;
  static constexpr int TEH = TE ? 1 : 0;
  // Two-endpoint writes through the shift identity h'_t = h_t - gamma_t B_t X_t:
  //   h'_t = A_t h'_{t-1} + B^_{t-1} X_{t-1},  B^_{t-1} = (gamma_{t-1} A_t + beta_t) B_{t-1},
  //   y_t  = C_t^T h'_t + gamma_t (C_t . B_t) X_t + D X_t,
  // one key row per (token, rank) instead of two, plus a same-token term.  Used for
  // 32-token chunks (the two-chunk walk of the 16-token plan), where it keeps the keys
  // within the tiles of a 16-token chunk; at 16 tokens the two-endpoint keys
  // [gamma_s B_s | beta_s B_{s-1}] with values [X_s ; X_{s-1}] measured faster.
  static constexpr bool SHIFT = TE && QT >= 32 && (QT * R) % 32 == 0;
  static constexpr int KEYS = SHIFT ? R : KR;  // key rows per token
  // Per-row decay in shifted form can also save the state after the first QT / 2 tokens of
  // each chunk (the boundary states of half-size chunks, which the chunk gradients consume):
  // those tokens' keys are the first (QT / 2) KEYS key rows, a whole number of 32-row MFMA
  // steps of the state update.
  static constexpr bool CAN_HALF = SHIFT && COORD && QT % 2 == 0 && ((QT / 2) * KEYS) % 32 == 0;
  static constexpr int KK_HALF = CAN_HALF ? (QT / 2) * KEYS / 32 : 0;
  static constexpr int QK = QT * KEYS;
  static constexpr int NS = NC + PAD;  // row stride of n-contiguous buffers
  static constexpr int KS = QK + PAD;  // row stride of key-contiguous buffers (scores)
  static constexpr int VS = PB + PAD;  // row stride of p-contiguous buffers (values, state)
  static constexpr int BROWS = (QT + TEH) * R;
  static constexpr int NTH = NTHREADS;
  static constexpr int NW = NTHREADS / 64;  // waves per workgroup
  static constexpr int NVEC_N = N / VEC;
  static constexpr int NVEC_P = PB / VEC;
  static constexpr int C_VECS = QO * NVEC_N;
  static constexpr int B_VECS = BROWS * NVEC_N;
  static constexpr int X_VECS = BROWS * NVEC_P;
  // staging items: C vectors, then key items (a B vector and the endpoint it is
  // written at: two per vector with two-endpoint writes), then X vectors
  static constexpr int K_ITEMS = B_VECS;  // with two-endpoint writes one B vector gives two key rows
  // Each kind starts on a wave boundary (a wave holding two kinds runs both code
  // paths).  With per-row decay the key items, the costliest to stage, come first:
  // they land on the first waves, which take no output tiles (those go from the last
  // wave down).  Head decay keeps C, K, X.
  static constexpr int CP = (C_VECS + 63) / 64 * 64, KP = (K_ITEMS + 63) / 64 * 64;
  static constexpr int K0 = COORD ? 0 : CP;
  static constexpr int C0 = COORD ? KP : 0;
  static constexpr int X0 = CP + KP;
  static constexpr int ALL_VECS = X0 + X_VECS;
  static constexpr int ALL_PER = (ALL_VECS + NTH - 1) / NTH;
  static constexpr int TQ = QO / 16, TK = QK / 16, TP = PB / 16, TN = N / 16;
  static constexpr int ST_TILES = TN * TP;
  // output tiles per wave: a YBQ x YBP block (query tiles x value-column tiles),
  // 2 x 2 only when there are at least four tiles per wave anyway (a block then
  // halves the fragment reads at the same MFMA count per wave)
  static constexpr bool YBLK = TQ % 2 == 0 && TP % 2 == 0 && TQ * TP >= 4 * NW;
  static constexpr int YBQ = YBLK ? 2 : 1;
  static constexpr int YBP = YBLK ? 2 : 1;
  static constexpr int ST_PER_WAVE = (ST_TILES + NW - 1) / NW;
  // score tiles (16 query rows ti x 16 keys tj) that hold at least one causal
  // entry: key token floor(16 tj / KEYS) <= query token floor((16 ti + 15) / R)
  static constexpr int row_tiles(int ti) {
    const int c = (((16 * ti + 15) / R) * KEYS) / 16 + 1;
    return c < TK ? c : TK;
  }
  static constexpr int score_tiles() {
    int n = 0;
    for (int ti = 0; ti < TQ; ++ti) n += row_tiles(ti);
    return n;
  }
  static constexpr int SC_TILES = score_tiles();
  static_assert(QO % 16 == 0 && QK % 32 == 0, "chunk rows must fill MFMA tiles");
  static_assert(N % 16 == 0 && PB % 16 == 0 && QT <= 64, "unsupported tile shape");
  static_assert(KR == R || KR == 2 * R, "keys per token are R or 2R");
  static_assert(16 % KEYS == 0 && 16 % R == 0, "a tile spans whole tokens");
  static_assert(N <= NTHREADS, "one thread per state row in the prologue");
};

template <bool BF16, int N, int PB, int R, int KR, int QT, bool COORD, int NTHREADS>
__global__ __launch_bounds__(NTHREADS) void ssm_fwd_kernel(FwdParams p) {
  using S = FwdShape<BF16, N, PB, R, KR, QT, COORD, NTHREADS>;
  using T = typename S::T;
  constexpr int NW = S::NW;
  constexpr int NS = S::NS, KS = S::KS, VS = S::VS, VEC = S::VEC;
  constexpr int QSZ = S::QO * NS, KSZ = S::QK * NS, VSZ = S::QK * S::VS;
  constexpr float kLog2e = 1.4426950408889634f;
  // the wave that computes the per-token factors: with per-row decay wave 0, which has the
  // most slack before the first barrier (measured), else the last wave
  constexpr int PW = COORD ? 0 : NW - 1;

  // double-buffered chunk operands: chunk c is consumed while chunk c+1 is staged
  __shared__ __align__(16) T sQ[2 * QSZ];                     // queries (folded; per-row: scaled)
  __shared__ __align__(16) T sK[2 * KSZ];                     // keys (per-row: scaled)
  __shared__ __align__(16) T sV[2 * VSZ];                     // values, natural [key row][p]
  __shared__ __align__(16) T sVw[COORD ? 8 : 2 * VSZ];        // head: values scaled to the chunk end
  __shared__ __align__(16) T sS[S::QO * KS];                  // masked scores [query row][key]
  // state entering chunk c (buffer (c - c0) & 1, [n][p]), the readout operand; with
  // per-row decay row n is stored scaled by e^{-A_n CD_end / 2} of that chunk
  __shared__ __align__(16) T sST[2 * S::NC * VS];
  // per-token factors of chunk c in slot c & 3 (written by wave PW two chunks ahead)
  constexpr int TC = COORD ? 64 : 1, TH = COORD ? 1 : 64;
  __shared__ __align__(16) float sCD[4][TC];   // per-row decay: cumulative step inside the chunk
  __shared__ __align__(16) float sLC[4][TH];   // head: -A CD log2(e), so e^{L_t - L_s} = 2^{LC_t - LC_s}
  __shared__ __align__(16) float sDT[2][64];   // steps Delta of chunk c in slot c & 1
  // beta / gamma of chunk c in slot c & 3 (a chunk's readout still reads its own after the
  // next-but-one chunk's are staged)
  __shared__ __align__(16) float sGa[4][S::TE ? 64 : 1], sBe[4][S::TE ? 64 : 1];
  __shared__ float sMisc[4][3];                // CD_end, head: e^{-A CD_end}, tokens in the chunk
  // per-row decay: the exponent of row n over a stretch of tokens is
  // sRate[n] (summed step) + sRateS[n] (token count): a dynamic row has its rate in
  // sRate, a static row (decay e^{-A} per token, whatever the step) in sRateS
  __shared__ float sRate[COORD ? N : 1], sRateS[COORD ? N : 1], sOmega[COORD ? N / 2 + 1 : 1];
  // per-row decay: factor tables of the next chunk to stage, [token][n] (see tables)
  __shared__ __align__(16) float sTC[COORD ? QT * N : 4], sTK0[COORD ? QT * N : 4];
  __shared__ __align__(16) float sTK1[COORD && S::TE && !S::SHIFT ? QT * N : 4];
  // shift identity: raw C and B rows of the chunk (for the same-token products
  // C_t . B_t), the last token's X rows (by operand buffer), those products, and gamma
  // of the token before the chunk
  constexpr bool SH = S::SHIFT;
  __shared__ __align__(16) T sCraw[SH ? S::QO * NS : 8], sBraw[SH ? QT * R * NS : 8];
  __shared__ __align__(16) T sXl[SH ? 2 * R * VS : 8];
  __shared__ __align__(16) float sDG[SH ? S::QO * R : 4];
  __shared__ __align__(16) T sYo[S::QO * VS];                 // output rows of the previous chunk

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const int slice = lid / (p.npblk * p.nseg), seg = (lid / p.npblk) % p.nseg, pblk = lid % p.npblk;
  const int c0 = seg * p.cps, c1 = min(p.nchunks, c0 + p.cps);  // this workgroup's chunks
  const int b = slice / p.H, h = slice % p.H;
  const int g = h / (p.H / p.G);
  const int p0 = pblk * PB;
  const int L = p.L, H = p.H, G = p.G, P = p.P;
  const int nreal = p.n_real;

  // per-row rates (thread n < N) and pair frequencies (thread k < n_pairs): read first,
  // written to LDS once the prologue's other reads are in flight
  float r_rate = 0.f, r_rs = 0.f, r_om = 0.f;
  if (COORD) {
    const int na = p.n_real + p.n_pairs;
    if (tid < N)
      r_rate = p.head_rates ? p.A[h]  // one rate per head
                            : p.A[(size_t)h * na + (tid < nreal ? tid : nreal + ((tid - nreal) >> 1))];
    if (tid < p.n_static) {  // a static row's rate goes with the token count
      r_rs = r_rate;
      r_rate = 0.f;
    }
    if (tid < p.n_pairs) r_om = p.omega[(size_t)h * p.n_pairs + tid];
  }
  // the state entering the first chunk: h0 (rows < N, this P-block), the combined
  // state entering a later segment, or zero
  const float* h0s = seg == 0 ? (p.h0 ? p.h0 + (size_t)slice * N * P + p0 : nullptr)
                              : p.seg_in + ((size_t)slice * p.nseg + seg) * N * P + p0;
  const float Ah = COORD ? 0.f : p.A[h];
  const float Dh = p.has_D ? p.D[h] : 0.f;

  // slice bases (64-bit once); offsets inside a slice fit in 32 bits (the host
  // rejects tensors of 2^31 or more elements)
  const int rin = p.rin, rout = p.rout;
  const T* xg = static_cast<const T*>(p.x) + ((size_t)b * L * H + h) * rin * P + p0;
  const T* Bg = static_cast<const T*>(p.B) + ((size_t)b * L * G + g) * rin * N;
  const T* Cg = static_cast<const T*>(p.C) + ((size_t)b * L * G + g) * rout * N;
  T* yg = static_cast<T*>(p.y) + ((size_t)b * L * H + h) * rout * P + p0;
  const float* dtg = p.dt + (size_t)b * L * H + h;
  const float* beg = S::TE ? p.beta + (size_t)b * L * H + h : nullptr;
  const float* gag = S::TE ? p.gamma + (size_t)b * L * H + h : nullptr;
  // per-token strides of B, C, x, y
  const int tsB = G * rin * N, tsC = G * rout * N, tsX = H * rin * P, tsY = H * rout * P;
  // the carried token before the sequence (two-endpoint writes), or null
  const T* Bprev = p.B_prev ? static_cast<const T*>(p.B_prev) + ((size_t)b * G + g) * rin * N : nullptr;
  const T* xprev = p.x_prev ? static_cast<const T*>(p.x_prev) + ((size_t)b * H + h) * rin * P + p0 : nullptr;

  // shift identity: the state carried inside the kernel is h' = h - gamma B X of the
  // last token; a later segment's incoming state (h) loses gamma_{t0-1} B_{t0-1} X_{t0-1}
  const int tfirst = c0 * QT;
  const float gprev0 = (SH && tfirst > 0) ? gag[(size_t)(tfirst - 1) * H] : 0.f;
  auto shift_corr = [&](int n, int col) {
    float v = 0.f;
    if (SH && tfirst > 0) {
      for (int r = 0; r < rin; ++r)
        v += to_f32(Bg[(size_t)(tfirst - 1) * tsB + r * N + n]) * to_f32(xg[(size_t)(tfirst - 1) * tsX + r * P + col]);
      v *= gprev0;
    }
    return v;
  };

  // state tiles, transposed: st[k][i] = S[n = 16 tn + (lane & 15)][p = 16 tp + 4 (lane >> 4) + i]
  f32x4 st[S::ST_PER_WAVE];
  // The operand vectors of a chunk form one item list -- C rows, B rows (key items)
  // and X rows, 16 bytes each, in the order of FwdShape -- dealt round-robin over all
  // threads, so that every wave takes a share of the staging.
  uint4 rr[S::ALL_PER];
  float rdt = 0.f, rbe = 0.f, rga = 0.f;
  const uint4 zero4 = make_uint4(0, 0, 0, 0);

  auto load_chunk = [&](int c) {
    const int t0 = c * QT;
#pragma unroll
    for (int k = 0; k < S::ALL_PER; ++k) {
      const int u = tid + S::NTH * k;
      uint4 val = zero4;
      if (u >= S::C0 && u < S::C0 + S::C_VECS) {
        const int row = (u - S::C0) / S::NVEC_N, nv = (u - S::C0) % S::NVEC_N;
        const int t = t0 + row / R, o = row % R;
        if (t < L && o < rout) val = *reinterpret_cast<const uint4*>(Cg + t * tsC + o * N + nv * VEC);
      } else if (u >= S::K0 && u < S::K0 + S::K_ITEMS) {
        const int v = u - S::K0;
        const int row = v / S::NVEC_N, nv = v % S::NVEC_N;
        const int t = t0 + row / R - S::TEH, r = row % R;
        if (t >= 0 && t < L && r < rin) val = *reinterpret_cast<const uint4*>(Bg + t * tsB + r * N + nv * VEC);
        else if (t == -1 && r < rin && Bprev)  // the carried token before the sequence
          val = *reinterpret_cast<const uint4*>(Bprev + r * N + nv * VEC);
      } else if (u >= S::X0 && u < S::ALL_VECS) {
        const int v = u - S::X0;
        const int row = v / S::NVEC_P, pv = v % S::NVEC_P;
        const int t = t0 + row / R - S::TEH, r = row % R;
        if (t >= 0 && t < L && r < rin) val = *reinterpret_cast<const uint4*>(xg + t * tsX + r * P + pv * VEC);
        else if (t == -1 && r < rin && xprev)
          val = *reinterpret_cast<const uint4*>(xprev + r * P + pv * VEC);
      }
      rr[k] = val;
    }
    if (wave == PW) {
      // per-token scalars ahead of the operands (Delta of chunk c+2, beta / gamma of
      // chunk c+1): the staging of chunk c writes them to LDS, so the factor wave
      // never waits on global memory
      const int t2 = t0 + 2 * QT + lane, t1 = t0 + QT + lane;
      rdt = (lane < QT && t2 < L) ? dtg[t2 * H] : 0.f;
      if (S::TE) {
        const bool ok = lane < QT && t1 < L;
        rbe = ok ? beg[t1 * H] : 0.f;
        rga = ok ? gag[t1 * H] : 0.f;
      }
    }
  };

  // ---- a1: per-token factors of chunk c into slot c & 3 (wave PW only; lane = token,
  // dl = its step, 0 past the sequence end)
  // per-row decay: the largest |rate| of the head's rows (factor wave, from the rates its
  // lanes read) and whether a chunk of this range is too steep for the midpoint fold
  // (summed step times that rate above kFoldLimit)
  float amax = 0.f, smax = 0.f;  // dynamic rows' and static rows' largest |rate|
  bool steep = false;
  auto factors = [&](int c, float dl) {
    const int bi = c & 3;
    const float cd = wave_prefix_sum(dl);
    const float cdend = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cd), QT - 1));
    const int nv = min(QT, L - c * QT);  // tokens of the chunk inside the sequence
    if (COORD) steep = steep || amax * cdend + smax * nv > kFoldLimit;
    if (lane < QT) {
      if (COORD) sCD[bi][lane] = cd;
      if (!COORD) {
        sLC[bi][lane] = -Ah * kLog2e * cd;
      }
    }
    if (lane == 0) {
      sMisc[bi][0] = cdend;
      sMisc[bi][1] = COORD ? 0.f : __builtin_amdgcn_exp2f(-Ah * kLog2e * cdend);
      sMisc[bi][2] = static_cast<float>(nv);
    }
  };

  // Per-row decay: factor tables of chunk c (all threads, one entry pair per thread),
  // with E_t[n] = e^{-A_n (CD_t - CD_end/2)} and Theta_t[k] = omega_k CD_t:
  //   TC[t]  = E_t on real rows; (E_t cos, E_t sin)(Theta_t) on the rows of pair k,
  //   TK0[t] = g_t / E_t, likewise with the pair rotation (g = gamma with two-endpoint
  //            writes, else 1),   TK1[t] = beta_t / E_t, likewise.
  // A staged element is then one multiply (real rows) or one 2 x 2 product (pairs):
  //   q = R(-Theta_t) C_t E_t,  k = R(-Theta_s) (g B) / E_s.
  // With the shift identity the key table is TK0 = TK1[t] + TK0[t-1] (the key at t
  // carries B_{t-1}), where the entry at t = -1 is gamma of the token before the chunk
  // (gprev) at CD = 0, Theta = 0.  A static row counts tokens instead: CD_t is t + 1 and
  // CD_end the chunk's token count.
  auto tables = [&](int c, float gprev) {
    const int sc = c & 3, sg = c & 3;
    const float hc = 0.5f * sMisc[sc][0], hn = 0.5f * sMisc[sc][2];
    for (int i = tid; i < QT * (N / 2); i += S::NTH) {
      const int t = i / (N / 2), n = 2 * (i % (N / 2));
      const float cd = sCD[sc][t] - hc;
      const float g0 = S::TE ? sGa[sg][t] : 1.f, g1 = S::TE ? sBe[sg][t] : 0.f;
      // shift identity: gamma and the factors of the token before
      const float cdm = t > 0 ? sCD[sc][t - 1] : 0.f;
      float gm = 0.f;
      if constexpr (SH) gm = t > 0 ? sGa[sg][t - 1] : gprev;
      float2 tc, tk0, tk1;
      if (n >= nreal) {
        const float x = sRate[n] * cd;
        const float e = __expf(-x), ei = __expf(x);
        float sn, cs;
        fast_sincos(sOmega[(n - nreal) >> 1] * sCD[sc][t], &sn, &cs);
        tc = make_float2(e * cs, e * sn);
        tk0 = make_float2(g0 * ei * cs, g0 * ei * sn);
        tk1 = make_float2(g1 * ei * cs, g1 * ei * sn);
        if (SH) {
          const float eim = __expf(sRate[n] * (cdm - hc));
          float snm, csm;
          fast_sincos(sOmega[(n - nreal) >> 1] * cdm, &snm, &csm);
          tk0 = make_float2(tk1.x + gm * eim * csm, tk1.y + gm * eim * snm);
        }
      } else {
        // static rows: the token count t + 1 in place of the summed step
        const float cn = static_cast<float>(t + 1) - hn, cnm = static_cast<float>(t) - hn;
        const float x0 = sRate[n] * cd + sRateS[n] * cn, x1 = sRate[n + 1] * cd + sRateS[n + 1] * cn;
        const float ei0 = __expf(x0), ei1 = __expf(x1);
        tc = make_float2(__expf(-x0), __expf(-x1));
        tk0 = make_float2(g0 * ei0, g0 * ei1);
        tk1 = make_float2(g1 * ei0, g1 * ei1);
        if (SH)
          tk0 = make_float2(tk1.x + gm * __expf(sRate[n] * (cdm - hc) + sRateS[n] * cnm),
                            tk1.y + gm * __expf(sRate[n + 1] * (cdm - hc) + sRateS[n + 1] * cnm));
      }
      *reinterpret_cast<float2*>(sTC + t * N + n) = tc;
      *reinterpret_cast<float2*>(sTK0 + t * N + n) = tk0;
      if (S::TE && !SH) *reinterpret_cast<float2*>(sTK1 + t * N + n) = tk1;
    }
  };

  // one staged vector times its table row: per-row factors, or (cos, sin)-style 2 x 2
  // products on pair rows, q = (a u0 + b u1, -b u0 + a u1)
  auto apply_table = [&](float* v, const float* tab, int n0) {
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

  // ---- a2: the operands of chunk c (held in registers) into operand buffer bi, using
  // the chunk's per-token factors (head decay) or its factor tables (per-row decay).
  // Wave PW also stores the per-token scalars loaded with the operands (Delta of chunk
  // c+2, beta / gamma of chunk c+1).
  auto stage = [&](int c, int bi) {
    if (wave == PW && lane < 64) {
      sDT[c & 1][lane] = p.softplus ? softplus_f32(rdt) : rdt;
      if (S::TE) {
        sGa[(c + 1) & 3][lane] = rga;
        sBe[(c + 1) & 3][lane] = rbe;
      }
    }
    const int sc = c & 3;
    T* q = sQ + bi * QSZ;
    T* kb = sK + bi * KSZ;
    T* vb = sV + bi * VSZ;
    T* vwb = sVw + (COORD ? 0 : bi * VSZ);
#pragma unroll
    for (int k = 0; k < S::ALL_PER; ++k) {
      const int u = tid + S::NTH * k;
      if (u >= S::C0 && u < S::C0 + S::C_VECS) {
        const int row = (u - S::C0) / S::NVEC_N, nv = (u - S::C0) % S::NVEC_N;
        const int n0 = nv * VEC;
        if (COORD) {
          const int t = row / R;
          float vals[VEC];
          unpack<BF16>(rr[k], vals);
          apply_table(vals, sTC + t * N, n0);
          *reinterpret_cast<uint4*>(q + row * NS + n0) = pack<BF16>(vals);
          if (SH) *reinterpret_cast<uint4*>(sCraw + row * NS + n0) = rr[k];
        } else {
          *reinterpret_cast<uint4*>(q + row * NS + n0) = rr[k];
        }
      } else if (u >= S::K0 && u < S::K0 + S::K_ITEMS) {
        const int v = u - S::K0;
        const int row = v / S::NVEC_N, nv = v % S::NVEC_N;
        const int n0 = nv * VEC;
        const int sl = row / R - S::TEH, r = row % R;
        if (!COORD && !S::TE) {
          *reinterpret_cast<uint4*>(kb + (sl * KR + r) * NS + n0) = rr[k];
          continue;
        }
        float bv[VEC];
        unpack<BF16>(rr[k], bv);
        if constexpr (SH) {
          // the key at s = sl + 1 carries B_sl; the raw row feeds C_t . B_t
          if (sl + 1 < QT) {
            apply_table(bv, sTK0 + (sl + 1) * N, n0);
            *reinterpret_cast<uint4*>(kb + ((sl + 1) * R + r) * NS + n0) = pack<BF16>(bv);
          }
          if (sl >= 0) *reinterpret_cast<uint4*>(sBraw + (sl * R + r) * NS + n0) = rr[k];
          continue;
        }
        // e = 0: gamma_s B_s written at s = sl; e = 1: beta_{s+1} B_s written at s+1
#pragma unroll
        for (int e = 0; e < 1 + S::TEH; ++e) {
          const int tau = sl + e;
          if (tau < 0 || tau >= QT) continue;
          const int j = tau * KR + (e ? R : 0) + r;
          float uu[VEC];
#pragma unroll
          for (int i = 0; i < VEC; ++i) uu[i] = bv[i];
          apply_table(uu, (e ? sTK1 : sTK0) + tau * N, n0);
          *reinterpret_cast<uint4*>(kb + j * NS + n0) = pack<BF16>(uu);
        }
      } else if (u >= S::X0 && u < S::ALL_VECS) {
        const int v = u - S::X0;
        const int row = v / S::NVEC_P, pv = v % S::NVEC_P;
        const int sl = row / R - S::TEH, r = row % R;
        if constexpr (SH) {
          // X_sl is the value of the key at sl + 1; the last token's goes aside
          if (sl + 1 < QT) *reinterpret_cast<uint4*>(vb + ((sl + 1) * R + r) * VS + pv * VEC) = rr[k];
          else *reinterpret_cast<uint4*>(sXl + (bi * R + r) * VS + pv * VEC) = rr[k];
          continue;
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          if (e == 1 && !S::TE) break;
          const int tau = sl + e;
          if (tau < 0 || tau >= QT || (e == 0 && sl < 0)) continue;
          const int j = tau * KR + (e ? R : 0) + r;
          *reinterpret_cast<uint4*>(vb + j * VS + pv * VEC) = rr[k];
          if (!COORD) {
            const float w = __builtin_amdgcn_exp2f(sLC[sc][QT - 1] - sLC[sc][tau]);  // e^{L_end - L_s}
            float xv[VEC];
            unpack<BF16>(rr[k], xv);
#pragma unroll
            for (int i = 0; i < VEC; ++i) xv[i] *= w;
            *reinterpret_cast<uint4*>(vwb + j * VS + pv * VEC) = pack<BF16>(xv);
          }
        }
      }
    }
  };

  // output rows of chunk c (staged in sYo) to HBM: whole PB-wide row segments,
  // one 16-byte vector per thread
  auto store_rows = [&](int c) {
    const int t0 = c * QT;
    for (int v = tid; v < S::QO * S::NVEC_P; v += S::NTH) {
      const int row = v / S::NVEC_P, pv = v % S::NVEC_P;
      const int t = row / R, o = row % R;
      if (t0 + t < L && o < rout)
        *reinterpret_cast<uint4*>(yg + (t0 + t) * tsY + o * P + pv * VEC) =
            *reinterpret_cast<const uint4*>(sYo + row * VS + pv * VEC);
    }
  };

  // shift identity: h = h' + gamma_t B_t X_t with t the last token of chunk c (operand
  // buffer bi), for four columns pl.. of state row n.  A chunk cut by the sequence end
  // already holds that write: the key at t + 1 (past the end, where beta = 0 and the
  // transition is the identity) carries it.
  auto add_last_write = [&](float* v, int c, int bi, int n, int pl) {
    if constexpr (SH) {
      if ((c + 1) * QT > L) return;
      const int tl = QT - 1;
      const float gl = sGa[c & 3][tl];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float xv[4];
        load4<BF16>(sXl + (bi * R + r) * VS + pl, xv);
        const float bw = gl * to_f32(sBraw[(tl * R + r) * NS + n]);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] += bw * xv[i];
      }
    }
  };

  const int nch = p.nchunks;
  // chunk-boundary states, stored in the io dtype, for chunks of save_chunk tokens: QT, or
  // QT / 2 (the state after each chunk's first half is saved too)
  const size_t sl_saved = (size_t)slice * (p.save_nchunks + 1);
  T* saved = static_cast<T*>(p.saved);
  const bool save_half = S::CAN_HALF && saved && 2 * p.save_chunk == QT;

  // prologue.  The global reads come first -- the factor wave's steps of the first two
  // chunks and beta / gamma of the first, the first chunk's operands, the incoming
  // state -- and are waited for before the first barrier.
  float dt0 = 0.f, dt1 = 0.f, be0 = 0.f, ga0 = 0.f;
  if (wave == PW) {
    const int ta = c0 * QT + lane, tb = ta + QT;
    if (lane < QT && ta < L) {
      dt0 = dtg[ta * H];
      if (S::TE) {
        be0 = beg[ta * H];
        ga0 = gag[ta * H];
      }
    }
    if (lane < QT && tb < L) dt1 = dtg[tb * H];
  }
  load_chunk(c0);
#pragma unroll
  for (int k = 0; k < S::ST_PER_WAVE; ++k) {
    st[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int tile = wave * S::ST_PER_WAVE + k;
    if (h0s && tile < S::ST_TILES) {
      const int n = 16 * (tile / S::TP) + (lane & 15), pl = 16 * (tile % S::TP) + 4 * (lane >> 4);
      const float4 v = *reinterpret_cast<const float4*>(h0s + n * P + pl);
      st[k] = f32x4{v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) st[k][i] -= shift_corr(n, pl + i);
    }
  }
  // score entries above the causal diagonal are zero and never rewritten; so are the
  // operands' padding columns n >= N
  {
    uint4* z = reinterpret_cast<uint4*>(sS);
    for (int i = tid; i < S::QO * KS * (int)sizeof(T) / 16; i += S::NTH) z[i] = zero4;
  }
  if (S::NC > N) {
    for (int i = tid; i < 2 * S::QO * (S::NC - N); i += S::NTH) {
      const int r = i / (S::NC - N), c = N + i % (S::NC - N);
      sQ[r * NS + c] = T(0);
    }
    for (int i = tid; i < 2 * S::QK * (S::NC - N); i += S::NTH) {
      const int r = i / (S::NC - N), c = N + i % (S::NC - N);
      sK[r * NS + c] = T(0);
    }
    if (SH)
      for (int i = tid; i < S::QO * (S::NC - N); i += S::NTH) {
        const int r = i / (S::NC - N), c = N + i % (S::NC - N);
        sCraw[r * NS + c] = T(0);
        sBraw[r * NS + c] = T(0);
      }
  }
  // the readout copy's second buffer, padding rows and padding columns start at zero
  {
    uint4* z = reinterpret_cast<uint4*>(sST + S::NC * VS);
    for (int i = tid; i < S::NC * VS * (int)sizeof(T) / 16; i += S::NTH) z[i] = zero4;
    for (int i = tid; i < (S::NC - N) * VS; i += S::NTH) sST[N * VS + i] = T(0);
    for (int i = tid; i < N * (VS - PB); i += S::NTH) sST[(i / (VS - PB)) * VS + PB + i % (VS - PB)] = T(0);
  }
  // take the incoming state here: left pending into the chunk loop, its loads would
  // make the compiler wait on every outstanding memory operation before each state
  // update
#pragma unroll
  for (int k = 0; k < S::ST_PER_WAVE; ++k) asm volatile("" : "+v"(st[k]));
  if (COORD) {
    if (tid < N) {
      sRate[tid] = r_rate;
      sRateS[tid] = r_rs;
    }
    if (tid < p.n_pairs) sOmega[tid] = r_om;
  }
  if (saved && seg == 0) {
    // slot 0: the state entering chunk 0 (h, not the shifted h')
#pragma unroll
    for (int k = 0; k < S::ST_PER_WAVE; ++k) {
      const int tile = wave * S::ST_PER_WAVE + k;
      if (tile < S::ST_TILES) {
        const int n = 16 * (tile / S::TP) + (lane & 15), pl = 16 * (tile % S::TP) + 4 * (lane >> 4);
        float v[4] = {st[k][0], st[k][1], st[k][2], st[k][3]};
        if (SH)
          for (int i = 0; i < 4; ++i) v[i] += shift_corr(n, pl + i);
        store4<BF16>(saved + (sl_saved * N + n) * P + p0 + pl, v);
      }
    }
  }
  if (COORD && wave == PW) {
    amax = wave_max(tid < N ? fabsf(r_rate) : 0.f);
    smax = wave_max(tid < N ? fabsf(r_rs) : 0.f);
  }
  if (wave == PW) {
    factors(c0, (lane < QT && c0 * QT + lane < L) ? (p.softplus ? softplus_f32(dt0) : dt0) : 0.f);
    if (c0 + 1 < c1) factors(c0 + 1, (lane < QT && (c0 + 1) * QT + lane < L) ? (p.softplus ? softplus_f32(dt1) : dt1) : 0.f);
    if (S::TE) {
      sBe[c0 & 3][lane] = be0;
      sGa[c0 & 3][lane] = ga0;
    }
  }
  __syncthreads();
  // buffer 0 of the readout copy: the incoming state from this wave's state tiles
  // (per-row decay: pre-scaled by e^{-A CD_end / 2} of the first chunk)
  {
    const float hc0 = 0.5f * sMisc[c0 & 3][0], hn0 = 0.5f * sMisc[c0 & 3][2];
#pragma unroll
    for (int k = 0; k < S::ST_PER_WAVE; ++k) {
      const int tile = wave * S::ST_PER_WAVE + k;
      if (tile < S::ST_TILES) {
        const int n = 16 * (tile / S::TP) + (lane & 15), pl = 16 * (tile % S::TP) + 4 * (lane >> 4);
        const float sc0 = COORD ? __expf(-sRate[n] * hc0 - sRateS[n] * hn0) : 1.f;
        const float v[4] = {sc0 * st[k][0], sc0 * st[k][1], sc0 * st[k][2], sc0 * st[k][3]};
        store4<BF16>(sST + n * VS + pl, v);
      }
    }
  }
  if (COORD) tables(c0, gprev0);
  __syncthreads();
  stage(c0, 0);
  if (c0 + 1 < c1) load_chunk(c0 + 1);
  __syncthreads();

  for (int c = c0; c < c1; ++c) {
    const int bi = (c - c0) & 1;
    if (c > c0) store_rows(c - 1);  // drains while the scores compute
    const int sc = c & 3;
    const T* q = sQ + bi * QSZ;
    const T* kb = sK + bi * KSZ;
    const T* vb = sV + bi * VSZ;
    const T* vwb = sVw + (COORD ? 0 : bi * VSZ);

    // ---- phase 1 -- a3: masked intra-chunk scores of chunk c (computed transposed:
    // lane l holds query row 16 ti + (l & 15) against keys 16 tj + 4 (l >> 4) + i),
    // the a4/a5 state update of chunk c, the factor tables of chunk c+1; wave PW also
    // forms the per-token factors of chunk c+2
    for (int tile = wave; tile < S::SC_TILES; tile += NW) {
      int ti = 0, tj = tile;
#pragma unroll
      for (int a = 0; a < S::TQ - 1; ++a) {
        if (tj >= S::row_tiles(ti)) {
          tj -= S::row_tiles(ti);
          ++ti;
        }
      }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < S::NC / 32; ++kk) {
        const auto fk = load_frag<BF16>(kb + (16 * tj + (lane & 15)) * NS + kk * 32 + 8 * (lane >> 4));
        const auto fq = load_frag<BF16>(q + (16 * ti + (lane & 15)) * NS + kk * 32 + 8 * (lane >> 4));
        mma<BF16>(acc, fk, fq);
      }
      const int row = 16 * ti + (lane & 15);
      const int t = row / R;
      const int j0 = 16 * tj + 4 * (lane >> 4);
      float val[4];
      if (COORD) {
#pragma unroll
        for (int i = 0; i < 4; ++i) val[i] = ((j0 + i) / S::KEYS <= t) ? acc[i] : 0.f;
      } else {
        const float lt = sLC[sc][t];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = (j0 + i) / S::KEYS;
          val[i] = (s <= t) ? acc[i] * __builtin_amdgcn_exp2f(lt - sLC[sc][s]) : 0.f;
        }
      }
      store4<BF16>(sS + row * KS + j0, val);
    }
    if constexpr (SH) {
      // same-token products C_t[o] . B_t[r] (raw rows): the diagonal tiles of C B^T,
      // one per query tile, from the wave below the factor wave down
      for (int ti = (2 * NW - 2 - wave) % NW; ti < S::TQ; ti += NW) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < S::NC / 32; ++kk) {
          const auto fb = load_frag<BF16>(sBraw + (16 * ti + (lane & 15)) * NS + kk * 32 + 8 * (lane >> 4));
          const auto fc = load_frag<BF16>(sCraw + (16 * ti + (lane & 15)) * NS + kk * 32 + 8 * (lane >> 4));
          mma<BF16>(acc, fb, fc);
        }
        // lane: query row 16 ti + (lane & 15), key rows 16 ti + 4 (lane >> 4) + i
        const int row = 16 * ti + (lane & 15), j0 = 16 * ti + 4 * (lane >> 4);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if ((j0 + i) / R == row / R) sDG[row * R + (j0 + i) % R] = acc[i];
      }
    }
    // a4/a5: state update of chunk c (needs only this chunk's keys / values and the
    // state entering it); its bf16 copy is the readout operand of chunk c+1.
    // Head decay: S <- e^{-A CD_end} S + K^T (V scaled to the chunk end).  Per-row decay,
    // with the keys k = K~ e^{L_end/2 - L_s} folded around the chunk midpoint and
    // hh = e^{-A_n CD_end/2}:  S <- hh o (hh o S + k^T V)  (= e^{L_end} S + sum_s
    // e^{L_end - L_s} K~_s V_s), then the chunk-total rotation of the pairs.
    {
      // state tiles of this wave: wave * ST_PER_WAVE + k, so a wave's tiles share
      // their n-block whenever TP is a multiple of ST_PER_WAVE (one key fragment
      // then serves all of them)
      const float cdend = sMisc[sc][0], nvend = sMisc[sc][2];
      const float cdnext = c + 1 < c1 ? sMisc[(c + 1) & 3][0] : 0.f;
      const float nvnext = c + 1 < c1 ? sMisc[(c + 1) & 3][2] : 0.f;
      constexpr bool SHARE = S::TP % S::ST_PER_WAVE == 0;
      f32x4 acc[S::ST_PER_WAVE];
      f32x4 acch[S::CAN_HALF ? S::ST_PER_WAVE : 1];  // after the first half's keys
      float hh[S::ST_PER_WAVE];
#pragma unroll
      for (int k = 0; k < S::ST_PER_WAVE; ++k) {
        const int tile = wave * S::ST_PER_WAVE + k;
        const int n = 16 * (tile / S::TP) + (lane & 15);
        const int nn = n < N ? n : 0;
        hh[k] = COORD ? __expf(-0.5f * (sRate[nn] * cdend + sRateS[nn] * nvend)) : sMisc[sc][1];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[k][i] = st[k][i] * hh[k];
      }
#pragma unroll
      for (int kk = 0; kk < S::QK / 32; ++kk) {
        if constexpr (S::CAN_HALF) {
          if (kk == S::KK_HALF) {
#pragma unroll
            for (int k = 0; k < S::ST_PER_WAVE; ++k) acch[k] = acc[k];
          }
        }
        Frag<BF16> fk;
        if (SHARE) {
          const int tn = (wave * S::ST_PER_WAVE) / S::TP;
          if (wave * S::ST_PER_WAVE < S::ST_TILES)
            fk = load_frag_tr<BF16>(kb + (kk * 32) * NS + 16 * tn, NS);
        }
#pragma unroll
        for (int k = 0; k < S::ST_PER_WAVE; ++k) {
          const int tile = wave * S::ST_PER_WAVE + k;
          if (tile < S::ST_TILES) {
            const int tn = tile / S::TP, tp = tile % S::TP;
            if (!SHARE) fk = load_frag_tr<BF16>(kb + (kk * 32) * NS + 16 * tn, NS);
            const auto fv = load_frag_tr<BF16>((COORD ? vb : vwb) + (kk * 32) * VS + 16 * tp, VS);
            mma<BF16>(acc[k], fv, fk);
          }
        }
      }
#pragma unroll
      for (int k = 0; k < S::ST_PER_WAVE; ++k) {
        const int tile = wave * S::ST_PER_WAVE + k;
        if (tile < S::ST_TILES) {
          const int tn = tile / S::TP, tp = tile % S::TP;
          const int n = 16 * tn + (lane & 15);
          float sst = 1.f;  // scale of the readout copy
          if (COORD) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[k][i] *= hh[k];
            sst = __expf(-0.5f * (sRate[n] * cdnext + sRateS[n] * nvnext));
            // chunk-total rotation of the pairs: rows (n, n+1) sit in lanes (l, l^1)
            const bool pair = n >= nreal;
            float sn = 0.f, cs = 1.f;
            if (pair) fast_sincos(sOmega[(n - nreal) >> 1] * cdend, &sn, &cs);
            const float sg = (lane & 1) ? sn : -sn;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float other = swap_adjacent_lanes(acc[k][i]);
              acc[k][i] = pair ? cs * acc[k][i] + sg * other : acc[k][i];
            }
          }
          st[k] = acc[k];
          // the new state is the readout operand of chunk c+1 (other buffer)
          const int pl = 16 * tp + 4 * (lane >> 4);
          float v4[4] = {acc[k][0], acc[k][1], acc[k][2], acc[k][3]};
          const float r4[4] = {sst * acc[k][0], sst * acc[k][1], sst * acc[k][2], sst * acc[k][3]};
          store4<BF16>(sST + (bi ^ 1) * S::NC * VS + n * VS + pl, COORD ? r4 : v4);
          if (saved) {
            if (SH) add_last_write(v4, c, bi, n, pl);  // saved states are h, not h'
            const int slot = save_half ? min(2 * c + 2, p.save_nchunks) : c + 1;
            store4<BF16>(saved + ((sl_saved + slot) * N + n) * P + p0 + pl, v4);
          }
          if constexpr (S::CAN_HALF) {
            // the state after the first half (when the chunk holds more tokens than that):
            // e^{L_m - L_end/2} times the accumulator after the first half's keys
            // (= e^{L_m} S + sum_{s <= m} e^{L_m - L_s} K~_s V_s), turned by the pairs'
            // rotation up to token m, plus the gamma write of token m (whose key, at m + 1,
            // belongs to the second half)
            constexpr int TM = QT / 2 - 1;
            if (save_half && c * QT + TM + 1 < L) {
              const float cdm = sCD[sc][TM];
              const float fm = __expf(-(sRate[n] * (cdm - 0.5f * cdend) +
                                        sRateS[n] * (static_cast<float>(TM + 1) - 0.5f * nvend)));
              float m4[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) m4[i] = acch[k][i] * fm;
              const bool pair = n >= nreal;
              float sn = 0.f, cs = 1.f;
              if (pair) fast_sincos(sOmega[(n - nreal) >> 1] * cdm, &sn, &cs);
              const float sg = (lane & 1) ? sn : -sn;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float other = swap_adjacent_lanes(m4[i]);
                m4[i] = pair ? cs * m4[i] + sg * other : m4[i];
              }
              const float gm = sGa[c & 3][TM];
#pragma unroll
              for (int r = 0; r < R; ++r) {
                float xv[4];  // X_m: the value row of the key at m + 1
                load4<BF16>(sV + bi * VSZ + ((TM + 1) * R + r) * VS + pl, xv);
                const float bw = gm * to_f32(sBraw[(TM * R + r) * NS + n]);
#pragma unroll
                for (int i = 0; i < 4; ++i) m4[i] += bw * xv[i];
              }
              store4<BF16>(saved + ((sl_saved + 2 * c + 1) * N + n) * P + p0 + pl, m4);
            }
          }
        }
      }
    }
    if constexpr (COORD) {
      if (c + 1 < c1) {
        float gp = 0.f;  // shift identity: gamma of this chunk's last token
        if constexpr (SH) gp = sGa[c & 3][QT - 1];
        tables(c + 1, gp);
      }
    }
    if (wave == PW && c + 2 < c1) factors(c + 2, (lane < QT && (c + 2) * QT + lane < L) ? sDT[c & 1][lane] : 0.f);
    __syncthreads();

    // ---- phase 2 -- a2 staging of chunk c+1 (other buffer) and the loads of chunk
    // c+2 first: the staging waits on this wave's outstanding memory operations, so
    // it runs before this phase's stores are issued (they then drain for a whole
    // chunk).  Then a6 readout + output of chunk c.
    // Output tiles are transposed: lane l holds row 16 ti + (l & 15), columns
    // p = 16 tp + 4 (l >> 4) + i.
    if (c + 1 < c1) {
      stage(c + 1, bi ^ 1);
      if (c + 2 < c1) load_chunk(c + 2);
    }
    // Output tiles in blocks of YBQ x YBP per wave (each fragment read from LDS feeds
    // YBP or YBQ MFMAs), taken from the last wave down so that they overlap the
    // staging, which loads the first waves.
    {
      constexpr int BQ = S::YBQ, BP = S::YBP, NBP = S::TP / BP;
      constexpr int NBLK = (S::TQ / BQ) * NBP;
      for (int blk = NW - 1 - wave; blk < NBLK; blk += NW) {
        const int ti0 = (blk / NBP) * BQ, tp0 = (blk % NBP) * BP;
        f32x4 acc[BQ][BP];
#pragma unroll
        for (int a = 0; a < BQ; ++a)
#pragma unroll
          for (int bb = 0; bb < BP; ++bb) acc[a][bb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < S::NC / 32; ++kk) {
          Frag<BF16> fs[BP], fq[BQ];
#pragma unroll
          for (int bb = 0; bb < BP; ++bb)
            fs[bb] = load_frag_tr<BF16>(sST + bi * S::NC * VS + (kk * 32) * VS + 16 * (tp0 + bb), VS);
#pragma unroll
          for (int a = 0; a < BQ; ++a)
            fq[a] = load_frag<BF16>(q + (16 * (ti0 + a) + (lane & 15)) * NS + kk * 32 + 8 * (lane >> 4));
#pragma unroll
          for (int a = 0; a < BQ; ++a)
#pragma unroll
            for (int bb = 0; bb < BP; ++bb) mma<BF16>(acc[a][bb], fs[bb], fq[a]);
        }
        if (!COORD) {
#pragma unroll
          for (int a = 0; a < BQ; ++a) {
            const int t = (16 * (ti0 + a) + (lane & 15)) / R;
            const float el = __builtin_amdgcn_exp2f(sLC[sc][t]);  // e^{L_t}
#pragma unroll
            for (int bb = 0; bb < BP; ++bb)
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[a][bb][i] *= el;
          }
        }
        // intra-chunk part: keys up to the block's last query token (the lower query
        // tiles see zero scores past their own diagonal)
        const int tmax = (16 * (ti0 + BQ - 1) + 15) / R;
        const int kend = ((tmax + 1) * S::KEYS + 31) / 32;
        for (int kk = 0; kk < kend; ++kk) {
          Frag<BF16> fv[BP], fsc[BQ];
#pragma unroll
          for (int bb = 0; bb < BP; ++bb)
            fv[bb] = load_frag_tr<BF16>(vb + (kk * 32) * VS + 16 * (tp0 + bb), VS);
#pragma unroll
          for (int a = 0; a < BQ; ++a)
            fsc[a] = load_frag<BF16>(sS + (16 * (ti0 + a) + (lane & 15)) * KS + kk * 32 + 8 * (lane >> 4));
#pragma unroll
          for (int a = 0; a < BQ; ++a)
#pragma unroll
            for (int bb = 0; bb < BP; ++bb) mma<BF16>(acc[a][bb], fv[bb], fsc[a]);
        }
#pragma unroll
        for (int a = 0; a < BQ; ++a) {
          const int row = 16 * (ti0 + a) + (lane & 15);
          const int t = row / R, o = row % R;
#pragma unroll
          for (int bb = 0; bb < BP; ++bb) {
            const int pl = 16 * (tp0 + bb) + 4 * (lane >> 4);
            float val[4] = {acc[a][bb][0], acc[a][bb][1], acc[a][bb][2], acc[a][bb][3]};
            // X_t of rank r: a value row of this chunk (shift identity: the key at t + 1,
            // or the last token's rows set aside)
            auto xrow = [&](int r) -> const T* {
              if (!SH) return vb + (t * KR + r) * VS + pl;
              return t + 1 < QT ? vb + ((t + 1) * R + r) * VS + pl : sXl + (bi * R + r) * VS + pl;
            };
            if constexpr (SH) {
              // same-token term gamma_t (C_t . B_t) X_t
              const float gt = sGa[c & 3][t];
#pragma unroll
              for (int r = 0; r < R; ++r) {
                float xv[4];
                load4<BF16>(xrow(r), xv);
                const float w = gt * sDG[row * R + r];
#pragma unroll
                for (int i = 0; i < 4; ++i) val[i] += w * xv[i];
              }
            }
            if (p.has_D) {
              float xv[4];
              load4<BF16>(xrow(o), xv);
#pragma unroll
              for (int i = 0; i < 4; ++i) val[i] += Dh * xv[i];
            }
            store4<BF16>(sYo + row * VS + pl, val);
          }
        }
      }
    }
    __syncthreads();
  }
  // per-row decay: flag the range when one of its chunks was too steep for the fold (its
  // outputs are then rewritten by the token-by-token forward)
  if constexpr (COORD)
    if (tid == 0 && p.wild) p.wild[lid] = steep ? 1 : 0;
  store_rows(c1 - 1);
  // the final state after the last segment
  float* hf = (seg == p.nseg - 1 && p.h_final) ? p.h_final + (size_t)slice * N * P + p0 : nullptr;
  if (hf) {
#pragma unroll
    for (int k = 0; k < S::ST_PER_WAVE; ++k) {
      const int tile = wave * S::ST_PER_WAVE + k;
      if (tile < S::ST_TILES) {
        const int n = 16 * (tile / S::TP) + (lane & 15), pl = 16 * (tile % S::TP) + 4 * (lane >> 4);
        float v[4] = {st[k][0], st[k][1], st[k][2], st[k][3]};
        if (SH) add_last_write(v, c1 - 1, (c1 - 1 - c0) & 1, n, pl);
        *reinterpret_cast<float4*>(hf + n * P + pl) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
  }
}

// ------------------------------------------------------------------ segment combine
// States entering the segments of each slice, in order: starting from h0 (or 0), the
// local-pass ranges of every segment are chained in token order,
//   S <- rho_u R(theta_u) S + S_local[u],
// with rho_u = e^{-A_n D_u} per row, theta_u = omega_k D_u per pair and D_u the range's
// summed step (the token-by-token decays and rotations of a range compose to exactly
// these); after the last range of segment s, S is the state entering segment s + 1.
// One thread per (slice, row pair, value column).
__global__ __launch_bounds__(256) void ssm_fwd_combine(FwdParams p, int per_row) {
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
    // decay by their rate once per token: over a range, the range's token count
    const bool stat = per_row && n < p.n_static;
    const bool pair = per_row && n >= nreal;
    const float om = pair ? p.omega[(size_t)h * p.n_pairs + ((n - nreal) >> 1)] : 0.f;
    const size_t sb = (size_t)slice * p.nseg, sl = (size_t)slice * (p.nseg - 1) * p.nsub;
    float a = 0.f, bv = 0.f;
    if (p.h0) {
      a = p.h0[((size_t)slice * N + n) * P + pp];
      bv = p.h0[((size_t)slice * N + n + 1) * P + pp];
    }
    for (int s = 0; s + 1 < p.nseg; ++s) {
      // ranges in blocks of kCombineBlock: a block's reads are issued together, then
      // chained (one memory round trip per block instead of per range)
      for (int u0 = 0; u0 < p.nsub; u0 += kCombineBlock) {
        const int cnt = min(kCombineBlock, p.nsub - u0);
        float ds[kCombineBlock], l0[kCombineBlock], l1[kCombineBlock];
#pragma unroll
        for (int k = 0; k < kCombineBlock; ++k) {
          const size_t unit = sl + (size_t)s * p.nsub + u0 + (k < cnt ? k : 0);
          const float* loc = p.seg_local + (unit * N + n) * P + pp;
          ds[k] = p.seg_delta[unit];
          l0[k] = loc[0];
          l1[k] = loc[P];
        }
#pragma unroll
        for (int k = 0; k < kCombineBlock; ++k) {
          if (k >= cnt) break;
          float dsum = ds[k];
          if (stat) {  // tokens of range u0 + k of segment s (ranges past the sequence end are empty)
            const int ta = s * p.seg_tokens + (u0 + k) * p.lsub;
            const int tb = min(min(ta + p.lsub, (s + 1) * p.seg_tokens), p.L) - 1;
            dsum = static_cast<float>(max(tb - ta + 1, 0));
          }
          float a2 = a * expf(-ra * dsum), b2 = bv * expf(-rb * dsum);
          if (pair) {
            float sn, cs;
            sincosf(om * dsum, &sn, &cs);
            const float x0 = a2, x1 = b2;
            a2 = cs * x0 - sn * x1;
            b2 = sn * x0 + cs * x1;
          }
          a = a2 + l0[k];
          bv = b2 + l1[k];
        }
      }
      float* out = p.seg_in + ((sb + s + 1) * N + n) * P + pp;
      out[0] = a;
      out[P] = bv;
    }
  }
}

// ------------------------------------------------------------------ dispatch
// (io bf16?, N, P-block, R, keys per token, tokens per chunk, per-row decay, threads)
#define SSM_FWD_VARIANTS(X)                 \
  /* fp32 io */                             \
  X(false, 16, 16, 1, 1, 64, false, 256)         \
  X(false, 32, 16, 1, 1, 64, false, 256)         \
  X(false, 32, 16, 2, 2, 32, false, 256)         \
  X(false, 16, 16, 1, 2, 16, true, 256)          \
  X(false, 32, 16, 1, 2, 16, true, 256)          \
  X(false, 32, 16, 2, 4, 16, true, 256)          \
  X(false, 32, 16, 1, 1, 32, true, 256)          \
  X(false, 32, 16, 2, 2, 16, true, 256)          \
  /* bf16 io, head decay */                 \
  X(true, 32, 16, 1, 1, 64, false, 256)          \
  X(true, 64, 16, 1, 1, 64, false, 256)          \
  X(true, 64, 16, 1, 1, 32, false, 256)          \
  X(true, 128, 16, 1, 1, 64, false, 256)         \
  X(true, 128, 32, 1, 1, 64, false, 256)         \
  X(true, 128, 64, 1, 1, 64, false, 256)         \
  X(true, 128, 16, 1, 1, 64, false, 512)    \
  X(true, 128, 32, 1, 1, 64, false, 512)    \
  X(true, 128, 64, 1, 1, 64, false, 512)    \
  X(true, 128, 64, 1, 1, 64, false, 1024)   \
  X(true, 128, 32, 1, 1, 64, false, 1024)   \
  X(true, 64, 16, 2, 2, 32, false, 256)          \
  X(true, 64, 16, 4, 4, 16, false, 256)          \
  X(true, 64, 32, 4, 4, 16, false, 256)          \
  X(true, 64, 16, 4, 4, 8, false, 256)           \
  /* bf16 io, per-row decay / pairs / two-endpoint */ \
  X(true, 32, 16, 1, 2, 16, true, 256)           \
  X(true, 64, 16, 1, 2, 16, true, 256)           \
  X(true, 64, 16, 2, 4, 16, true, 256)           \
  X(true, 64, 16, 2, 4, 8, true, 256)            \
  X(true, 64, 32, 2, 4, 16, true, 256)           \
  X(true, 64, 16, 1, 1, 32, true, 256)           \
  X(true, 64, 16, 2, 2, 16, true, 256)           \
  X(true, 64, 16, 4, 4, 16, true, 256)           \
  X(true, 64, 16, 4, 8, 8, true, 256)      \
  X(true, 64, 64, 1, 1, 64, false, 1024)   \
  X(true, 64, 64, 4, 4, 16, false, 1024)   \
  X(true, 64, 32, 4, 4, 16, false, 1024)   \
  X(true, 64, 16, 4, 4, 16, false, 1024)   \
  X(true, 64, 64, 2, 4, 16, true, 1024)    \
  X(true, 64, 32, 2, 4, 16, true, 1024)    \
  X(true, 64, 16, 2, 4, 16, true, 1024)    \
  X(true, 64, 16, 2, 4, 16, true, 512)     \
  X(true, 64, 64, 1, 2, 16, true, 1024)    \
  X(true, 64, 32, 1, 2, 16, true, 1024)    \
  X(true, 64, 16, 1, 2, 16, true, 1024)    \
  /* two-endpoint writes, two chunks per step (forward without saved states) */ \
  X(false, 16, 16, 1, 2, 32, true, 256)    \
  X(false, 32, 16, 1, 2, 32, true, 256)    \
  X(false, 32, 16, 2, 4, 32, true, 256)    \
  X(true, 32, 16, 1, 2, 32, true, 256)     \
  X(true, 64, 16, 1, 2, 32, true, 256)     \
  X(true, 64, 16, 2, 4, 32, true, 256)     \
  X(true, 64, 32, 2, 4, 32, true, 256)     \
  X(true, 64, 64, 2, 4, 32, true, 1024)    \
  X(true, 64, 32, 2, 4, 32, true, 1024)    \
  X(true, 64, 16, 2, 4, 32, true, 1024)    \
  X(true, 64, 16, 2, 4, 32, true, 512)     \
  X(true, 64, 64, 1, 2, 32, true, 1024)    \
  X(true, 64, 32, 1, 2, 32, true, 1024)    \
  X(true, 64, 16, 1, 2, 32, true, 1024)

bool fwd_variant_exists(const FwdKey& k) {
#define SSM_FWD_MATCH(BF, NN, PBB, RR, KRR, QTT, CO, NT)                                     \
  if (k.bf16 == BF && k.N == NN && k.PB == PBB && k.R == RR && k.KR == KRR && k.QT == QTT && \
      k.coord == CO && k.nthreads == NT)                                                     \
    return true;
  SSM_FWD_VARIANTS(SSM_FWD_MATCH)
#undef SSM_FWD_MATCH
  return false;
}

// the forward's local pass: B keys and x values over the ranges of segments 0 .. nseg-2
static LocalParams local_params(const FwdParams& p) {
  LocalParams l{};
  l.key = p.B; l.val = p.x; l.key_prev = p.B_prev; l.val_prev = p.x_prev;
  l.dt = p.dt; l.A = p.A; l.omega = p.omega; l.beta = p.beta;
  l.gamma = p.gamma; l.out = p.seg_local; l.delta = p.seg_delta; l.rk = p.rin;
  l.batch = p.batch; l.L = p.L; l.H = p.H; l.G = p.G; l.P = p.P; l.n_real = p.n_real;
  l.n_static = p.n_static;
  l.n_pairs = p.n_pairs; l.softplus = p.softplus; l.head_rates = p.head_rates;
  l.nseg = p.nseg; l.seg_tokens = p.seg_tokens; l.nsub = p.nsub; l.lsub = p.lsub;
  return l;
}

hipError_t launch_fwd(const FwdKey& k, const FwdParams& p, hipStream_t stream,
                      void* const* events) {
  const int nwg = p.batch * p.H * p.npblk * p.nseg;
  if (nwg == 0 || p.nchunks == 0) return hipSuccess;
  auto mark = [&](int i) {
    if (events && events[i]) (void)hipEventRecord(static_cast<hipEvent_t>(events[i]), stream);
  };
#define SSM_FWD_LAUNCH(BF, NN, PBB, RR, KRR, QTT, CO, NT)                                    \
  if (k.bf16 == BF && k.N == NN && k.PB == PBB && k.R == RR && k.KR == KRR && k.QT == QTT && \
      k.coord == CO && k.nthreads == NT) {                                                   \
    mark(0);                                                                                 \
    if (p.nseg > 1) {                                                                        \
      launch_local<BF, NN, RR, (KRR > RR), CO, false>(local_params(p), stream);            \
      const long total = (long)p.batch * p.H * (NN / 2) * p.P;                               \
      const int cb = (int)std::min<long>((total + 255) / 256, 2048);                         \
      hipLaunchKernelGGL(ssm_fwd_combine, dim3(cb), dim3(256), 0, stream, p, CO ? 1 : 0);    \
    }                                                                                        \
    hipLaunchKernelGGL((ssm_fwd_kernel<BF, NN, PBB, RR, KRR, QTT, CO, NT>), dim3(nwg),        \
                       dim3(NT), 0, stream, p);                                              \
    if constexpr (CO) launch_fwd_exact<BF, NN, RR>(p, QTT, stream);                           \
    mark(1);                                                                                 \
    return hipGetLastError();                                                                \
  }
  SSM_FWD_VARIANTS(SSM_FWD_LAUNCH)
#undef SSM_FWD_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace ssm
