// ssm_api.cpp -- the exported C ABI (include/ssm_scan.h): descriptor validation,
// plan selection (kernel variant, chunk length, P-blocks), launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "ssm_kernels.hpp"
#include "ssm_scan.h"

namespace {

using ssm::BwdKey;
using ssm::FwdKey;

// Fills for an empty sequence or batch, where no scan runs but some outputs are not empty:
// the state after no tokens is the initial one, and sums over no tokens are zero.  A fill
// kernel rather than a memset, so that a caller may capture the call in a graph.
__global__ void __launch_bounds__(256) copy_or_zero_kernel(float* __restrict__ dst,
                                                           const float* __restrict__ src,
                                                           size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = src ? src[i] : 0.f;
}

// dst[0, n) = src[0, n), or zeros when src is NULL; nothing when dst is NULL or n is 0.
hipError_t copy_or_zero(float* dst, const float* src, size_t n, hipStream_t s) {
  if (!dst || n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 2048);
  hipLaunchKernelGGL(copy_or_zero_kernel, dim3(blocks), dim3(256), 0, s, dst, src, n);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) zero_bytes_kernel(unsigned char* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = 0;
}

// dst[0, n) = 0 (any element type); nothing when dst is NULL or n is 0
hipError_t zero_bytes(void* dst, size_t n, hipStream_t s) {
  if (!dst || n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 2048);
  hipLaunchKernelGGL(zero_bytes_kernel, dim3(blocks), dim3(256), 0, s,
                     static_cast<unsigned char*>(dst), n);
  return hipGetLastError();
}

size_t state_floats(const ssm_desc* d) {
  return (size_t)d->batch * d->nheads * d->dstate * d->headdim;
}

struct Plan {
  bool coord_kernel;  // per-row kernel (per-row rates, pairs or two-endpoint writes)
  bool head_rates;    // per-row kernel fed one rate per head
  int R, KR, QT, nchunks;
  bool bf16;
};

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  return (v && *v) ? std::atoi(v) : dflt;
}

// Shape rules of the operation itself (independent of what is implemented).
int check_operation(const ssm_desc* d) {
  if (!d) return SSM_ERR_NULL;
  if (d->io_dtype != SSM_F32 && d->io_dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (d->batch < 0 || d->seqlen < 0 || d->nheads <= 0 || d->ngroups <= 0 || d->headdim <= 0 ||
      d->dstate <= 0 || d->rank_in <= 0 || d->rank_out <= 0 || d->n_real < 0 ||
      d->n_pairs < 0 || d->chunk < 0)
    return SSM_ERR_SHAPE;
  if (d->nheads % d->ngroups) return SSM_ERR_SHAPE;
  if (d->n_real + 2 * d->n_pairs != d->dstate) return SSM_ERR_SHAPE;
  if (d->decay_mode != SSM_DECAY_HEAD && d->decay_mode != SSM_DECAY_COORD) return SSM_ERR_SHAPE;
  if (d->decay_mode == SSM_DECAY_HEAD && d->n_pairs != 0) return SSM_ERR_SHAPE;
  if (d->flags & ~(SSM_F_DT_SOFTPLUS | SSM_F_TWO_ENDPOINT | SSM_F_HAS_D)) return SSM_ERR_SHAPE;
  if ((d->flags & SSM_F_HAS_D) && d->rank_in != d->rank_out) return SSM_ERR_SHAPE;
  if (d->n_static < 0 || d->n_static > d->n_real) return SSM_ERR_SHAPE;
  if (d->decay_mode == SSM_DECAY_HEAD && d->n_static != 0) return SSM_ERR_SHAPE;
  return SSM_OK;
}

int make_plan(const ssm_desc* d, Plan* pl) {
  int rc = check_operation(d);
  if (rc) return rc;
  if (d->headdim % 16) return SSM_ERR_UNSUPPORTED;
  if (d->n_pairs > 0 && (d->n_real % 2)) return SSM_ERR_UNSUPPORTED;
  if (d->n_static % 2) return SSM_ERR_UNSUPPORTED;  // the kernels take real rows in pairs
  // kernels index inside a tensor with 32-bit offsets
  const int rmax = std::max(d->rank_in, d->rank_out);
  const double elems = (double)d->batch * d->seqlen * d->nheads * rmax *
                       (d->headdim > d->dstate ? d->headdim : d->dstate);
  if (elems >= 2147483648.0) return SSM_ERR_UNSUPPORTED;
  const bool te = (d->flags & SSM_F_TWO_ENDPOINT) != 0;
  pl->bf16 = d->io_dtype == SSM_BF16;
  pl->coord_kernel = d->decay_mode == SSM_DECAY_COORD || te || d->n_pairs > 0;
  pl->head_rates = d->decay_mode == SSM_DECAY_HEAD;
  // the kernels tile with the larger rank; the narrower side's extra rows are zero
  pl->R = rmax;
  pl->KR = te ? 2 * rmax : rmax;
  int qt = d->chunk;
  if (qt == 0) {
    if (!pl->coord_kernel) qt = 64 / rmax;
    else qt = (16 * pl->KR >= 32) ? 16 : 32 / pl->KR;
    if (qt < 1) qt = 1;
  }
  pl->QT = qt;
  pl->nchunks = (d->seqlen + qt - 1) / qt;
  // a forward variant must exist for this shape
  for (int pb : {64, 32, 16})
    for (int nt : {1024, 512, 256}) {
      FwdKey k{pl->bf16, d->dstate, pb, pl->R, pl->KR, pl->QT, pl->coord_kernel, nt};
      if (d->headdim % pb == 0 && ssm::fwd_variant_exists(k)) return SSM_OK;
    }
  return SSM_ERR_UNSUPPORTED;
}

// Forward variant: P-block width and workgroup size.  Preference: the widest
// workgroup that exists, with the P-block chosen so that (batch x heads x
// P-blocks) workgroups cover the machine without needless P-splitting (a split
// recomputes the chunk scores once per block).  SSM_FWD_PB / SSM_FWD_THREADS
// force a choice among the instantiated variants (experiments).
// Sequence segments: when the (slice, P-block) units alone leave compute units idle,
// each sequence is split into segments that run in parallel and exchange their
// boundary states (local pass, combine, full pass).  Each segment keeps at least
// kMinSegChunks chunks.  The choice depends on the descriptor only, because the
// workspace size follows from it.
constexpr long kTargetUnits = 256;  // compute units of an MI355X
constexpr int kMinSegChunks = 4;
struct Segs {
  int nseg, cps;
};
Segs segments(long units, int nch) {
  if (nch <= 0) return {1, 1};  // empty sequence: nothing to split
  int nseg = 1;
  const int force = env_int("SSM_NSEG", 0);
  if (force > 0) {
    nseg = force;
  } else if (units < kTargetUnits * 3 / 4) {
    nseg = (int)std::min<long>(kTargetUnits / std::max(units, 1L), nch / kMinSegChunks);
  }
  nseg = std::max(1, std::min(nseg, std::max(nch, 1)));
  const int cps = (nch + nseg - 1) / nseg;
  return {(nch + cps - 1) / cps, cps};  // no empty segment
}

FwdKey choose_fwd(const ssm_desc* d, const Plan& pl) {
  const int force_pb = env_int("SSM_FWD_PB", 0);
  const int force_nt = env_int("SSM_FWD_THREADS", 0);
  const long slices = (long)d->batch * d->nheads;
  FwdKey best{pl.bf16, d->dstate, 0, pl.R, pl.KR, pl.QT, pl.coord_kernel, 0};
  long best_score = -1;
  for (int pb : {64, 32, 16}) {
    if (d->headdim % pb) continue;
    if (force_pb && pb != force_pb) continue;
    for (int nt : {1024, 512, 256}) {
      if (force_nt && nt != force_nt) continue;
      FwdKey k{pl.bf16, d->dstate, pb, pl.R, pl.KR, pl.QT, pl.coord_kernel, nt};
      if (!ssm::fwd_variant_exists(k)) continue;
      // score: enough workgroups (counting sequence segments) to occupy the 256
      // compute units (at least ~0.75 of them), then the widest P-block, then the
      // fewest segments, then the widest workgroup
      const long wgs = slices * (d->headdim / pb);
      const Segs sg = segments(wgs, pl.nchunks);
      const long units = wgs * sg.nseg;
      const long score = (units >= 192 ? 1000000L : units * 1000L) + pb * 100L - sg.nseg + nt / 64;
      if (score > best_score) {
        best_score = score;
        best = k;
      }
    }
  }
  if (best_score < 0) {
    // forced combination not instantiated: fall back to any existing variant
    for (int pb : {64, 32, 16})
      for (int nt : {1024, 512, 256}) {
        FwdKey k{pl.bf16, d->dstate, pb, pl.R, pl.KR, pl.QT, pl.coord_kernel, nt};
        if (d->headdim % pb == 0 && ssm::fwd_variant_exists(k)) return k;
      }
  }
  return best;
}

}  // namespace

extern "C" {

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

const char* ssm_status_string(int s) {
  switch (s) {
    case SSM_OK: return "ok";
    case SSM_ERR_NULL: return "required pointer is NULL (or an unused one is set)";
    case SSM_ERR_SHAPE: return "inconsistent sizes or flags";
    case SSM_ERR_DTYPE: return "unknown io dtype";
    case SSM_ERR_ALIGN: return "pointer not 16-byte aligned";
    case SSM_ERR_UNSUPPORTED: return "shape or mode not implemented by this library";
    case SSM_ERR_WORKSPACE: return "workspace too small";
    case SSM_ERR_HIP: return "HIP launch failed";
    case SSM_ERR_SCRATCH: return "problem needs more workspace than the static scratch array holds";
    default: return "unknown status";
  }
}

int ssm_check_desc(const ssm_desc* d) {
  Plan pl;
  return make_plan(d, &pl);
}

int ssm_chunk_tokens(const ssm_desc* d) {
  Plan pl;
  const int rc = make_plan(d, &pl);
  return rc ? rc : pl.QT;
}

size_t ssm_saved_bytes(const ssm_desc* d) {
  Plan pl;
  if (make_plan(d, &pl)) return 0;
  return (size_t)d->batch * d->nheads * (pl.nchunks + 1) * d->dstate * d->headdim * (pl.bf16 ? 2 : 4);
}

static int npart_of(const ssm_desc* d, const Plan& pl) {
  const int na = (pl.coord_kernel && !pl.head_rates) ? d->n_real + d->n_pairs : 1;
  return na + d->n_pairs + 1;
}

// boundary adjoints: one slot per chunk and one after the last token (dh_final or zero)
static size_t bwd_gseg_bytes(const ssm_desc* d, const Plan& pl) {
  return (size_t)d->batch * d->nheads * (pl.nchunks + 1) * d->dstate * d->headdim * (pl.bf16 ? 2 : 4);
}

// head groups shared by several heads: per-head dB and dC partials in the io dtype
static size_t group_partial_one(const ssm_desc* d, const Plan& pl) {
  const size_t one = (size_t)d->batch * d->seqlen * d->nheads * pl.R * d->dstate * (pl.bf16 ? 2 : 4);
  return (one + 255) / 256 * 256;
}
static size_t group_partial_bytes(const ssm_desc* d, const Plan& pl) {
  return d->ngroups == d->nheads ? 0 : 2 * group_partial_one(d, pl);
}

// per-row kernel: one flag per (slice, chunk) item marking chunks too steep for the fold
static size_t bwd_flags_bytes(const ssm_desc* d, const Plan& pl) {
  if (!pl.coord_kernel) return 0;
  return ((size_t)(d->batch * d->nheads * pl.nchunks + 1) * sizeof(int) + 255) / 256 * 256;
}

// local-pass ranges of a segment: as few as keep each within kLocalMaxTokens tokens
struct LocalRanges {
  int seg_tokens, nsub, lsub;
};
static LocalRanges local_ranges(const Plan& pl, const Segs& sg) {
  const int st = sg.cps * pl.QT;
  const int nsub = (st + ssm::kLocalMaxTokens - 1) / ssm::kLocalMaxTokens;
  return {st, nsub, (st + nsub - 1) / nsub};
}

// workspace of the segmented forward: the range states of the local pass, the states
// entering the segments and the ranges' summed steps
static size_t fwd_segment_bytes(const ssm_desc* d, const Plan& pl, const FwdKey& key) {
  const long slices = (long)d->batch * d->nheads;
  const Segs sg = segments(slices * (d->headdim / key.PB), pl.nchunks);
  if (sg.nseg <= 1) return 0;
  const LocalRanges lr = local_ranges(pl, sg);
  const size_t np = (size_t)d->dstate * d->headdim;
  const size_t loc = (size_t)slices * (sg.nseg - 1) * lr.nsub * np * sizeof(float);
  const size_t in = (size_t)slices * sg.nseg * np * sizeof(float);
  return loc + in + ((size_t)slices * (sg.nseg - 1) * lr.nsub * sizeof(float) + 255) / 256 * 256;
}

static size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// workspace of the forward: the segment buffers, then (per-row kernel) one flag per
// workgroup marking ranges that hold a chunk too steep for the midpoint fold
static size_t fwd_flags_bytes(const ssm_desc* d, const Plan& pl, const FwdKey& key) {
  if (!pl.coord_kernel) return 0;
  const long slices = (long)d->batch * d->nheads;
  const int npblk = d->headdim / key.PB;
  const Segs sg = segments(slices * npblk, pl.nchunks);
  return align256((size_t)slices * npblk * sg.nseg * sizeof(int));
}
static size_t fwd_workspace(const ssm_desc* d, const Plan& pl, const FwdKey& key) {
  return align256(fwd_segment_bytes(d, pl, key)) + fwd_flags_bytes(d, pl, key);
}

// boundary-adjoint sweep segments: one workgroup per (slice, segment)
static Segs adj_segments(const ssm_desc* d, const Plan& pl) {
  return segments((long)d->batch * d->nheads, pl.nchunks);
}

// workspace of the segmented boundary-adjoint sweep: the range adjoints of the local
// pass, the adjoints flowing into the segments and the ranges' summed steps
static size_t adj_segment_bytes(const ssm_desc* d, const Plan& pl) {
  const Segs sg = adj_segments(d, pl);
  if (sg.nseg <= 1) return 0;
  const LocalRanges lr = local_ranges(pl, sg);
  const size_t slices = (size_t)d->batch * d->nheads, np = (size_t)d->dstate * d->headdim;
  const size_t loc = slices * (sg.nseg - 1) * lr.nsub * np * sizeof(float);
  const size_t in = slices * sg.nseg * np * sizeof(float);
  return loc + in + (slices * (sg.nseg - 1) * lr.nsub * sizeof(float) + 255) / 256 * 256;
}

size_t ssm_workspace_bytes(const ssm_desc* d, int for_backward) {
  Plan pl;
  if (make_plan(d, &pl)) return 0;
  if (!for_backward) {
    const FwdKey key = choose_fwd(d, pl);
    return key.PB > 0 ? fwd_workspace(d, pl, key) : 0;
  }
  const size_t g = (bwd_gseg_bytes(d, pl) + 255) / 256 * 256;
  const size_t part = (size_t)d->batch * d->nheads * pl.nchunks * npart_of(d, pl) * sizeof(float);
  return g + (part + 255) / 256 * 256 + adj_segment_bytes(d, pl) + group_partial_bytes(d, pl) +
         bwd_flags_bytes(d, pl);
}

}  // extern "C"

namespace {

// ------------------------------------------------------------------ static scratch
// Workspace of ssm_scan_fwd_noalloc: one array per device in the library's code object,
// held until the process ends.  Host code never passes `scratch` itself to a kernel (in
// host code the name is a stand-in, not a device address): each device's address comes
// from hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's scratch address (SSM_OK), or SSM_ERR_HIP.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SSM_ERR_HIP;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!ptr) {
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SSM_ERR_HIP;
      g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return SSM_OK;
}

// The forward scan.  With `use_scratch` the workspace is the device's static scratch
// array (ws / ws_bytes unused): a problem whose workspace exceeds it is rejected before
// any HIP call.
int scan_fwd_impl(const ssm_desc* d, const ssm_fwd_args* a, void* ws, size_t ws_bytes,
                  void* stream, bool use_scratch) {
  Plan pl;
  int rc = make_plan(d, &pl);
  if (rc) return rc;
  if (!a) return SSM_ERR_NULL;
  // an empty problem reads no inputs (empty tensors may have NULL pointers); with no tokens
  // the final state is h0 (zero without it)
  if (d->batch == 0 || d->seqlen == 0) {
    const hipError_t e = copy_or_zero(a->h_final, a->h0, state_floats(d),
                                      static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
  }
  const bool te = (d->flags & SSM_F_TWO_ENDPOINT) != 0;
  const bool hasD = (d->flags & SSM_F_HAS_D) != 0;
  if (!a->x || !a->B || !a->C || !a->dt || !a->A || !a->y) return SSM_ERR_NULL;
  if ((d->n_pairs > 0) != (a->omega != nullptr)) return SSM_ERR_NULL;
  if (te != (a->beta != nullptr) || te != (a->gamma != nullptr)) return SSM_ERR_NULL;
  if (hasD != (a->D != nullptr)) return SSM_ERR_NULL;
  if ((a->x_prev != nullptr) != (a->B_prev != nullptr) || (a->x_prev && !te)) return SSM_ERR_NULL;
  for (const void* q : {a->x, a->B, a->C, (const void*)a->y})
    if (!aligned(q, 16)) return SSM_ERR_ALIGN;
  for (const void* q : {a->x_prev, a->B_prev})
    if (q && !aligned(q, 16)) return SSM_ERR_ALIGN;
  for (const void* q : {(const void*)a->dt, (const void*)a->A, (const void*)a->omega,
                        (const void*)a->beta, (const void*)a->gamma, (const void*)a->D})
    if (q && !aligned(q, 4)) return SSM_ERR_ALIGN;
  for (const void* q : {(const void*)a->saved, (const void*)a->h0, (const void*)a->h_final})
    if (q && !aligned(q, 16)) return SSM_ERR_ALIGN;

  FwdKey key = choose_fwd(d, pl);
  if (key.PB <= 0 || d->headdim % key.PB) return SSM_ERR_UNSUPPORTED;
  const int pb = key.PB;
  ssm::FwdParams p{};
  p.x = a->x; p.B = a->B; p.C = a->C; p.dt = a->dt; p.A = a->A; p.omega = a->omega;
  p.beta = a->beta; p.gamma = a->gamma; p.D = a->D; p.y = a->y; p.saved = a->saved;
  p.h0 = a->h0; p.h_final = a->h_final; p.x_prev = a->x_prev; p.B_prev = a->B_prev;
  p.batch = d->batch; p.L = d->seqlen; p.H = d->nheads; p.G = d->ngroups; p.P = d->headdim;
  p.n_real = d->n_real; p.n_pairs = d->n_pairs; p.nchunks = pl.nchunks;
  p.n_static = d->n_static;
  p.save_chunk = pl.QT;
  p.save_nchunks = pl.nchunks;
  p.npblk = d->headdim / pb;
  p.rin = d->rank_in;
  p.rout = d->rank_out;
  p.softplus = (d->flags & SSM_F_DT_SOFTPLUS) ? 1 : 0;
  p.has_D = hasD ? 1 : 0;
  p.head_rates = pl.head_rates ? 1 : 0;
  const Segs sg = segments((long)d->batch * d->nheads * p.npblk, pl.nchunks);
  p.nseg = sg.nseg;
  p.cps = sg.cps;
  // A two-endpoint forward may walk two chunks per step: the shift identity keeps a double
  // chunk's keys within the plan chunk's tiles; segment boundaries stay where they are (an
  // even number of chunks per segment).  Saved states still follow the plan's chunk: with
  // per-row decay and an even rank, the double-chunk kernel also saves the state after each
  // double chunk's first half; otherwise a forward that saves states keeps the plan's chunk.
  const bool half_save = pl.coord_kernel && (pl.QT * pl.R) % 32 == 0;
  if ((!a->saved || half_save) && (d->flags & SSM_F_TWO_ENDPOINT) &&
      (sg.nseg == 1 || sg.cps % 2 == 0) && env_int("SSM_FWD_SINGLE", 0) == 0) {
    FwdKey k2 = key;
    k2.QT = 2 * pl.QT;
    if (ssm::fwd_variant_exists(k2)) {
      key = k2;
      p.nchunks = (d->seqlen + k2.QT - 1) / k2.QT;
      p.cps = sg.nseg == 1 ? p.nchunks : sg.cps / 2;
    }
  }
  const size_t need = fwd_workspace(d, pl, key);
  if (need > 0) {
    if (use_scratch) {
      if (need > kScratchBytes) return SSM_ERR_SCRATCH;
      const int src = scratch_address(&ws);
      if (src != SSM_OK) return src;
      ws_bytes = kScratchBytes;
    }
    if (!ws || ws_bytes < need) return SSM_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return SSM_ERR_ALIGN;
    if (pl.coord_kernel)
      p.wild = reinterpret_cast<int*>(static_cast<char*>(ws) + align256(fwd_segment_bytes(d, pl, key)));
  }
  if (sg.nseg > 1) {
    const LocalRanges lr = local_ranges(pl, sg);
    p.seg_tokens = lr.seg_tokens;
    p.nsub = lr.nsub;
    p.lsub = lr.lsub;
    const size_t slices = (size_t)d->batch * d->nheads, np = (size_t)d->dstate * d->headdim;
    p.seg_local = static_cast<float*>(ws);
    p.seg_in = p.seg_local + slices * (sg.nseg - 1) * lr.nsub * np;
    p.seg_delta = p.seg_in + slices * sg.nseg * np;
  }
  const hipError_t e = ssm::launch_fwd(key, p, static_cast<hipStream_t>(stream), a->events);
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace

extern "C" {

int ssm_scan_fwd(const ssm_desc* d, const ssm_fwd_args* a, void* ws, size_t ws_bytes,
                 void* stream) {
  return scan_fwd_impl(d, a, ws, ws_bytes, stream, false);
}

size_t ssm_scratch_bytes(void) { return kScratchBytes; }

int ssm_scan_fwd_noalloc(const ssm_desc* d, const ssm_fwd_args* a, void* stream) {
  return scan_fwd_impl(d, a, nullptr, 0, stream, true);
}

int ssm_scan_bwd(const ssm_desc* d, const ssm_bwd_args* a, void* ws, size_t ws_bytes,
                 void* stream) {
  Plan pl;
  int rc = make_plan(d, &pl);
  if (rc) return rc;
  if (!a) return SSM_ERR_NULL;
  BwdKey key{pl.bf16, d->dstate, d->headdim, pl.R, pl.KR, pl.QT, pl.coord_kernel,
             d->rank_in != d->rank_out};
  if (!ssm::bwd_variant_exists(key)) return SSM_ERR_UNSUPPORTED;
  if (d->batch == 0 || d->seqlen == 0) {
    // no tokens: the parameter gradients are sums over nothing, and no output depends on h0
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t na = (size_t)d->nheads * (pl.head_rates ? 1 : d->n_real + d->n_pairs);
    hipError_t e = copy_or_zero(a->dA, nullptr, na, s);
    if (e == hipSuccess) e = copy_or_zero(a->domega, nullptr, (size_t)d->nheads * d->n_pairs, s);
    if (e == hipSuccess) e = copy_or_zero(a->dD, nullptr, (size_t)d->nheads, s);
    // with no tokens h_final is h0, so dh0 is the final state's gradient; the carried
    // token writes nothing, so its gradients are zero
    if (e == hipSuccess) e = copy_or_zero(a->dh0, d->seqlen == 0 ? a->dh_final : nullptr, state_floats(d), s);
    const size_t io = pl.bf16 ? 2 : 4;
    if (e == hipSuccess)
      e = zero_bytes(a->dx_prev, (size_t)d->batch * d->nheads * d->rank_in * d->headdim * io, s);
    if (e == hipSuccess)
      e = zero_bytes(a->dB_prev, (size_t)d->batch * d->ngroups * d->rank_in * d->dstate * io, s);
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
  }
  const bool te = (d->flags & SSM_F_TWO_ENDPOINT) != 0;
  const bool hasD = (d->flags & SSM_F_HAS_D) != 0;
  if (!a->x || !a->B || !a->C || !a->dy || !a->dt || !a->A || !a->saved || !a->dx || !a->dB ||
      !a->dC || !a->ddt)
    return SSM_ERR_NULL;
  if ((d->n_pairs > 0) != (a->omega != nullptr)) return SSM_ERR_NULL;
  if (te != (a->beta != nullptr) || te != (a->gamma != nullptr)) return SSM_ERR_NULL;
  if (hasD != (a->D != nullptr)) return SSM_ERR_NULL;
  if (!te && (a->dbeta || a->dgamma)) return SSM_ERR_NULL;
  if (d->n_pairs == 0 && a->domega) return SSM_ERR_NULL;
  if (!hasD && a->dD) return SSM_ERR_NULL;
  if ((a->x_prev != nullptr) != (a->B_prev != nullptr) || (a->x_prev && !te)) return SSM_ERR_NULL;
  if ((a->dx_prev || a->dB_prev) && !a->x_prev) return SSM_ERR_NULL;
  for (const void* q : {a->x, a->B, a->C, a->dy, (const void*)a->dx, (const void*)a->dB,
                        (const void*)a->dC, (const void*)a->saved, (const void*)ws, a->x_prev,
                        a->B_prev, (const void*)a->dh_final, (const void*)a->dx_prev,
                        (const void*)a->dB_prev})
    if (q && !aligned(q, 16)) return SSM_ERR_ALIGN;
  for (const void* q : {(const void*)a->dt, (const void*)a->A, (const void*)a->omega,
                        (const void*)a->beta, (const void*)a->gamma, (const void*)a->D,
                        (const void*)a->ddt, (const void*)a->dA, (const void*)a->domega,
                        (const void*)a->dbeta, (const void*)a->dgamma, (const void*)a->dD})
    if (q && !aligned(q, 4)) return SSM_ERR_ALIGN;
  if (a->dh0 && !aligned(a->dh0, 16)) return SSM_ERR_ALIGN;
  const size_t need = ssm_workspace_bytes(d, 1);
  if (!ws || ws_bytes < need) return SSM_ERR_WORKSPACE;

  ssm::BwdParams p{};
  p.x = a->x; p.B = a->B; p.C = a->C; p.dy = a->dy; p.dt = a->dt; p.A = a->A;
  p.omega = a->omega; p.beta = a->beta; p.gamma = a->gamma; p.D = a->D; p.saved = a->saved;
  p.dx = a->dx; p.dB = a->dB; p.dC = a->dC; p.ddt = a->ddt; p.dbeta = a->dbeta;
  p.dgamma = a->dgamma; p.dA = a->dA; p.domega = a->domega; p.dD = a->dD; p.dh0 = a->dh0;
  p.x_prev = a->x_prev; p.B_prev = a->B_prev; p.dh_final = a->dh_final;
  p.dx_prev = a->dx_prev; p.dB_prev = a->dB_prev;
  p.gseg = ws;
  p.part = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                    (bwd_gseg_bytes(d, pl) + 255) / 256 * 256);
  p.batch = d->batch; p.L = d->seqlen; p.H = d->nheads; p.G = d->ngroups; p.P = d->headdim;
  p.n_real = d->n_real; p.n_pairs = d->n_pairs; p.nchunks = pl.nchunks;
  p.n_static = d->n_static;
  p.rin = d->rank_in; p.rout = d->rank_out;
  const Segs sg = adj_segments(d, pl);
  p.nseg = sg.nseg;
  p.chunks_per_seg = sg.cps;
  if (sg.nseg > 1) {
    const size_t part = (size_t)d->batch * d->nheads * pl.nchunks * npart_of(d, pl) * sizeof(float);
    char* base = reinterpret_cast<char*>(p.part) + (part + 255) / 256 * 256;
    const LocalRanges lr = local_ranges(pl, sg);
    p.seg_tokens = lr.seg_tokens;
    p.nsub = lr.nsub;
    p.lsub = lr.lsub;
    const size_t slices = (size_t)d->batch * d->nheads, np = (size_t)d->dstate * d->headdim;
    p.gloc = reinterpret_cast<float*>(base);
    p.gin = p.gloc + slices * (sg.nseg - 1) * lr.nsub * np;
    p.gdel = p.gin + slices * sg.nseg * np;
  }
  if (pl.coord_kernel) {  // item flags and the "any flagged" word at the end of the workspace
    p.wild = reinterpret_cast<int*>(static_cast<char*>(ws) + (need - bwd_flags_bytes(d, pl)));
    p.wild_any = p.wild + (size_t)d->batch * d->nheads * pl.nchunks;
  }
  if (d->ngroups != d->nheads) {
    // per-head dB / dC partials before the flags
    char* base = static_cast<char*>(ws) + (need - bwd_flags_bytes(d, pl) - group_partial_bytes(d, pl));
    p.dBh = base;
    p.dCh = base + group_partial_one(d, pl);
  }
  p.softplus = (d->flags & SSM_F_DT_SOFTPLUS) ? 1 : 0;
  p.has_D = hasD ? 1 : 0;
  p.npart = npart_of(d, pl);
  p.head_rates = pl.head_rates ? 1 : 0;
  p.chunk_grid_cap = env_int("SSM_BWD_CHUNK_GRID", 0);
  const hipError_t e = ssm::launch_bwd(key, p, static_cast<hipStream_t>(stream), a->events);
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int ssm_decode_step(const ssm_desc* d, const ssm_decode_args* a, void* stream) {
  int rc = check_operation(d);
  if (rc) return rc;
  if (!a) return SSM_ERR_NULL;
  if (d->seqlen != 1) return SSM_ERR_SHAPE;
  if (d->rank_in > ssm::kDecodeMaxRank || d->rank_out > ssm::kDecodeMaxRank ||
      d->headdim % 4 || d->headdim > 1024 || (d->n_real % 2) || (d->n_static % 2))
    return SSM_ERR_UNSUPPORTED;
  if ((double)d->batch * d->nheads * d->dstate * d->headdim >= 2147483648.0)
    return SSM_ERR_UNSUPPORTED;
  const int tps = env_int("SSM_DECODE_TPS", 0) > 0 ? env_int("SSM_DECODE_TPS", 0)
                                                   : ssm::decode_tps(d->dstate, d->headdim);
  if (tps != 64 && tps != 128 && tps != 256) return SSM_ERR_UNSUPPORTED;
  if (d->headdim / 4 > tps) return SSM_ERR_UNSUPPORTED;
  if ((long)(256 / tps) * ssm::decode_lds_floats(d->dstate, d->rank_in, d->rank_out, d->headdim, tps) * 4 >
      ssm::kDecodeMaxLdsBytes)
    return SSM_ERR_UNSUPPORTED;
  if (d->batch == 0) return SSM_OK;
  const bool te = (d->flags & SSM_F_TWO_ENDPOINT) != 0;
  const bool hasD = (d->flags & SSM_F_HAS_D) != 0;
  if (!a->x || !a->B || !a->C || !a->dt || !a->A || !a->state || !a->y) return SSM_ERR_NULL;
  if ((d->n_pairs > 0) != (a->omega != nullptr)) return SSM_ERR_NULL;
  if (te != (a->beta != nullptr) || te != (a->gamma != nullptr)) return SSM_ERR_NULL;
  if (hasD != (a->D != nullptr)) return SSM_ERR_NULL;
  if ((a->x_prev != nullptr) != (a->B_prev != nullptr)) return SSM_ERR_NULL;
  if (!te && a->x_prev) return SSM_ERR_NULL;
  for (const void* q : {a->x, a->B, a->C, (const void*)a->y, a->x_prev, a->B_prev,
                        (const void*)a->state})
    if (q && !aligned(q, 16)) return SSM_ERR_ALIGN;
  for (const void* q : {(const void*)a->dt, (const void*)a->A, (const void*)a->omega,
                        (const void*)a->beta, (const void*)a->gamma, (const void*)a->D})
    if (q && !aligned(q, 4)) return SSM_ERR_ALIGN;
  ssm::DecodeParams p{};
  p.x = a->x; p.B = a->B; p.C = a->C; p.dt = a->dt; p.A = a->A; p.omega = a->omega;
  p.beta = a->beta; p.gamma = a->gamma; p.D = a->D; p.x_prev = a->x_prev; p.B_prev = a->B_prev;
  p.state = a->state; p.y = a->y;
  p.batch = d->batch; p.H = d->nheads; p.G = d->ngroups; p.P = d->headdim;
  p.R = d->rank_in; p.O = d->rank_out; p.n_real = d->n_real; p.n_pairs = d->n_pairs;
  p.n_static = d->n_static;
  p.softplus = (d->flags & SSM_F_DT_SOFTPLUS) ? 1 : 0;
  p.head_rates = d->decay_mode == SSM_DECAY_HEAD ? 1 : 0;
  p.tps = tps;
  const hipError_t e =
      ssm::launch_decode(d->io_dtype == SSM_BF16, p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // extern "C"
