// kata.hip - libkata: host side of the C ABI declared in include/kata.h.
//
// Validates arguments on the host (nothing is enqueued on error), sizes the
// workspace, selects the kernel instance for (input dtype, output dtype, chunk,
// head dims) and enqueues the chunked forward as three stream-ordered launches:
//   kata_chunk_state -> kata_state_scan -> kata_chunk_intra
// (the chunked-state form with an associative inter-chunk scan described in the
// gist.science summary of "Kernelized Linear Attention", arXiv 2607.17419,
// section 2.3, and in the paper's abstract).
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/kata.h"
#include "kata_bwd.h"
#include "kata_chunk.h"
#include "kata_decode.h"
#include "kata_delta.h"
#include "kata_flash.h"
#include "kata_scan.h"

using namespace kata;

namespace {

struct Plan {
  int64_t n_chunks = 0;
  int64_t leaf = 1;        // chunks per leaf
  int64_t n_leaf = 0;
  bool direct = false;     // plain forward: no scan, the intra pass sums the earlier leaves
  int E = 0;               // floats per leaf state block
  size_t ws_bytes = 0;
};

// The enum arguments come from C callers, who may pass any int.  Loading an out-of-range
// value as the C++ enum type is undefined, so arguments are validated from their bits
// (read as an int, never as the enum) before any other use.
template <typename E>
int bits(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized here");
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

kata_status check_dtype(const kata_dtype& t) {
  const int v = bits(t);
  return (v == KATA_F32 || v == KATA_BF16) ? KATA_OK : KATA_ERR_UNSUPPORTED;
}

bool valid_mode(const kata_factor_mode& m) {
  const int v = bits(m);
  return v == KATA_FACTORS_CONCAT || v == KATA_FACTORS_SUM;
}

kata_status validate(const kata_forward_desc* d) {
  if (!d) return KATA_ERR_NULL;
  if (d->B < 0 || d->H < 0 || d->T < 0 || d->d <= 0 || d->dv <= 0 || d->p <= 0 || d->chunk <= 0 ||
      d->scan_leaf < 0)
    return KATA_ERR_SHAPE;
  if (d->B > 65535 || d->H > 65535 || d->B * d->H > 65535) return KATA_ERR_SHAPE;
  // a sequence of q, k, v or y is addressed with 32-bit byte offsets (< 2 GiB)
  const int64_t widest = (int64_t)(d->d > d->dv ? d->d : d->dv) * 4;
  if (d->T > (((int64_t)1 << 31) - 4096) / widest - 256) return KATA_ERR_SHAPE;
  if (d->p != P_DIM) return KATA_ERR_UNSUPPORTED;
  if (!((d->d == 16 && d->dv == 16) || (d->d == 64 && d->dv == 64))) return KATA_ERR_UNSUPPORTED;
  if (!(d->chunk == 32 || d->chunk == 64 || d->chunk == 128)) return KATA_ERR_UNSUPPORTED;
  if ((check_dtype(d->in_dtype) != KATA_OK && bits(d->in_dtype) != KATA_BF16_HILO) ||
      check_dtype(d->out_dtype) != KATA_OK)
    return KATA_ERR_UNSUPPORTED;
  if (bits(d->scan) != KATA_SCAN_ASSOC && bits(d->scan) != KATA_SCAN_SEQUENTIAL) return KATA_ERR_UNSUPPORTED;
  return KATA_OK;
}

// Concurrent workgroups of kata_chunk_intra on one MI355X (256 compute units): the
// instance's waves per SIMD (one 4-wave workgroup per SIMD set) limited by its LDS.
// The LDS that co-resident workgroups can share is taken as 156 KiB: measured on
// MI355X, three 256-thread workgroups of 52 KiB start together but three of 53 KiB
// do not (the occupancy query of the runtime still reports three for 53 KiB).
constexpr int64_t kComputeUnits = 256;
constexpr int64_t kLdsPerCU = 156 * 1024;

template <int C, int DV, bool SPLIT, bool PREC = false>
int64_t intra_slots() {
  using S = Shape<C, DV, DV, SPLIT, PREC>;
  const int64_t by_lds = kLdsPerCU / S::SMEM;
  const int64_t per_cu = by_lds < S::OCC_INTRA ? by_lds : S::OCC_INTRA;
  return kComputeUnits * (per_cu < 1 ? 1 : per_cu);
}

int64_t slots_for(const kata_forward_desc* d) {
  const bool split = d->in_dtype == KATA_F32;
  if (d->in_dtype == KATA_BF16_HILO) {
    if (d->dv == 16)
      return d->chunk == 32 ? intra_slots<32, 16, false, true>()
                            : (d->chunk == 64 ? intra_slots<64, 16, false, true>() : intra_slots<128, 16, false, true>());
    return d->chunk == 32 ? intra_slots<32, 64, false, true>()
                          : (d->chunk == 64 ? intra_slots<64, 64, false, true>() : intra_slots<128, 64, false, true>());
  }
  if (d->dv == 16) {
    if (d->chunk == 32) return split ? intra_slots<32, 16, true>() : intra_slots<32, 16, false>();
    if (d->chunk == 64) return split ? intra_slots<64, 16, true>() : intra_slots<64, 16, false>();
    return split ? intra_slots<128, 16, true>() : intra_slots<128, 16, false>();
  }
  if (d->chunk == 32) return split ? intra_slots<32, 64, true>() : intra_slots<32, 64, false>();
  if (d->chunk == 64) return split ? intra_slots<64, 64, true>() : intra_slots<64, 64, false>();
  return split ? intra_slots<128, 64, true>() : intra_slots<128, 64, false>();
}

// Leaf size: SEQUENTIAL = the whole sequence; ASSOC = the caller's value, else the
// smallest number of leaves that fills the concurrent workgroup slots of the intra
// kernel in whole rounds (leaves of at most kMaxLeaf chunks), so no round runs
// partly empty and the scanned state tensor stays small.  Where the leaf states would
// then move more than a quarter of the bytes of the tokens (every leaf state is written,
// scanned and read back: four passes of 37.9 KB at dv = 64), as for many short sequences,
// the plan fills one workgroup fewer per compute unit: on the 340M-layer shape (B=8, H=16,
// T=2048) 4 leaves of 8 chunks per sequence took 64.5 us per step against 71.7 us for
// 6 leaves of 5-6 chunks, on the mid shape (B=4, H=8, T=4096) 16 leaves of 4 chunks
// 40.0 us against 42.7 us for 22 leaves of 3, while the long shape (the states 11% of the
// token bytes) keeps its plan.  The choice depends only on the descriptor, so the
// workspace size is reproducible.
constexpr int64_t kMaxLeaf = 64;
constexpr int64_t kDirectMaxLeaves = 8;

int64_t leaf_for_slots(int64_t n_chunks, int64_t bh, int64_t slots) {
  const int64_t units = bh * n_chunks;
  int64_t rounds = (units + slots * kMaxLeaf - 1) / (slots * kMaxLeaf);
  if (rounds < 1) rounds = 1;
  const int64_t leaves_per_bh = (rounds * slots + bh - 1) / bh;      // want >= this many
  int64_t leaf = (n_chunks + leaves_per_bh - 1) / leaves_per_bh;
  if (leaf < 1) leaf = 1;
  if (leaf > n_chunks) leaf = n_chunks;
  // fewer leaves than slots per round would idle compute units: shrink the leaf
  while (leaf > 1 && bh * ((n_chunks + leaf - 1) / leaf) < rounds * slots &&
         bh * ((n_chunks + leaf - 2) / (leaf - 1)) <= rounds * slots)
    --leaf;
  return leaf;
}

Plan make_plan(const kata_forward_desc* d, int64_t slots) {
  Plan p;
  p.n_chunks = (d->T + d->chunk - 1) / d->chunk;
  p.E = DPACK * d->dv + P_DIM * P_DIM;
  const int64_t bh = d->B * d->H;
  if (p.n_chunks == 0 || bh == 0) {
    p.leaf = 1;
  } else if (d->scan == KATA_SCAN_SEQUENTIAL) {
    p.leaf = p.n_chunks;
  } else if (d->scan_leaf > 0) {
    p.leaf = d->scan_leaf < p.n_chunks ? d->scan_leaf : p.n_chunks;
  } else {
    p.leaf = leaf_for_slots(p.n_chunks, bh, slots);
    const int64_t per_cu = slots / kComputeUnits;
    if (per_cu >= 3) {
      const int in_bytes = bits(d->in_dtype) == KATA_F32 ? 4 : 2, out_bytes = bits(d->out_dtype) == KATA_F32 ? 4 : 2;
      const double tokens = (double)bh * (double)d->T * ((2.0 * d->d + d->dv) * in_bytes + d->dv * out_bytes);
      const double states = 4.0 * (double)bh * (double)((p.n_chunks + p.leaf - 1) / p.leaf) * p.E * sizeof(float);
      if (states > 0.25 * tokens) p.leaf = leaf_for_slots(p.n_chunks, bh, kComputeUnits * (per_cu - 1));
    }
  }
  p.n_leaf = p.n_chunks == 0 ? 0 : (p.n_chunks + p.leaf - 1) / p.leaf;
  p.ws_bytes = (size_t)bh * (size_t)p.n_leaf * (size_t)p.E * sizeof(float);
  // With few leaves per sequence (many short sequences) a separate scan costs more than
  // it saves: the intra pass's workgroup of leaf g adds the states of leaves 0 .. g-1 itself
  // (at most kDirectMaxLeaves - 1 blocks of 37.9 KB, read from the caches they were just
  // written to) and the last one exports the final state.  Only for the plan the library
  // picks, so a caller's explicit scan_leaf keeps the scanned workspace.
  p.direct = d->scan == KATA_SCAN_ASSOC && d->scan_leaf == 0 && p.n_leaf > 0 && p.n_leaf <= kDirectMaxLeaves;
  return p;
}

Plan make_plan(const kata_forward_desc* d) { return make_plan(d, slots_for(d)); }

kata_status launch_status() {
  return hipGetLastError() == hipSuccess ? KATA_OK : KATA_ERR_LAUNCH;
}

// ---- the scratch buffer of kata_forward_noalloc -------------------------------------
// A file-scope device array: every GPU the library runs on holds its own copy, at its
// own address, until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory, so kernels get the address hipGetSymbolAddress returns for the
// current device, looked up once per device and kept.
__device__ __align__(256) unsigned char scratch[KATA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, or nullptr on failure.
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// Kernels whose LDS footprint exceeds the default 64 KiB dynamic limit need the
// per-function attribute raised (gfx950 has 160 KiB of LDS per compute unit).
template <typename F>
kata_status allow_smem(F* fn, int bytes) {
  if (bytes <= 65536) return KATA_OK;
  return hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess
             ? KATA_OK
             : KATA_ERR_LAUNCH;
}

__global__ void kata_copy_or_zero(float* __restrict__ dst, const float* __restrict__ src, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.f;
}

// dst = the symmetric part of a state (or of a state gradient) src [n_blocks, p*p, cols]:
// entry (i, j, c) is the mean of src's entries (i, j, c) and (j, i, c), 0 when src is NULL.
// A symmetric src is copied bit for bit (0.5 * (x + x) = x).  This is how every entry point
// reads a caller's state, so the state exported for zero tokens is the one a token is
// added to.
__global__ void kata_sym_copy_or_zero(float* __restrict__ dst, const float* __restrict__ src, int64_t n, int cols) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  if (!src) {
    dst[e] = 0.f;
    return;
  }
  const int c = (int)(e % cols);
  const int64_t f = e / cols;
  const int64_t blk = f / (P_DIM * P_DIM);
  const int ij = (int)(f % (P_DIM * P_DIM));
  const int i = ij / P_DIM, j = ij % P_DIM;
  dst[e] = 0.5f * (src[e] + src[((blk * P_DIM + j) * P_DIM + i) * cols + c]);
}

// segments per column quad of kata_state_scan: the smallest power of two with at most
// SCAN_ROWS leaf rows each, capped at SCAN_GMAX (more leaves take several passes)
int scan_segments(const Plan& pl) {
  int G = 1;
  while (G < SCAN_GMAX && (int64_t)G * SCAN_ROWS < pl.n_leaf) G *= 2;
  return G;
}
dim3 scan_grid(const Plan& pl, int G, int64_t bh) {
  const int quads = (int)(pl.E / 4);
  return dim3((unsigned)((quads + 256 / G - 1) / (256 / G)), (unsigned)bh);
}

// DECAY: lam [B,H,T] log-decays; dec (B*H*n_leaf floats) receives the leaf decays.
template <class S, typename TIn, typename TOut, bool DECAY = false>
kata_status run_forward(const kata_forward_desc* d, const Plan& pl, const void* q, const void* k,
                        const void* v, const float* P, const float* S0, const float* z0, void* y,
                        float* ST, float* zT, float* ws, hipStream_t st, hipEvent_t* ev,
                        const float* lam = nullptr, float* dec = nullptr) {
  const int64_t bh = d->B * d->H;
  constexpr int smem_state = S::SMEM_STATE + (DECAY ? S::DEC_BYTES : 0);
  constexpr int smem_intra = S::SMEM + (DECAY ? S::DEC_BYTES : 0);
  if (allow_smem(kata_chunk_state<S, TIn, DECAY>, smem_state) != KATA_OK ||
      allow_smem(kata_chunk_intra<S, TIn, TOut, DECAY>, smem_intra) != KATA_OK)
    return KATA_ERR_LAUNCH;
  const dim3 grid((unsigned)pl.n_leaf, (unsigned)bh);
  // With events, the launches themselves stamp them (hipExtLaunchKernel: start of
  // each kernel, end of the last), so timing adds no commands to the stream.
  hipEvent_t e0 = ev ? ev[0] : nullptr, e1 = ev ? ev[1] : nullptr;
  hipEvent_t e2 = ev ? ev[2] : nullptr, e3 = ev ? ev[3] : nullptr;
  const bool direct = pl.direct && !DECAY;
  // direct: no scan; events[1] is stamped by the state pass's end instead of the scan's start
  hipExtLaunchKernelGGL((kata_chunk_state<S, TIn, DECAY>), grid, dim3(256), smem_state, st, e0, direct ? e1 : nullptr,
                        0, (const TIn*)k, (const TIn*)v, P, ws, d->T, (int)d->H, pl.leaf * S::C, lam, dec);
  if (launch_status() != KATA_OK) return KATA_ERR_LAUNCH;
  if (!direct) {
    const int G = scan_segments(pl);
    const dim3 sgrid = scan_grid(pl, G, bh);
    hipExtLaunchKernelGGL(kata_state_scan, sgrid, dim3(256), 0, st, e1, nullptr, 0, ws, pl.n_leaf, (int)pl.E,
                          (int)S::DV, G, S0, z0, ST, zT, 0, (const float*)dec);
    if (launch_status() != KATA_OK) return KATA_ERR_LAUNCH;
  }
  hipExtLaunchKernelGGL((kata_chunk_intra<S, TIn, TOut, DECAY>), grid, dim3(256), smem_intra, st, e2, e3, 0,
                        (const TIn*)q, (const TIn*)k, (const TIn*)v, P, (const float*)ws, (TOut*)y, d->T,
                        (int)d->H, (int)pl.leaf, pl.n_chunks, lam, direct ? 1 : 0, direct ? S0 : nullptr,
                        direct ? z0 : nullptr, direct ? ST : nullptr, direct ? zT : nullptr);
  if (launch_status() != KATA_OK) return KATA_ERR_LAUNCH;
  return KATA_OK;
}

template <int C, int DIN, int DV>
kata_status dispatch_dtypes(const kata_forward_desc* d, const Plan& pl, const void* q, const void* k,
                            const void* v, const float* P, const float* S0, const float* z0, void* y,
                            float* ST, float* zT, float* ws, hipStream_t st, hipEvent_t* ev) {
  if (d->in_dtype == KATA_F32) {
    using S = Shape<C, DIN, DV, true>;
    if (d->out_dtype == KATA_F32) return run_forward<S, float, float>(d, pl, q, k, v, P, S0, z0, y, ST, zT, ws, st, ev);
    return run_forward<S, float, bf16>(d, pl, q, k, v, P, S0, z0, y, ST, zT, ws, st, ev);
  }
  if (d->in_dtype == KATA_BF16_HILO) {
    using SP = Shape<C, DIN, DV, false, true>;
    if (d->out_dtype == KATA_F32) return run_forward<SP, bf16, float>(d, pl, q, k, v, P, S0, z0, y, ST, zT, ws, st, ev);
    return run_forward<SP, bf16, bf16>(d, pl, q, k, v, P, S0, z0, y, ST, zT, ws, st, ev);
  }
  using S = Shape<C, DIN, DV, false>;
  if (d->out_dtype == KATA_F32) return run_forward<S, bf16, float>(d, pl, q, k, v, P, S0, z0, y, ST, zT, ws, st, ev);
  return run_forward<S, bf16, bf16>(d, pl, q, k, v, P, S0, z0, y, ST, zT, ws, st, ev);
}

template <int C>
kata_status dispatch_dims(const kata_forward_desc* d, const Plan& pl, const void* q, const void* k,
                          const void* v, const float* P, const float* S0, const float* z0, void* y,
                          float* ST, float* zT, float* ws, hipStream_t st, hipEvent_t* ev) {
  if (d->d == 16) return dispatch_dtypes<C, 16, 16>(d, pl, q, k, v, P, S0, z0, y, ST, zT, ws, st, ev);
  return dispatch_dtypes<C, 64, 64>(d, pl, q, k, v, P, S0, z0, y, ST, zT, ws, st, ev);
}

// The state export when there are no tokens: ST, zT = the symmetric part of S0, z0 (or 0),
// the state as every entry point reads it.
kata_status copy_initial_state(const kata_forward_desc* d, const float* S0, const float* z0, float* ST,
                               float* zT, hipStream_t st) {
  const int64_t nS = d->B * d->H * P_DIM * P_DIM * d->dv;
  const int64_t nz = d->B * d->H * P_DIM * P_DIM;
  if (ST) {
    hipLaunchKernelGGL(kata_sym_copy_or_zero, dim3((unsigned)((nS + 255) / 256)), dim3(256), 0, st, ST, S0, nS,
                       d->dv);
    hipLaunchKernelGGL(kata_sym_copy_or_zero, dim3((unsigned)((nz + 255) / 256)), dim3(256), 0, st, zT, z0, nz, 1);
  }
  return launch_status();
}

// The flash-style forward supports bf16 q/k/v with d = dv = 64 and p = 16.
kata_status validate_flash(const kata_forward_desc* d) {
  if (!d) return KATA_ERR_NULL;
  if (d->B < 0 || d->H < 0 || d->T < 0 || d->d <= 0 || d->dv <= 0 || d->p <= 0) return KATA_ERR_SHAPE;
  if (d->B > 65535 || d->H > 65535 || d->B * d->H > 65535) return KATA_ERR_SHAPE;
  // a sequence's workspace (flash_ws_elems bf16 per padded token) and its y rows are
  // addressed with 32-bit byte offsets
  const int64_t per_tok = (int64_t)(4 * P_DIM + FL_DV) * 2 > FL_DV * 4 ? (4 * P_DIM + FL_DV) * 2 : FL_DV * 4;
  if (d->T > (((int64_t)1 << 31) - 4096) / per_tok - 256) return KATA_ERR_SHAPE;
  if (d->p != P_DIM || d->d != 64 || d->dv != FL_DV) return KATA_ERR_UNSUPPORTED;
  if (d->in_dtype != KATA_BF16 || check_dtype(d->out_dtype) != KATA_OK) return KATA_ERR_UNSUPPORTED;
  return KATA_OK;
}

int64_t flash_tpad(int64_t T) { return (T + FL_QB - 1) / FL_QB * FL_QB; }

size_t flash_ws_bytes(const kata_forward_desc* d) {
  return (size_t)(d->B * d->H) * (size_t)flash_ws_elems(flash_tpad(d->T)) * sizeof(bf16);
}

// ---- backward ----------------------------------------------------------------------
// Supported: p = 16, d = dv = 64, chunk 64, bf16 q/k/v (and dq/dk/dv), y and gy in
// out_dtype.  Concurrent workgroup slots for the leaf plan: two kata_bwd_query
// workgroups per compute unit (kata_bwd_key, at one 8-wave workgroup per compute unit,
// then runs the same leaves in two rounds).
constexpr int64_t kBwdSlots = kComputeUnits * 2;

kata_status validate_bwd(const kata_forward_desc* d) {
  const kata_status s = validate(d);
  if (s != KATA_OK) return s;
  if (d->d != 64 || d->dv != 64 || d->chunk != 64 || d->in_dtype != KATA_BF16) return KATA_ERR_UNSUPPORTED;
  return KATA_OK;
}

struct BwdLayout {
  Plan pl;
  size_t off_wsr = 0, off_ih = 0, off_dpa = 0, off_dpb = 0, total = 0;
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace of the backward: the forward's leaf prefix states, the backward's leaf
// suffix states, (1/den_t, h_t) per token, and the dP partials of the two chunk walks
// (one 16 x 64 block per workgroup).
BwdLayout bwd_layout(const kata_forward_desc* d) {
  BwdLayout L;
  L.pl = make_plan(d, kBwdSlots);
  const size_t bh = (size_t)(d->B * d->H);
  const size_t tok = bh * (size_t)d->T;
  const size_t st = bh * (size_t)L.pl.n_leaf * (size_t)L.pl.E * sizeof(float);
  const size_t dp = bh * (size_t)L.pl.n_leaf * (size_t)BW_DP * sizeof(float);
  L.off_wsr = align256(st);
  L.off_ih = L.off_wsr + align256(st);
  L.off_dpa = L.off_ih + align256(tok * 8);
  L.off_dpb = L.off_dpa + align256(dp);
  L.total = L.off_dpb + align256(dp);
  return L;
}

template <typename TY>
kata_status run_backward(const kata_forward_desc* d, const BwdLayout& L, const void* q, const void* k,
                         const void* v, const float* P, const float* S0, const float* z0, const void* gy, const float* gST, const float* gzT, void* dq, void* dk, void* dv,
                         float* dP, float* dS0, float* dz0, unsigned char* wsb, hipStream_t st,
                         hipEvent_t* ev) {
  using S = BS;
  const Plan& pl = L.pl;
  const int64_t bh = d->B * d->H;
  if (allow_smem(kata_chunk_state<S, bf16, false>, S::SMEM_STATE) != KATA_OK ||
      allow_smem(kata_bwd_query<TY>, QaGy<TY>::SMEM) != KATA_OK ||
      allow_smem(kata_bwd_rstate<TY>, RS_SMEM) != KATA_OK || allow_smem(kata_bwd_key<TY>, KB_SMEM) != KATA_OK)
    return KATA_ERR_LAUNCH;
  float* wsf = reinterpret_cast<float*>(wsb);
  float* wsr = reinterpret_cast<float*>(wsb + L.off_wsr);
  float* ih = reinterpret_cast<float*>(wsb + L.off_ih);
  float* dpa = reinterpret_cast<float*>(wsb + L.off_dpa);
  float* dpb = reinterpret_cast<float*>(wsb + L.off_dpb);
  hipEvent_t e[8];
  for (int i = 0; i < 8; ++i) e[i] = ev ? ev[i] : nullptr;
  const dim3 grid((unsigned)pl.n_leaf, (unsigned)bh);
  const int G = scan_segments(pl);
  const dim3 sgrid = scan_grid(pl, G, bh);
  const bf16* qb = (const bf16*)q;
  const bf16* kb = (const bf16*)k;
  const bf16* vb = (const bf16*)v;
  // forward prefix states at every leaf start
  hipExtLaunchKernelGGL((kata_chunk_state<S, bf16, false>), grid, dim3(256), S::SMEM_STATE, st, e[0], nullptr, 0, kb,
                        vb, P, wsf, d->T, (int)d->H, pl.leaf * S::C, (const float*)nullptr, (float*)nullptr);
  if (launch_status() != KATA_OK) return KATA_ERR_LAUNCH;
  hipExtLaunchKernelGGL(kata_state_scan, sgrid, dim3(256), 0, st, e[1], nullptr, 0, wsf, pl.n_leaf, (int)pl.E, 64, G,
                        S0, z0, (float*)nullptr, (float*)nullptr, 0, (const float*)nullptr);
  if (launch_status() != KATA_OK) return KATA_ERR_LAUNCH;
  hipExtLaunchKernelGGL((kata_bwd_query<TY>), grid, dim3(256), QaGy<TY>::SMEM, st, e[2], nullptr, 0, qb, kb, vb,
                        (const TY*)gy, P, (const float*)wsf, ih, (bf16*)dq, dpa, d->T,
                        (int)d->H, (int)pl.leaf, pl.n_chunks);
  if (launch_status() != KATA_OK) return KATA_ERR_LAUNCH;
  hipExtLaunchKernelGGL((kata_bwd_rstate<TY>), grid, dim3(256), RS_SMEM, st, e[3], nullptr, 0, qb, (const TY*)gy,
                        (const float*)ih, P, wsr, d->T, (int)d->H, (int)pl.leaf, pl.n_chunks);
  if (launch_status() != KATA_OK) return KATA_ERR_LAUNCH;
  hipExtLaunchKernelGGL(kata_state_scan, sgrid, dim3(256), 0, st, e[4], nullptr, 0, wsr, pl.n_leaf, (int)pl.E, 64, G,
                        gST, gzT, dS0, dz0, 1, (const float*)nullptr);
  if (launch_status() != KATA_OK) return KATA_ERR_LAUNCH;
  hipExtLaunchKernelGGL((kata_bwd_key<TY>), grid, dim3(512), KB_SMEM, st, e[5], nullptr, 0, qb, kb, vb, (const TY*)gy,
                        (const float*)ih, P, (const float*)wsr, (bf16*)dk, (bf16*)dv, dpb, d->T,
                        (int)d->H, (int)pl.leaf, pl.n_chunks);
  if (launch_status() != KATA_OK) return KATA_ERR_LAUNCH;
  hipExtLaunchKernelGGL(kata_bwd_dp_reduce, dim3((unsigned)d->H, 4), dim3(256), 0, st, e[6], e[7], 0,
                        (const float*)dpa, (const float*)dpb, dP, d->B, (int)d->H, pl.n_leaf);
  return launch_status();
}

// ---- decay-gated forward -----------------------------------------------------------
// Supported: p = 16, d = dv = 64, chunk 64, bf16 q/k/v, f32 or bf16 y (the plain forward's
// fast instance).  Workspace: the plain forward's, then one float per leaf (its decay).
kata_status validate_decay(const kata_forward_desc* d) {
  const kata_status s = validate(d);
  if (s != KATA_OK) return s;
  if (d->d != 64 || d->dv != 64 || d->chunk != 64 || d->in_dtype != KATA_BF16) return KATA_ERR_UNSUPPORTED;
  return KATA_OK;
}

size_t decay_ws_bytes(const Plan& pl, const kata_forward_desc* d) {
  return align256(pl.ws_bytes) + (size_t)(d->B * d->H) * (size_t)pl.n_leaf * sizeof(float);
}

// DeltaKATA token recurrence: one workgroup per (sequence, head), T tokens each.
// PACKED: the state in the packed symmetric layout (kata_decode_step_delta_packed)
template <bool PACKED = false>
kata_status launch_delta(int64_t BH, int64_t T, int H, int d, int dv, kata_dtype in_dtype, kata_dtype out_dtype,
                         const float* S0, float* ST, const void* q, const void* k, const void* v,
                         const float* beta, const float* P, void* y, hipStream_t st) {
  const dim3 grid((unsigned)BH);
#define KATA_DELTA(TI, TO, DVV)                                                                                      \
  hipLaunchKernelGGL((kata::kata_delta_recurrent<TI, TO, DVV, PACKED>), grid, dim3(256), 0, st, S0, ST, (const TI*)q, \
                     (const TI*)k, (const TI*)v, beta, P, (TO*)y, H, d, T)
  const bool fi = in_dtype == KATA_F32, fo = out_dtype == KATA_F32;
  if (dv == 64) {
    if (fi && fo) KATA_DELTA(float, float, 64);
    else if (fi) KATA_DELTA(float, bf16, 64);
    else if (fo) KATA_DELTA(bf16, float, 64);
    else KATA_DELTA(bf16, bf16, 64);
  } else {
    if (fi && fo) KATA_DELTA(float, float, 16);
    else if (fi) KATA_DELTA(float, bf16, 16);
    else if (fo) KATA_DELTA(bf16, float, 16);
    else KATA_DELTA(bf16, bf16, 16);
  }
#undef KATA_DELTA
  return launch_status();
}

// ---- KATA-Mg / KATA-Sigma-g (several PSD factors, concatenated or summed) ----------------
// Supported for g > 1: p = 16, d = dv = 64, chunk 64, bf16 q/k/v, f32 or bf16 y, g <= 3.
// g = 1 is one-factor KATA in both modes and runs the plain forward (P [H,1,p,d] is
// P [H,p,d]).  Workspace: CONCAT g times the one-factor leaf states, SUM the one-factor's.
constexpr int kMaxFactors = 3;

template <int SMEM>
int64_t slots_by_lds() {
  const int64_t by_lds = kLdsPerCU / SMEM;
  const int64_t per_cu = by_lds < 2 ? by_lds : 2;   // the factor kernels run at most 2 per CU
  return kComputeUnits * (per_cu < 1 ? 1 : per_cu);
}

kata_status validate_factors(const kata_forward_desc* d, int g, const kata_factor_mode& mode) {
  const kata_status s = validate(d);
  if (s != KATA_OK) return s;
  if (!valid_mode(mode)) return KATA_ERR_UNSUPPORTED;
  if (g < 1) return KATA_ERR_SHAPE;
  if (g == 1) return KATA_OK;
  if (g > kMaxFactors) return KATA_ERR_UNSUPPORTED;
  if (d->d != 64 || d->dv != 64 || d->chunk != 64 || d->in_dtype != KATA_BF16) return KATA_ERR_UNSUPPORTED;
  if (d->B * d->H * g > 65535) return KATA_ERR_SHAPE;
  return KATA_OK;
}

Plan factors_plan(const kata_forward_desc* d, int g, const kata_factor_mode& mode) {
  using S = Shape<64, 64, 64, false>;
  if (g <= 1) return make_plan(d);
  if (mode == KATA_FACTORS_SUM)
    return make_plan(d, g == 2 ? slots_by_lds<kata::SgLayout<S, 2>::SMEM>() : slots_by_lds<kata::SgLayout<S, 3>::SMEM>());
  Plan p = make_plan(d, g == 2 ? slots_by_lds<kata::MgLayout<S, 2>::SMEM>() : slots_by_lds<kata::MgLayout<S, 3>::SMEM>());
  p.ws_bytes *= (size_t)g;
  return p;
}

template <class S, typename TIn, typename TOut, int G>
kata_status run_forward_mg(const kata_forward_desc* d, const Plan& pl, const void* q, const void* k,
                           const void* v, const float* P, const float* S0, const float* z0, void* y,
                           float* ST, float* zT, float* ws, hipStream_t st, hipEvent_t* ev) {
  const int64_t bh = d->B * d->H;
  constexpr int smem_state = S::SMEM_STATE;
  constexpr int smem_intra = kata::MgLayout<S, G>::SMEM;
  if (allow_smem(kata_chunk_state<S, TIn, false, G>, smem_state) != KATA_OK ||
      allow_smem(kata_chunk_intra_mg<S, TIn, TOut, G>, smem_intra) != KATA_OK)
    return KATA_ERR_LAUNCH;
  hipEvent_t e0 = ev ? ev[0] : nullptr, e1 = ev ? ev[1] : nullptr;
  hipEvent_t e2 = ev ? ev[2] : nullptr, e3 = ev ? ev[3] : nullptr;
  hipExtLaunchKernelGGL((kata_chunk_state<S, TIn, false, G>), dim3((unsigned)pl.n_leaf, (unsigned)(bh * G)),
                        dim3(256), smem_state, st, e0, nullptr, 0, (const TIn*)k, (const TIn*)v, P, ws, d->T,
                        (int)d->H, pl.leaf * S::C, (const float*)nullptr, (float*)nullptr);
  if (launch_status() != KATA_OK) return KATA_ERR_LAUNCH;
  const int segs = scan_segments(pl);
  hipExtLaunchKernelGGL(kata_state_scan, scan_grid(pl, segs, bh * G), dim3(256), 0, st, e1, nullptr, 0, ws,
                        pl.n_leaf, (int)pl.E, (int)S::DV, segs, S0, z0, ST, zT, 0, (const float*)nullptr);
  if (launch_status() != KATA_OK) return KATA_ERR_LAUNCH;
  hipExtLaunchKernelGGL((kata_chunk_intra_mg<S, TIn, TOut, G>), dim3((unsigned)pl.n_leaf, (unsigned)bh), dim3(256),
                        smem_intra, st, e2, e3, 0, (const TIn*)q, (const TIn*)k, (const TIn*)v, P,
                        (const float*)ws, (TOut*)y, d->T, (int)d->H, (int)pl.leaf, pl.n_chunks);
  return launch_status();
}

template <class S, typename TIn, typename TOut, int G>
kata_status run_forward_sg(const kata_forward_desc* d, const Plan& pl, const void* q, const void* k,
                           const void* v, const float* P, const float* S0, const float* z0, void* y,
                           float* ST, float* zT, float* ws, hipStream_t st, hipEvent_t* ev) {
  const int64_t bh = d->B * d->H;
  constexpr int smem_state = kata::SgStateLayout<S, G>::SMEM;
  constexpr int smem_intra = kata::SgLayout<S, G>::SMEM;
  if (allow_smem(kata_chunk_state<S, TIn, false, G, true>, smem_state) != KATA_OK ||
      allow_smem(kata_chunk_intra_sg<S, TIn, TOut, G>, smem_intra) != KATA_OK)
    return KATA_ERR_LAUNCH;
  hipEvent_t e0 = ev ? ev[0] : nullptr, e1 = ev ? ev[1] : nullptr;
  hipEvent_t e2 = ev ? ev[2] : nullptr, e3 = ev ? ev[3] : nullptr;
  const dim3 grid((unsigned)pl.n_leaf, (unsigned)bh);
  hipExtLaunchKernelGGL((kata_chunk_state<S, TIn, false, G, true>), grid, dim3(256), smem_state, st, e0, nullptr, 0,
                        (const TIn*)k, (const TIn*)v, P, ws, d->T, (int)d->H, pl.leaf * S::C,
                        (const float*)nullptr, (float*)nullptr);
  if (launch_status() != KATA_OK) return KATA_ERR_LAUNCH;
  const int segs = scan_segments(pl);
  hipExtLaunchKernelGGL(kata_state_scan, scan_grid(pl, segs, bh), dim3(256), 0, st, e1, nullptr, 0, ws, pl.n_leaf,
                        (int)pl.E, (int)S::DV, segs, S0, z0, ST, zT, 0, (const float*)nullptr);
  if (launch_status() != KATA_OK) return KATA_ERR_LAUNCH;
  hipExtLaunchKernelGGL((kata_chunk_intra_sg<S, TIn, TOut, G>), grid, dim3(256), smem_intra, st, e2, e3, 0,
                        (const TIn*)q, (const TIn*)k, (const TIn*)v, P, (const float*)ws, (TOut*)y, d->T,
                        (int)d->H, (int)pl.leaf, pl.n_chunks);
  return launch_status();
}

// ---- chunked DeltaKATA ---------------------------------------------------------------------
// Workspace: u^, w^ [B*H, n_chunks*64, 16] float32 and T per chunk as hi/lo bf16 matrix-core
// fragments (64 x 64 x 2 bf16 per chunk), each block 256-byte aligned.
struct DeltaChunkLayout {
  int64_t n_chunks = 0;
  int64_t nseg = 1, seg_chunks = 0;   // segments of a sequence's walk, chunks per segment
  size_t off_w = 0, off_t = 0, off_prog = 0, off_aff = 0, off_s0 = 0, total = 0;
};

// Segments.  A sequence's walk runs on dv/16 workgroups, one per CU; with few sequences
// most CUs idle and the walk takes the chunk count times one chunk's dependency chain.
// Cut into segments, the segments' affine maps are formed side by side, chained in a short
// pass, and the segments' walks run side by side.  The library segments where the walks
// fill fewer than a quarter of the workgroup slots (4 per CU): nseg = 1024 / (B*H*dv/16),
// at most kDeltaMaxSegments (the chain visits the segments in order, about 10 us each)
// and at least 16 chunks per segment.  desc->scan_leaf > 0 sets the chunks per segment,
// and KATA_SCAN_SEQUENTIAL one walk per sequence.  Either way B*H*nseg stays within the
// 65535 workgroup rows of a launch (the segments' walks are its rows).
constexpr int64_t kDeltaMaxSegments = 32;
int64_t delta_segments(const kata_forward_desc* d, int64_t n_chunks, int64_t* seg_chunks) {
  const int64_t bh = d->B * d->H;
  const int64_t walks = bh * (d->dv / 16);
  int64_t per = n_chunks;
  if (d->scan == KATA_SCAN_SEQUENTIAL || n_chunks == 0) {
    per = n_chunks;
  } else if (d->scan_leaf > 0) {
    per = d->scan_leaf < n_chunks ? d->scan_leaf : n_chunks;
  } else if (walks > 0 && walks < kComputeUnits * 4) {
    int64_t want = (kComputeUnits * 4) / walks;
    if (want > kDeltaMaxSegments) want = kDeltaMaxSegments;
    if (want > n_chunks / 16) want = n_chunks / 16;
    if (want > 1) per = (n_chunks + want - 1) / want;
  }
  if (per < 1) per = 1;
  if (bh > 0) {   // at most 65535 / (B*H) segments per sequence
    const int64_t most = 65535 / bh;
    if ((n_chunks + per - 1) / per > most) per = (n_chunks + most - 1) / most;
  }
  *seg_chunks = per;
  return n_chunks == 0 ? 1 : (n_chunks + per - 1) / per;   // no empty segment
}

// u^, w^ (fp32), T (hi/lo bf16 fragments), then the walk's progress counters (one int per
// column-block workgroup); with segments, the affine maps of all but the last segment of
// each sequence [B*H*(nseg - 1), 144, dv + 144] and every segment's start state
// [B*H*nseg, 256, dv] (fp32).
DeltaChunkLayout delta_chunk_layout(const kata_forward_desc* d) {
  DeltaChunkLayout L;
  const int64_t bh = d->B * d->H;
  L.n_chunks = (d->T + kata::DC - 1) / kata::DC;
  L.nseg = delta_segments(d, L.n_chunks, &L.seg_chunks);
  const size_t uw = (size_t)bh * (size_t)L.n_chunks * kata::DC * P_DIM * sizeof(float);
  L.off_w = align256(uw);
  L.off_t = L.off_w + align256(uw);
  L.off_prog = L.off_t + align256((size_t)bh * (size_t)L.n_chunks * kata::DC * kata::DC * 2 * sizeof(bf16));
  L.off_aff = L.off_prog + align256((size_t)bh * (size_t)(d->dv / 16) * sizeof(int));
  const size_t nw = L.nseg > 1 ? (size_t)bh * (size_t)L.nseg : 0;
  const size_t nmaps = L.nseg > 1 ? (size_t)bh * (size_t)(L.nseg - 1) : 0;
  L.off_s0 = L.off_aff + align256(nmaps * DPACK * (size_t)(d->dv + DPACK) * sizeof(float));
  L.total = L.off_s0 + nw * P_DIM * P_DIM * (size_t)d->dv * sizeof(float);
  return L;
}

kata_status validate_delta_chunked(const kata_forward_desc* d) {
  if (!d) return KATA_ERR_NULL;
  if (d->B < 0 || d->H < 0 || d->T < 0 || d->d <= 0 || d->dv <= 0 || d->p <= 0) return KATA_ERR_SHAPE;
  if (d->B > 65535 || d->H > 65535 || d->B * d->H > 65535) return KATA_ERR_SHAPE;
  // the walk reads a sequence's v (and beta) with 32-bit byte offsets, as the chunked forward
  const int64_t widest = (int64_t)(d->d > d->dv ? d->d : d->dv) * 4;
  if (d->T > (((int64_t)1 << 31) - 4096) / widest - 256) return KATA_ERR_SHAPE;
  if (d->p != P_DIM || !((d->d == 16 && d->dv == 16) || (d->d == 64 && d->dv == 64))) return KATA_ERR_UNSUPPORTED;
  if (d->chunk != kata::DC) return KATA_ERR_UNSUPPORTED;
  if (check_dtype(d->in_dtype) != KATA_OK || check_dtype(d->out_dtype) != KATA_OK) return KATA_ERR_UNSUPPORTED;
  return KATA_OK;
}

template <typename TIn, typename TOut, int DV>
kata_status run_delta_chunked(const kata_forward_desc* d, const DeltaChunkLayout& L, const void* q, const void* k,
                              const void* v, const float* P, const float* beta, const float* S0, void* y,
                              float* ST, unsigned char* ws, hipStream_t st, hipEvent_t* ev) {
  const int64_t bh = d->B * d->H;
  float* U = (float*)ws;
  float* W = (float*)(ws + L.off_w);
  bf16* Tf = (bf16*)(ws + L.off_t);
  int* prog = (int*)(ws + L.off_prog);
  hipEvent_t e0 = ev ? ev[0] : nullptr, e1 = ev ? ev[1] : nullptr, e2 = ev ? ev[2] : nullptr;
  hipExtLaunchKernelGGL((kata::kata_delta_prep<TIn, DV>), dim3((unsigned)L.n_chunks, (unsigned)bh), dim3(256), 0,
                        st, e0, nullptr, 0, (const TIn*)q, (const TIn*)k, beta, P, U, W, Tf, prog, d->T, (int)d->H);
  if (launch_status() != KATA_OK) return KATA_ERR_LAUNCH;
  if (L.nseg == 1) {
    hipExtLaunchKernelGGL((kata::kata_delta_chunk<TIn, TOut, DV>), dim3((unsigned)(DV / 16), (unsigned)bh),
                          dim3(512), 0, st, e1, e2, 0, prog, (const float*)U, (const float*)W, (const bf16*)Tf,
                          (const TIn*)v, beta, S0, ST, S0, (TOut*)y, d->T, L.n_chunks, 1, L.n_chunks,
                          (float*)nullptr);
    return launch_status();
  }
  // segments: the affine maps of all but the last segment side by side (the last
  // segment's walk ends the sequence and exports S_T itself), the chain of start states,
  // the segments' walks
  float* aff = (float*)(ws + L.off_aff);
  float* S0seg = (float*)(ws + L.off_s0);
  const unsigned nmaps = (unsigned)(bh * (L.nseg - 1)), nw = (unsigned)(bh * L.nseg);
  hipExtLaunchKernelGGL((kata::kata_delta_chunk<TIn, TOut, DV, true>), dim3((unsigned)((DV + DPACK) / 16), nmaps),
                        dim3(256), 0, st, e1, nullptr, 0, prog, (const float*)U, (const float*)W, (const bf16*)Tf,
                        (const TIn*)v, beta, S0, (float*)nullptr, (const float*)nullptr, (TOut*)nullptr, d->T,
                        L.n_chunks, (int)(L.nseg - 1), L.seg_chunks, aff);
  if (launch_status() != KATA_OK) return KATA_ERR_LAUNCH;
  hipLaunchKernelGGL((kata::kata_delta_seg_combine<DV>), dim3((unsigned)(DV / 16), (unsigned)bh), dim3(kata::SEG_THREADS),
                     0, st, (const float*)aff, S0, S0seg, (int)L.nseg);
  if (launch_status() != KATA_OK) return KATA_ERR_LAUNCH;
  hipExtLaunchKernelGGL((kata::kata_delta_chunk<TIn, TOut, DV>), dim3((unsigned)(DV / 16), nw), dim3(512), 0, st,
                        nullptr, e2, 0, prog, (const float*)U, (const float*)W, (const bf16*)Tf, (const TIn*)v, beta,
                        (const float*)S0seg, ST, S0, (TOut*)y, d->T, L.n_chunks, (int)L.nseg, L.seg_chunks,
                        (float*)nullptr);
  return launch_status();
}

// KATA-Mg / Sigma-g decode step: one workgroup per (stream, head).
template <int G, bool SUMG>
kata_status launch_decode_factors(int64_t NH, int H, int d, int dv, kata_dtype in_dtype, kata_dtype out_dtype,
                                  float* S, float* z, const void* q, const void* k, const void* v, const float* P,
                                  void* y, hipStream_t st) {
  const dim3 grid((unsigned)NH);
#define KATA_DF(TI, TO, DVV)                                                                                   \
  hipLaunchKernelGGL((kata::kata_decode_step_factors<TI, TO, DVV, G, SUMG>), grid, dim3(256), 0, st, S, z,      \
                     (const TI*)q, (const TI*)k, (const TI*)v, P, (TO*)y, H, d)
  const bool fi = in_dtype == KATA_F32, fo = out_dtype == KATA_F32;
  if (dv == 64) {
    if (fi && fo) KATA_DF(float, float, 64);
    else if (fi) KATA_DF(float, bf16, 64);
    else if (fo) KATA_DF(bf16, float, 64);
    else KATA_DF(bf16, bf16, 64);
  } else {
    if (fi && fo) KATA_DF(float, float, 16);
    else if (fi) KATA_DF(float, bf16, 16);
    else if (fo) KATA_DF(bf16, float, 16);
    else KATA_DF(bf16, bf16, 16);
  }
#undef KATA_DF
  return launch_status();
}

// The decode step on the packed symmetric state (kata_decode_step_packed): one-factor,
// decay-gated (DECAY) or several PSD factors (G > 1, concatenated or SUMG).
template <int G, bool SUMG, bool DECAY>
kata_status launch_decode_packed(int64_t NH, int H, int d, int dv, kata_dtype in_dtype, kata_dtype out_dtype,
                                 float* Sp, float* zp, const void* q, const void* k, const void* v, const float* P,
                                 const float* lam, void* y, hipStream_t st) {
  const dim3 grid((unsigned)NH);
#define KATA_DP(TI, TO, DVV)                                                                                      \
  hipLaunchKernelGGL((kata::kata_decode_step_packed<TI, TO, DVV, G, SUMG, DECAY>), grid, dim3(256), 0, st, Sp, zp, \
                     (const TI*)q, (const TI*)k, (const TI*)v, P, (TO*)y, H, d, lam)
  const bool fi = in_dtype == KATA_F32, fo = out_dtype == KATA_F32;
  if (dv == 64) {
    if (fi && fo) KATA_DP(float, float, 64);
    else if (fi) KATA_DP(float, bf16, 64);
    else if (fo) KATA_DP(bf16, float, 64);
    else KATA_DP(bf16, bf16, 64);
  } else {
    if (fi && fo) KATA_DP(float, float, 16);
    else if (fi) KATA_DP(float, bf16, 16);
    else if (fo) KATA_DP(bf16, float, 16);
    else KATA_DP(bf16, bf16, 16);
  }
#undef KATA_DP
  return launch_status();
}

// Shared checks of the decode entry points: sizes, supported shapes and dtypes.
kata_status validate_decode(int64_t N, int64_t H, int d, int dv, int p, const kata_dtype& in_dtype,
                            const kata_dtype& out_dtype) {
  if (N < 0 || H < 0 || d <= 0 || dv <= 0 || p <= 0) return KATA_ERR_SHAPE;
  if (p != P_DIM || !((d == 16 && dv == 16) || (d == 64 && dv == 64))) return KATA_ERR_UNSUPPORTED;
  if (check_dtype(in_dtype) != KATA_OK || check_dtype(out_dtype) != KATA_OK) return KATA_ERR_UNSUPPORTED;
  if (N > 0 && H > 0x7fffffff / N) return KATA_ERR_SHAPE;
  return KATA_OK;
}

}  // namespace

extern "C" {

int kata_abi_version(void) { return KATA_ABI_VERSION; }

const char* kata_status_string(kata_status s) {
  switch (bits(s)) {
    case KATA_OK: return "KATA_OK";
    case KATA_ERR_NULL: return "KATA_ERR_NULL: a required pointer is NULL";
    case KATA_ERR_SHAPE: return "KATA_ERR_SHAPE: invalid or inconsistent size";
    case KATA_ERR_UNSUPPORTED: return "KATA_ERR_UNSUPPORTED: p, d, dv, chunk, dtype or scan mode not supported";
    case KATA_ERR_WORKSPACE: return "KATA_ERR_WORKSPACE: workspace missing or too small";
    case KATA_ERR_LAUNCH: return "KATA_ERR_LAUNCH: a kernel launch failed";
    case KATA_ERR_SCRATCH:
      return "KATA_ERR_SCRATCH: the problem needs more than the KATA_NOALLOC_SCRATCH_BYTES (64 MiB) scratch buffer "
             "of kata_forward_noalloc";
  }
  return "KATA: unknown status";
}

kata_status kata_forward_workspace_bytes(const kata_forward_desc* desc, size_t* bytes) {
  if (!bytes) return KATA_ERR_NULL;
  const kata_status s = validate(desc);
  if (s != KATA_OK) return s;
  *bytes = make_plan(desc).ws_bytes;
  return KATA_OK;
}

kata_status kata_forward_plan(const kata_forward_desc* desc, int64_t* n_leaf, int64_t* leaf_chunks, int* scanned) {
  const kata_status s = validate(desc);
  if (s != KATA_OK) return s;
  const Plan pl = make_plan(desc);
  if (n_leaf) *n_leaf = pl.n_leaf;
  if (leaf_chunks) *leaf_chunks = pl.leaf;
  if (scanned) *scanned = pl.direct ? 0 : 1;
  return KATA_OK;
}

kata_status kata_forward_timed(const kata_forward_desc* desc, const void* q, const void* k, const void* v,
                               const float* P, const float* S0, const float* z0, void* y, float* ST, float* zT,
                               void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
  kata_status s = validate(desc);
  if (s != KATA_OK) return s;
  if ((S0 == nullptr) != (z0 == nullptr)) return KATA_ERR_NULL;
  if ((ST == nullptr) != (zT == nullptr)) return KATA_ERR_NULL;
  const Plan pl = make_plan(desc);
  const int64_t bh = desc->B * desc->H;
  hipStream_t st = (hipStream_t)stream;
  if (bh == 0) return KATA_OK;
  if (desc->T == 0) return copy_initial_state(desc, S0, z0, ST, zT, st);
  if (!q || !k || !v || !P || !y) return KATA_ERR_NULL;
  if (!workspace || workspace_bytes < pl.ws_bytes) return KATA_ERR_WORKSPACE;
  if (pl.n_leaf > 0x7fffffff) return KATA_ERR_SHAPE;
  hipEvent_t ev[4];
  hipEvent_t* evp = nullptr;
  if (events) {
    for (int i = 0; i < 4; ++i) {
      ev[i] = (hipEvent_t)events[i];
    }
    evp = ev;
  }
  float* ws = (float*)workspace;
  switch (desc->chunk) {
    case 32: return dispatch_dims<32>(desc, pl, q, k, v, P, S0, z0, y, ST, zT, ws, st, evp);
    case 64: return dispatch_dims<64>(desc, pl, q, k, v, P, S0, z0, y, ST, zT, ws, st, evp);
    default: return dispatch_dims<128>(desc, pl, q, k, v, P, S0, z0, y, ST, zT, ws, st, evp);
  }
}

kata_status kata_forward(const kata_forward_desc* desc, const void* q, const void* k, const void* v,
                         const float* P, const float* S0, const float* z0, void* y, float* ST, float* zT,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return kata_forward_timed(desc, q, k, v, P, S0, z0, y, ST, zT, workspace, workspace_bytes, stream, nullptr);
}

kata_status kata_forward_noalloc(const kata_forward_desc* desc, const void* q, const void* k, const void* v,
                                 const float* P, const float* S0, const float* z0, void* y, float* ST, float* zT,
                                 void* stream) {
  kata_status s = validate(desc);
  if (s != KATA_OK) return s;
  if ((S0 == nullptr) != (z0 == nullptr)) return KATA_ERR_NULL;
  if ((ST == nullptr) != (zT == nullptr)) return KATA_ERR_NULL;
  const Plan pl = make_plan(desc);
  if (pl.ws_bytes > KATA_NOALLOC_SCRATCH_BYTES) return KATA_ERR_SCRATCH;
  if (desc->B * desc->H == 0) return KATA_OK;
  if (desc->T > 0 && (!q || !k || !v || !P || !y)) return KATA_ERR_NULL;
  void* ws = nullptr;
  if (desc->T > 0 && !(ws = scratch_address())) return KATA_ERR_LAUNCH;
  return kata_forward_timed(desc, q, k, v, P, S0, z0, y, ST, zT, ws, KATA_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

kata_status kata_flash_workspace_bytes(const kata_forward_desc* desc, size_t* bytes) {
  if (!bytes) return KATA_ERR_NULL;
  const kata_status s = validate_flash(desc);
  if (s != KATA_OK) return s;
  *bytes = flash_ws_bytes(desc);
  return KATA_OK;
}

kata_status kata_flash_forward(const kata_forward_desc* desc, const void* q, const void* k, const void* v,
                               const float* P, void* y, void* workspace, size_t workspace_bytes, void* stream,
                               void* const* events) {
  const kata_status s = validate_flash(desc);
  if (s != KATA_OK) return s;
  const int64_t bh = desc->B * desc->H;
  if (bh == 0 || desc->T == 0) return KATA_OK;
  if (!q || !k || !v || !P || !y) return KATA_ERR_NULL;
  if (!workspace || workspace_bytes < flash_ws_bytes(desc)) return KATA_ERR_WORKSPACE;
  hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
  if (events) {
    for (int i = 0; i < 3; ++i) {
      ev[i] = (hipEvent_t)events[i];
    }
  }
  hipStream_t st = (hipStream_t)stream;
  const int64_t tpad = flash_tpad(desc->T);
  bf16* ws = (bf16*)workspace;
  hipExtLaunchKernelGGL((kata_flash_prep<bf16>), dim3((unsigned)(tpad / 64), (unsigned)bh), dim3(256), 0, st,
                        ev[0], nullptr, 0, (const bf16*)q, (const bf16*)k, (const bf16*)v, P, ws, desc->T, tpad,
                        (int)desc->H);
  if (launch_status() != KATA_OK) return KATA_ERR_LAUNCH;
  if ((tpad / FL_QB) * bh > 0x7fffffff) return KATA_ERR_SHAPE;
  const dim3 grid((unsigned)((tpad / FL_QB) * bh));
  if (desc->out_dtype == KATA_F32)
    hipExtLaunchKernelGGL(kata_flash_attn<float>, grid, dim3(64 * FL_WAVES), 0, st, ev[1], ev[2], 0, (const bf16*)ws,
                          (float*)y, desc->T, tpad, (int)bh);
  else
    hipExtLaunchKernelGGL(kata_flash_attn<bf16>, grid, dim3(64 * FL_WAVES), 0, st, ev[1], ev[2], 0, (const bf16*)ws,
                          (bf16*)y, desc->T, tpad, (int)bh);
  return launch_status();
}

kata_status kata_backward_workspace_bytes(const kata_forward_desc* desc, size_t* bytes) {
  if (!bytes) return KATA_ERR_NULL;
  const kata_status s = validate_bwd(desc);
  if (s != KATA_OK) return s;
  *bytes = bwd_layout(desc).total;
  return KATA_OK;
}

kata_status kata_backward_timed(const kata_forward_desc* desc, const void* q, const void* k, const void* v,
                                const float* P, const float* S0, const float* z0, const void* gy,
                                const float* gST, const float* gzT, void* dq, void* dk, void* dv, float* dP,
                                float* dS0, float* dz0, void* workspace, size_t workspace_bytes, void* stream,
                                void* const* events) {
  const kata_status s = validate_bwd(desc);
  if (s != KATA_OK) return s;
  if ((S0 == nullptr) != (z0 == nullptr)) return KATA_ERR_NULL;
  if ((gST == nullptr) != (gzT == nullptr)) return KATA_ERR_NULL;
  if ((dS0 == nullptr) != (dz0 == nullptr)) return KATA_ERR_NULL;
  if (!dP) return KATA_ERR_NULL;
  hipStream_t st = (hipStream_t)stream;
  const int64_t bh = desc->B * desc->H;
  const int64_t nP = desc->H * BW_DP;
  if (bh == 0 || desc->T == 0) {
    // no token: dP = 0 and the initial state's gradient is the final state's (S_T = S0)
    if (nP > 0)
      hipLaunchKernelGGL(kata_copy_or_zero, dim3((unsigned)((nP + 255) / 256)), dim3(256), 0, st, dP,
                         (const float*)nullptr, nP);
    if (bh > 0 && dS0) {
      const int64_t nS = bh * P_DIM * P_DIM * desc->dv, nz = bh * P_DIM * P_DIM;
      hipLaunchKernelGGL(kata_sym_copy_or_zero, dim3((unsigned)((nS + 255) / 256)), dim3(256), 0, st, dS0, gST, nS,
                         desc->dv);
      hipLaunchKernelGGL(kata_sym_copy_or_zero, dim3((unsigned)((nz + 255) / 256)), dim3(256), 0, st, dz0, gzT, nz, 1);
    }
    return launch_status();
  }
  if (!q || !k || !v || !P || !gy || !dq || !dk || !dv) return KATA_ERR_NULL;
  const BwdLayout L = bwd_layout(desc);
  if (!workspace || workspace_bytes < L.total) return KATA_ERR_WORKSPACE;
  if (L.pl.n_leaf > 0x7fffffff) return KATA_ERR_SHAPE;
  hipEvent_t ev[8];
  hipEvent_t* evp = nullptr;
  if (events) {
    for (int i = 0; i < 8; ++i) {
      ev[i] = (hipEvent_t)events[i];
    }
    evp = ev;
  }
  unsigned char* wsb = (unsigned char*)workspace;
  if (desc->out_dtype == KATA_F32)
    return run_backward<float>(desc, L, q, k, v, P, S0, z0, gy, gST, gzT, dq, dk, dv, dP, dS0, dz0, wsb, st, evp);
  return run_backward<bf16>(desc, L, q, k, v, P, S0, z0, gy, gST, gzT, dq, dk, dv, dP, dS0, dz0, wsb, st, evp);
}

kata_status kata_backward(const kata_forward_desc* desc, const void* q, const void* k, const void* v,
                          const float* P, const float* S0, const float* z0, const void* gy,
                          const float* gST, const float* gzT, void* dq, void* dk, void* dv, float* dP, float* dS0,
                          float* dz0, void* workspace, size_t workspace_bytes, void* stream) {
  return kata_backward_timed(desc, q, k, v, P, S0, z0, gy, gST, gzT, dq, dk, dv, dP, dS0, dz0, workspace,
                             workspace_bytes, stream, nullptr);
}

kata_status kata_forward_decay_workspace_bytes(const kata_forward_desc* desc, size_t* bytes) {
  if (!bytes) return KATA_ERR_NULL;
  const kata_status s = validate_decay(desc);
  if (s != KATA_OK) return s;
  *bytes = decay_ws_bytes(make_plan(desc), desc);
  return KATA_OK;
}

kata_status kata_forward_decay_timed(const kata_forward_desc* desc, const void* q, const void* k, const void* v,
                                     const float* P, const float* lam, const float* S0, const float* z0, void* y,
                                     float* ST, float* zT, void* workspace, size_t workspace_bytes, void* stream,
                                     void* const* events) {
  const kata_status s = validate_decay(desc);
  if (s != KATA_OK) return s;
  if ((S0 == nullptr) != (z0 == nullptr)) return KATA_ERR_NULL;
  if ((ST == nullptr) != (zT == nullptr)) return KATA_ERR_NULL;
  const Plan pl = make_plan(desc);
  const int64_t bh = desc->B * desc->H;
  hipStream_t st = (hipStream_t)stream;
  if (bh == 0) return KATA_OK;
  if (desc->T == 0) return copy_initial_state(desc, S0, z0, ST, zT, st);
  if (!q || !k || !v || !P || !lam || !y) return KATA_ERR_NULL;
  if (!workspace || workspace_bytes < decay_ws_bytes(pl, desc)) return KATA_ERR_WORKSPACE;
  if (pl.n_leaf > 0x7fffffff) return KATA_ERR_SHAPE;
  hipEvent_t ev[4];
  hipEvent_t* evp = nullptr;
  if (events) {
    for (int i = 0; i < 4; ++i) {
      ev[i] = (hipEvent_t)events[i];
    }
    evp = ev;
  }
  float* ws = (float*)workspace;
  float* dec = (float*)((unsigned char*)workspace + align256(pl.ws_bytes));
  using S = Shape<64, 64, 64, false>;
  if (desc->out_dtype == KATA_F32)
    return run_forward<S, bf16, float, true>(desc, pl, q, k, v, P, S0, z0, y, ST, zT, ws, st, evp, lam, dec);
  return run_forward<S, bf16, bf16, true>(desc, pl, q, k, v, P, S0, z0, y, ST, zT, ws, st, evp, lam, dec);
}

kata_status kata_forward_decay(const kata_forward_desc* desc, const void* q, const void* k, const void* v,
                               const float* P, const float* lam, const float* S0, const float* z0, void* y,
                               float* ST, float* zT, void* workspace, size_t workspace_bytes, void* stream) {
  return kata_forward_decay_timed(desc, q, k, v, P, lam, S0, z0, y, ST, zT, workspace, workspace_bytes, stream,
                                  nullptr);
}

kata_status kata_decode_step_decay(int64_t N, int64_t H, int d, int dv, int p, kata_dtype in_dtype,
                                   kata_dtype out_dtype, float* S, float* z, const void* q, const void* k,
                                   const void* v, const float* P, const float* lam, void* y, void* stream) {
  if (N < 0 || H < 0 || d <= 0 || dv <= 0 || p <= 0) return KATA_ERR_SHAPE;
  if (p != P_DIM || !((d == 16 && dv == 16) || (d == 64 && dv == 64))) return KATA_ERR_UNSUPPORTED;
  if (check_dtype(in_dtype) != KATA_OK || check_dtype(out_dtype) != KATA_OK) return KATA_ERR_UNSUPPORTED;
  if (N * H == 0) return KATA_OK;
  if (N * H > 0x7fffffff) return KATA_ERR_SHAPE;
  if (!S || !z || !q || !k || !v || !P || !lam || !y) return KATA_ERR_NULL;
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid((unsigned)(N * H));
#define KATA_DECODE_D(TI, TO, DVV)                                                                         \
  hipLaunchKernelGGL((kata::kata_decode_step<TI, TO, DVV, true>), grid, dim3(256), 0, st, S, z, (const TI*)q, \
                     (const TI*)k, (const TI*)v, P, (TO*)y, (int)H, d, lam)
  const bool fi = in_dtype == KATA_F32, fo = out_dtype == KATA_F32;
  if (dv == 64) {
    if (fi && fo) KATA_DECODE_D(float, float, 64);
    else if (fi) KATA_DECODE_D(float, bf16, 64);
    else if (fo) KATA_DECODE_D(bf16, float, 64);
    else KATA_DECODE_D(bf16, bf16, 64);
  } else {
    if (fi && fo) KATA_DECODE_D(float, float, 16);
    else if (fi) KATA_DECODE_D(float, bf16, 16);
    else if (fo) KATA_DECODE_D(bf16, float, 16);
    else KATA_DECODE_D(bf16, bf16, 16);
  }
#undef KATA_DECODE_D
  return launch_status();
}

kata_status kata_decode_step(int64_t N, int64_t H, int d, int dv, int p, kata_dtype in_dtype,
                             kata_dtype out_dtype, float* S, float* z, const void* q, const void* k,
                             const void* v, const float* P, void* y, void* stream) {
  if (N < 0 || H < 0 || d <= 0 || dv <= 0 || p <= 0) return KATA_ERR_SHAPE;
  if (p != P_DIM || !((d == 16 && dv == 16) || (d == 64 && dv == 64))) return KATA_ERR_UNSUPPORTED;
  if (check_dtype(in_dtype) != KATA_OK || check_dtype(out_dtype) != KATA_OK) return KATA_ERR_UNSUPPORTED;
  if (N * H == 0) return KATA_OK;
  if (N * H > 0x7fffffff) return KATA_ERR_SHAPE;
  if (!S || !z || !q || !k || !v || !P || !y) return KATA_ERR_NULL;
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid((unsigned)(N * H));
#define KATA_DECODE(TI, TO, DVV)                                                                     \
  hipLaunchKernelGGL((kata::kata_decode_step<TI, TO, DVV, false>), grid, dim3(256), 0, st, S, z, (const TI*)q, \
                     (const TI*)k, (const TI*)v, P, (TO*)y, (int)H, d, (const float*)nullptr)
  const bool fi = in_dtype == KATA_F32, fo = out_dtype == KATA_F32;
  if (dv == 64) {
    if (fi && fo) KATA_DECODE(float, float, 64);
    else if (fi) KATA_DECODE(float, bf16, 64);
    else if (fo) KATA_DECODE(bf16, float, 64);
    else KATA_DECODE(bf16, bf16, 64);
  } else {
    if (fi && fo) KATA_DECODE(float, float, 16);
    else if (fi) KATA_DECODE(float, bf16, 16);
    else if (fo) KATA_DECODE(bf16, float, 16);
    else KATA_DECODE(bf16, bf16, 16);
  }
#undef KATA_DECODE
  return launch_status();
}

kata_status kata_decode_step_packed(int64_t N, int64_t H, int d, int dv, int p, kata_dtype in_dtype,
                                    kata_dtype out_dtype, float* Sp, float* zp, const void* q, const void* k,
                                    const void* v, const float* P, void* y, void* stream) {
  const kata_status s = validate_decode(N, H, d, dv, p, in_dtype, out_dtype);
  if (s != KATA_OK || N * H == 0) return s;
  if (!Sp || !zp || !q || !k || !v || !P || !y) return KATA_ERR_NULL;
  return launch_decode_packed<1, false, false>(N * H, (int)H, d, dv, in_dtype, out_dtype, Sp, zp, q, k, v, P,
                                               nullptr, y, (hipStream_t)stream);
}

kata_status kata_decode_step_decay_packed(int64_t N, int64_t H, int d, int dv, int p, kata_dtype in_dtype,
                                          kata_dtype out_dtype, float* Sp, float* zp, const void* q, const void* k,
                                          const void* v, const float* P, const float* lam, void* y, void* stream) {
  const kata_status s = validate_decode(N, H, d, dv, p, in_dtype, out_dtype);
  if (s != KATA_OK || N * H == 0) return s;
  if (!Sp || !zp || !q || !k || !v || !P || !lam || !y) return KATA_ERR_NULL;
  return launch_decode_packed<1, false, true>(N * H, (int)H, d, dv, in_dtype, out_dtype, Sp, zp, q, k, v, P, lam,
                                              y, (hipStream_t)stream);
}

kata_status kata_decode_step_factors_packed(int64_t N, int64_t H, int d, int dv, int p, int g,
                                            kata_factor_mode mode, kata_dtype in_dtype, kata_dtype out_dtype,
                                            float* Sp, float* zp, const void* q, const void* k, const void* v,
                                            const float* P, void* y, void* stream) {
  if (g < 1) return KATA_ERR_SHAPE;
  if (!valid_mode(mode)) return KATA_ERR_UNSUPPORTED;
  if (g > kMaxFactors) return KATA_ERR_UNSUPPORTED;
  const kata_status s = validate_decode(N, H, d, dv, p, in_dtype, out_dtype);
  if (s != KATA_OK || N * H == 0) return s;
  if (!Sp || !zp || !q || !k || !v || !P || !y) return KATA_ERR_NULL;
  hipStream_t st = (hipStream_t)stream;
  const int64_t NH = N * H;
  const bool sum = mode == KATA_FACTORS_SUM;
#define KATA_DFP(GG, SS) \
  launch_decode_packed<GG, SS, false>(NH, (int)H, d, dv, in_dtype, out_dtype, Sp, zp, q, k, v, P, nullptr, y, st)
  if (g == 1) return KATA_DFP(1, false);
  if (g == 2) return sum ? KATA_DFP(2, true) : KATA_DFP(2, false);
  return sum ? KATA_DFP(3, true) : KATA_DFP(3, false);
#undef KATA_DFP
}

kata_status kata_state_pack(int64_t n, int dv, const float* S, const float* z, float* Sp, float* zp, void* stream) {
  if (n < 0) return KATA_ERR_SHAPE;
  if (dv != 16 && dv != 64) return KATA_ERR_UNSUPPORTED;
  if (n > 0x7fffffff / kata::DPK) return KATA_ERR_SHAPE;
  if ((z == nullptr) != (zp == nullptr)) return KATA_ERR_NULL;
  if (n == 0) return KATA_OK;
  if (!S || !Sp) return KATA_ERR_NULL;
  hipLaunchKernelGGL(kata::kata_state_pack, dim3((unsigned)(n * kata::DPK)), dim3(64), 0, (hipStream_t)stream, S, z,
                     Sp, zp, dv);
  return launch_status();
}

kata_status kata_state_unpack(int64_t n, int dv, const float* Sp, const float* zp, float* S, float* z,
                              void* stream) {
  if (n < 0) return KATA_ERR_SHAPE;
  if (dv != 16 && dv != 64) return KATA_ERR_UNSUPPORTED;
  if (n > 0x7fffffff / (P_DIM * P_DIM)) return KATA_ERR_SHAPE;
  if ((z == nullptr) != (zp == nullptr)) return KATA_ERR_NULL;
  if (n == 0) return KATA_OK;
  if (!S || !Sp) return KATA_ERR_NULL;
  hipLaunchKernelGGL(kata::kata_state_unpack, dim3((unsigned)(n * P_DIM * P_DIM)), dim3(64), 0, (hipStream_t)stream,
                     Sp, zp, S, z, dv);
  return launch_status();
}

kata_status kata_forward_delta(const kata_forward_desc* desc, const void* q, const void* k, const void* v,
                               const float* P, const float* beta, const float* S0, void* y, float* ST,
                               void* stream) {
  if (!desc) return KATA_ERR_NULL;
  const kata_forward_desc* d = desc;
  if (d->B < 0 || d->H < 0 || d->T < 0 || d->d <= 0 || d->dv <= 0 || d->p <= 0) return KATA_ERR_SHAPE;
  if (d->p != P_DIM || !((d->d == 16 && d->dv == 16) || (d->d == 64 && d->dv == 64))) return KATA_ERR_UNSUPPORTED;
  if (check_dtype(d->in_dtype) != KATA_OK || check_dtype(d->out_dtype) != KATA_OK) return KATA_ERR_UNSUPPORTED;
  if (d->B > 0 && d->H > 0x7fffffff / d->B) return KATA_ERR_SHAPE;
  const int64_t BH = d->B * d->H;
  if (BH == 0) return KATA_OK;
  if (d->T > ((int64_t)1 << 40)) return KATA_ERR_SHAPE;
  if (!P) return KATA_ERR_NULL;
  if (d->T > 0 && (!q || !k || !v || !beta || !y)) return KATA_ERR_NULL;
  if (d->T == 0 && !ST) return KATA_OK;
  return launch_delta(BH, d->T, (int)d->H, d->d, d->dv, d->in_dtype, d->out_dtype, S0, ST, q, k, v, beta, P, y,
                      (hipStream_t)stream);
}

kata_status kata_decode_step_delta(int64_t N, int64_t H, int d, int dv, int p, kata_dtype in_dtype,
                                   kata_dtype out_dtype, float* S, const void* q, const void* k, const void* v,
                                   const float* P, const float* beta, void* y, void* stream) {
  if (N < 0 || H < 0 || d <= 0 || dv <= 0 || p <= 0) return KATA_ERR_SHAPE;
  if (p != P_DIM || !((d == 16 && dv == 16) || (d == 64 && dv == 64))) return KATA_ERR_UNSUPPORTED;
  if (check_dtype(in_dtype) != KATA_OK || check_dtype(out_dtype) != KATA_OK) return KATA_ERR_UNSUPPORTED;
  if (N > 0 && H > 0x7fffffff / N) return KATA_ERR_SHAPE;
  if (N * H == 0) return KATA_OK;
  if (!S || !q || !k || !v || !P || !beta || !y) return KATA_ERR_NULL;
  return launch_delta(N * H, 1, (int)H, d, dv, in_dtype, out_dtype, S, S, q, k, v, beta, P, y, (hipStream_t)stream);
}

kata_status kata_decode_step_delta_packed(int64_t N, int64_t H, int d, int dv, int p, kata_dtype in_dtype,
                                          kata_dtype out_dtype, float* Sp, const void* q, const void* k,
                                          const void* v, const float* P, const float* beta, void* y, void* stream) {
  const kata_status s = validate_decode(N, H, d, dv, p, in_dtype, out_dtype);
  if (s != KATA_OK || N * H == 0) return s;
  if (!Sp || !q || !k || !v || !P || !beta || !y) return KATA_ERR_NULL;
  return launch_delta<true>(N * H, 1, (int)H, d, dv, in_dtype, out_dtype, Sp, Sp, q, k, v, beta, P, y,
                            (hipStream_t)stream);
}

kata_status kata_forward_factors_workspace_bytes(const kata_forward_desc* desc, int g, kata_factor_mode mode,
                                                 size_t* bytes) {
  if (!bytes) return KATA_ERR_NULL;
  const kata_status s = validate_factors(desc, g, mode);
  if (s != KATA_OK) return s;
  *bytes = factors_plan(desc, g, mode).ws_bytes;
  return KATA_OK;
}

kata_status kata_forward_factors_timed(const kata_forward_desc* desc, int g, kata_factor_mode mode, const void* q,
                                       const void* k, const void* v, const float* P, const float* S0,
                                       const float* z0, void* y, float* ST, float* zT, void* workspace,
                                       size_t workspace_bytes, void* stream, void* const* events) {
  kata_status s = validate_factors(desc, g, mode);
  if (s != KATA_OK) return s;
  if (g == 1)
    return kata_forward_timed(desc, q, k, v, P, S0, z0, y, ST, zT, workspace, workspace_bytes, stream, events);
  if ((S0 == nullptr) != (z0 == nullptr)) return KATA_ERR_NULL;
  if ((ST == nullptr) != (zT == nullptr)) return KATA_ERR_NULL;
  const Plan pl = factors_plan(desc, g, mode);
  const int64_t bh = desc->B * desc->H;
  hipStream_t st = (hipStream_t)stream;
  if (bh == 0) return KATA_OK;
  if (desc->T == 0) {   // CONCAT: the export of g stacked factor states is that of B*H*g rows
    kata_forward_desc dd = *desc;
    if (mode == KATA_FACTORS_CONCAT) dd.H = desc->H * g;
    return copy_initial_state(&dd, S0, z0, ST, zT, st);
  }
  if (!q || !k || !v || !P || !y) return KATA_ERR_NULL;
  if (!workspace || workspace_bytes < pl.ws_bytes) return KATA_ERR_WORKSPACE;
  if (pl.n_leaf > 0x7fffffff) return KATA_ERR_SHAPE;
  hipEvent_t ev[4];
  hipEvent_t* evp = nullptr;
  if (events) {
    for (int i = 0; i < 4; ++i) {
      ev[i] = (hipEvent_t)events[i];
    }
    evp = ev;
  }
  float* ws = (float*)workspace;
  using S = Shape<64, 64, 64, false>;
  const bool fo = desc->out_dtype == KATA_F32;
  if (mode == KATA_FACTORS_SUM) {
    if (g == 2)
      return fo ? run_forward_sg<S, bf16, float, 2>(desc, pl, q, k, v, P, S0, z0, y, ST, zT, ws, st, evp)
                : run_forward_sg<S, bf16, bf16, 2>(desc, pl, q, k, v, P, S0, z0, y, ST, zT, ws, st, evp);
    return fo ? run_forward_sg<S, bf16, float, 3>(desc, pl, q, k, v, P, S0, z0, y, ST, zT, ws, st, evp)
              : run_forward_sg<S, bf16, bf16, 3>(desc, pl, q, k, v, P, S0, z0, y, ST, zT, ws, st, evp);
  }
  if (g == 2)
    return fo ? run_forward_mg<S, bf16, float, 2>(desc, pl, q, k, v, P, S0, z0, y, ST, zT, ws, st, evp)
              : run_forward_mg<S, bf16, bf16, 2>(desc, pl, q, k, v, P, S0, z0, y, ST, zT, ws, st, evp);
  return fo ? run_forward_mg<S, bf16, float, 3>(desc, pl, q, k, v, P, S0, z0, y, ST, zT, ws, st, evp)
            : run_forward_mg<S, bf16, bf16, 3>(desc, pl, q, k, v, P, S0, z0, y, ST, zT, ws, st, evp);
}

kata_status kata_forward_factors(const kata_forward_desc* desc, int g, kata_factor_mode mode, const void* q,
                                 const void* k, const void* v, const float* P, const float* S0, const float* z0,
                                 void* y, float* ST, float* zT, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return kata_forward_factors_timed(desc, g, mode, q, k, v, P, S0, z0, y, ST, zT, workspace, workspace_bytes,
                                    stream, nullptr);
}

kata_status kata_forward_delta_chunked_workspace_bytes(const kata_forward_desc* desc, size_t* bytes) {
  if (!bytes) return KATA_ERR_NULL;
  const kata_status s = validate_delta_chunked(desc);
  if (s != KATA_OK) return s;
  *bytes = delta_chunk_layout(desc).total;
  return KATA_OK;
}

kata_status kata_forward_delta_chunked_plan(const kata_forward_desc* desc, int64_t* segments,
                                            int64_t* segment_chunks) {
  const kata_status s = validate_delta_chunked(desc);
  if (s != KATA_OK) return s;
  const DeltaChunkLayout L = delta_chunk_layout(desc);
  if (segments) *segments = L.nseg;
  if (segment_chunks) *segment_chunks = L.seg_chunks;
  return KATA_OK;
}

kata_status kata_forward_delta_chunked_timed(const kata_forward_desc* desc, const void* q, const void* k,
                                             const void* v, const float* P, const float* beta, const float* S0,
                                             void* y, float* ST, void* workspace, size_t workspace_bytes,
                                             void* stream, void* const* events) {
  const kata_status s = validate_delta_chunked(desc);
  if (s != KATA_OK) return s;
  const int64_t bh = desc->B * desc->H;
  if (bh == 0) return KATA_OK;
  hipStream_t st = (hipStream_t)stream;
  if (desc->T == 0) {   // no tokens: ST = S0 (or 0)
    if (!ST) return KATA_OK;
    const int64_t nS = bh * P_DIM * P_DIM * desc->dv;
    hipLaunchKernelGGL(kata_copy_or_zero, dim3((unsigned)((nS + 255) / 256)), dim3(256), 0, st, ST, S0, nS);
    return launch_status();
  }
  if (!q || !k || !v || !P || !beta || !y) return KATA_ERR_NULL;
  const DeltaChunkLayout L = delta_chunk_layout(desc);
  if (!workspace || workspace_bytes < L.total) return KATA_ERR_WORKSPACE;
  if (L.n_chunks > 0x7fffffff) return KATA_ERR_SHAPE;
  hipEvent_t ev[3];
  hipEvent_t* evp = nullptr;
  if (events) {
    for (int i = 0; i < 3; ++i) {
      ev[i] = (hipEvent_t)events[i];
    }
    evp = ev;
  }
  unsigned char* ws = (unsigned char*)workspace;
  const bool fi = desc->in_dtype == KATA_F32, fo = desc->out_dtype == KATA_F32;
#define KATA_DCH(TI, TO, DVV) \
  return run_delta_chunked<TI, TO, DVV>(desc, L, q, k, v, P, beta, S0, y, ST, ws, st, evp)
  if (desc->dv == 64) {
    if (fi && fo) KATA_DCH(float, float, 64);
    if (fi) KATA_DCH(float, bf16, 64);
    if (fo) KATA_DCH(bf16, float, 64);
    KATA_DCH(bf16, bf16, 64);
  }
  if (fi && fo) KATA_DCH(float, float, 16);
  if (fi) KATA_DCH(float, bf16, 16);
  if (fo) KATA_DCH(bf16, float, 16);
  KATA_DCH(bf16, bf16, 16);
#undef KATA_DCH
}

kata_status kata_forward_delta_chunked(const kata_forward_desc* desc, const void* q, const void* k, const void* v,
                                       const float* P, const float* beta, const float* S0, void* y, float* ST,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  return kata_forward_delta_chunked_timed(desc, q, k, v, P, beta, S0, y, ST, workspace, workspace_bytes, stream,
                                          nullptr);
}

kata_status kata_decode_step_factors(int64_t N, int64_t H, int d, int dv, int p, int g, kata_factor_mode mode,
                                     kata_dtype in_dtype, kata_dtype out_dtype, float* S, float* z, const void* q,
                                     const void* k, const void* v, const float* P, void* y, void* stream) {
  if (N < 0 || H < 0 || d <= 0 || dv <= 0 || p <= 0 || g < 1) return KATA_ERR_SHAPE;
  if (!valid_mode(mode)) return KATA_ERR_UNSUPPORTED;
  if (check_dtype(in_dtype) != KATA_OK || check_dtype(out_dtype) != KATA_OK) return KATA_ERR_UNSUPPORTED;
  if (g == 1) return kata_decode_step(N, H, d, dv, p, in_dtype, out_dtype, S, z, q, k, v, P, y, stream);
  if (g > kMaxFactors) return KATA_ERR_UNSUPPORTED;
  if (p != P_DIM || !((d == 16 && dv == 16) || (d == 64 && dv == 64))) return KATA_ERR_UNSUPPORTED;
  if (check_dtype(in_dtype) != KATA_OK || check_dtype(out_dtype) != KATA_OK) return KATA_ERR_UNSUPPORTED;
  if (N > 0 && H > 0x7fffffff / N) return KATA_ERR_SHAPE;
  if (N * H == 0) return KATA_OK;
  if (!S || !z || !q || !k || !v || !P || !y) return KATA_ERR_NULL;
  hipStream_t st = (hipStream_t)stream;
  const bool sum = mode == KATA_FACTORS_SUM;
  if (g == 2)
    return sum ? launch_decode_factors<2, true>(N * H, (int)H, d, dv, in_dtype, out_dtype, S, z, q, k, v, P, y, st)
               : launch_decode_factors<2, false>(N * H, (int)H, d, dv, in_dtype, out_dtype, S, z, q, k, v, P, y, st);
  return sum ? launch_decode_factors<3, true>(N * H, (int)H, d, dv, in_dtype, out_dtype, S, z, q, k, v, P, y, st)
             : launch_decode_factors<3, false>(N * H, (int)H, d, dv, in_dtype, out_dtype, S, z, q, k, v, P, y, st);
}

kata_status kata_feature_map(const void* x, const float* P, int64_t n, int64_t H, int d, int p,
                             kata_feature_layout layout, kata_dtype dtype, float* phi, void* stream) {
  if (n < 0 || H < 0 || d <= 0 || p <= 0) return KATA_ERR_SHAPE;
  if (p != P_DIM || !(d == 16 || d == 64)) return KATA_ERR_UNSUPPORTED;
  if (check_dtype(dtype) != KATA_OK) return KATA_ERR_UNSUPPORTED;
  const int lv = bits(layout);
  if (lv != KATA_FEATURE_FULL && lv != KATA_FEATURE_PACKED_KEY && lv != KATA_FEATURE_PACKED_QUERY)
    return KATA_ERR_UNSUPPORTED;
  if (n * H == 0) return KATA_OK;
  if (n * H > 0x7fffffff) return KATA_ERR_SHAPE;
  if (!x || !P || !phi) return KATA_ERR_NULL;
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid((unsigned)(n * H));
  if (dtype == KATA_F32)
    hipLaunchKernelGGL(kata::kata_feature<float>, grid, dim3(256), 0, st, (const float*)x, P, phi, (int)H, d, (int)layout);
  else
    hipLaunchKernelGGL(kata::kata_feature<bf16>, grid, dim3(256), 0, st, (const bf16*)x, P, phi, (int)H, d, (int)layout);
  return launch_status();
}

}  // extern "C"
