// kata_scan.h - kata_state_scan: exclusive associative prefix of the per-leaf chunk
// states, in place, plus the inclusive total exported as the final state.
//
// The hardware section of the gist.science summary of "Kernelized Linear Attention"
// (arXiv 2607.17419, section 2.3) and the paper's abstract give the inter-chunk state
// propagation as an associative scan (a parallel prefix sum, log depth in T/C) in place
// of the chunk-after-chunk recurrence.  The combine operator on states [S | z] is
// elementwise addition.  What ships is a reduce-then-scan over leaves of L chunks: the
// leaf sums (kata_chunk_state) get their exclusive prefix here by a segmented scan (up
// to 16 rows summed in order per thread, up to 16 segment totals combined through LDS,
// passes of 256 leaves chained by a carry), and the pass that forms the outputs
// completes each chunk's prefix inside its leaf with a running sum.  Sequential depth:
// L chunk steps plus at most 32 combine steps per 256 leaves, i.e. O(L + n_leaf/16), not
// O(log(T/C)); at the leaf counts the library picks (tens per sequence) a log-depth
// combine of the leaf sums measured 1.5x slower than this one.
//
// Layout: ws[bh][leaf][e], e < E = 144*dv + 256 (packed S then Z, see kata_chunk.h).
// The exclusive prefix written for leaf g is S0 + sum_{g' < g} state_g' (or the suffix
// sum over g' > g in reverse mode).
#pragma once

#include "kata_common.h"

namespace kata {

// Element e of a leaf block -> canonical feature pair (a, b), value column and
// whether it is a z entry.  S part: packed slot (delta, a) in accumulator-tile order,
// pair (a, (a + delta) mod 16), stored once for both mirror entries (mirror = true
// when a != b).  z part: the 16 x 16 matrix Z in accumulator-tile order (lane
// (b, g) holds Z[4g + r][b]), every entry its own (mirror = false).  Returns false
// for the unused packed slots (delta = 8, a >= 8).
__device__ __forceinline__ bool packed_to_pair(int e, int dv, int& a, int& b, int& col, bool& is_z,
                                               bool& mirror) {
  const int nb_count = dv / 16;
  if (e < DPACK * dv) {
    const int tau = e >> 8, w = e & 255;
    const int l = w >> 2, r = w & 3;
    const int n = l & 15, g = l >> 4;
    const int delta = tau / nb_count;
    const int nb = tau % nb_count;
    a = 4 * g + r;
    col = 16 * nb + n;
    is_z = false;
    if (delta == 8 && a >= 8) return false;
    b = (a + delta) & 15;
    mirror = a != b;
    return true;
  }
  const int ez = e - DPACK * dv;
  const int l = ez >> 2, r = ez & 3;
  b = l & 15;
  a = 4 * (l >> 4) + r;
  col = 0;
  is_z = true;
  mirror = false;
  return true;
}

// One thread per 16-byte column quad (4 consecutive elements e) and per segment of
// leaf rows: a workgroup holds QW = 256/G quads x G segments.  A pass covers G*Lseg
// rows: segment s takes rows [s*Lseg, (s+1)*Lseg) of the pass, keeps them in
// registers, and forms its total; the totals of the segments of a quad are combined
// through LDS (segment s adds those of segments < s to the quad's running carry), and
// each thread then writes the exclusive prefix of its rows in order.  Passes chain by
// the carry.  Every element is read and written once, and each wavefront instruction
// moves 1 KB (QW >= 64) or 16-byte pieces of QW consecutive quads, contiguous in the
// leaf row.  Depth: Lseg sequential steps per pass plus the combination of G segments.
constexpr int SCAN_ROWS = 16;    // rows per segment and pass (registers)
constexpr int SCAN_GMAX = 16;    // segments per quad

// Canonical initial value of element e, 0 for none: the mean of the two mirror entries of
// S0 / z0 (i.e. the symmetric part of the caller's state, or of a gradient with respect to
// a state; only the symmetric part acts on the symmetric feature).  For the symmetric
// states this library produces the mean is the entry itself, bit for bit.
__device__ __forceinline__ float scan_initial(int e, int dv, int64_t bh, const float* S0, const float* z0) {
  int a, b, col;
  bool is_z, mirror;
  if (!packed_to_pair(e, dv, a, b, col, is_z, mirror)) return 0.f;
  const int64_t pp = (int64_t)P_DIM * P_DIM;
  if (!is_z) {
    if (!S0) return 0.f;
    return 0.5f * (S0[(bh * pp + a * P_DIM + b) * dv + col] + S0[(bh * pp + b * P_DIM + a) * dv + col]);
  }
  if (!z0) return 0.f;
  return 0.5f * (z0[bh * pp + a * P_DIM + b] + z0[bh * pp + b * P_DIM + a]);
}

// grid (ceil((E/4) / (256/G)), B*H), block 256.  E is a multiple of 4.  reverse = 1
// scans the leaves from the last to the first (an exclusive suffix: leaf g receives
// init + sum_{g' > g} state_g'), as the backward pass needs; init as in scan_initial.
//
// dec (decay-gated state, may be NULL): dec[bh * n_leaf + g] is the total decay D_g of leaf
// g, and the combine becomes affine: the prefix entering leaf g + 1 is D_g * (prefix
// entering leaf g) + state_g; a segment's total carries the product of its leaves' D.
__global__ void __launch_bounds__(256)
kata_state_scan(float* __restrict__ ws, int64_t n_leaf, int E, int dv, int G,
                const float* __restrict__ S0, const float* __restrict__ z0,
                float* __restrict__ ST, float* __restrict__ zT, int reverse, const float* __restrict__ dec) {
  __shared__ f32x4 tot[256];
  __shared__ f32x4 carry_s[256];
  __shared__ float dseg[SCAN_GMAX];
  const int tid = threadIdx.x;
  const int QW = 256 / G;
  const int ql = tid % QW, seg = tid / QW;
  const int64_t bh = blockIdx.y;
  const int e0 = (blockIdx.x * QW + ql) * 4;
  // The quads of the unused packed slots (delta = 8, a >= 8: lanes 32..63 of the delta = 8
  // tiles) are read with query weight 0 by the forward kernels, which is all they are
  // used for, so the forward scan leaves them as the state pass wrote them (finite leaf
  // sums); the reverse scan of the backward does them all.
  const bool unused = !reverse && e0 < DPACK * dv && (e0 >> 8) >= 8 * (dv / 16) && (e0 & 255) >= 128;
  const bool active = e0 < E && !unused;
  float* base = ws + bh * n_leaf * (int64_t)E + e0;
  const int64_t per_pass = (int64_t)SCAN_ROWS * G;
  const int lseg = (int)((n_leaf < per_pass ? n_leaf : per_pass) + G - 1) / G;
  auto row = [&](int64_t i) { return reverse ? n_leaf - 1 - i : i; };   // scan position -> leaf

  f32x4 carry = zero4();   // the quad's running carry, kept by segment 0
  if (seg == 0 && active) {
#pragma unroll
    for (int i = 0; i < 4; ++i) carry[i] = scan_initial(e0 + i, dv, bh, S0, z0);
  }
  const float* dl = dec ? dec + bh * n_leaf : nullptr;
  for (int64_t r0 = 0; r0 < n_leaf; r0 += (int64_t)lseg * G) {
    const int64_t rs = r0 + (int64_t)seg * lseg;
    f32x4 x[SCAN_ROWS];
    float dr[SCAN_ROWS];
    f32x4 tsum = zero4();
    float dprod = 1.f;
#pragma unroll
    for (int i = 0; i < SCAN_ROWS; ++i) {
      const bool in = i < lseg && rs + i < n_leaf;
      const bool ok = active && in;
      x[i] = ok ? *reinterpret_cast<const f32x4*>(base + row(rs + i) * E) : zero4();
      dr[i] = (dl && in) ? dl[row(rs + i)] : 1.f;
      tsum = dr[i] * tsum + x[i];
      dprod *= dr[i];
    }
    tot[tid] = tsum;
    if (ql == 0) dseg[seg] = dprod;
    if (seg == 0) carry_s[ql] = carry;
    __syncthreads();
    f32x4 c = carry_s[ql];
    for (int s2 = 0; s2 < seg; ++s2) c = dseg[s2] * c + tot[ql + s2 * QW];
#pragma unroll
    for (int i = 0; i < SCAN_ROWS; ++i) {
      if (active && i < lseg && rs + i < n_leaf) *reinterpret_cast<f32x4*>(base + row(rs + i) * E) = c;
      c = dr[i] * c + x[i];
    }
    if (seg == 0) {
      f32x4 nc = carry_s[ql];
      for (int s2 = 0; s2 < G; ++s2) nc = dseg[s2] * nc + tot[ql + s2 * QW];
      carry = nc;
    }
    __syncthreads();
  }

  // segment 0 now holds S0 + the sum of every leaf state: export it canonically
  if (seg == 0 && active && (ST || zT)) {
    const int64_t pp = (int64_t)P_DIM * P_DIM;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int a, b, col;
      bool is_z, mirror;
      if (!packed_to_pair(e0 + i, dv, a, b, col, is_z, mirror)) continue;
      const float val = carry[i];
      if (!is_z && ST) {
        ST[(bh * pp + a * P_DIM + b) * dv + col] = val;
        if (mirror) ST[(bh * pp + b * P_DIM + a) * dv + col] = val;
      }
      if (is_z && zT) zT[bh * pp + a * P_DIM + b] = val;
    }
  }
}

}  // namespace kata
