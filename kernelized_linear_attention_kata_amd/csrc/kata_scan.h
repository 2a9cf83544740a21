// kata_scan.h - kata_state_scan: exclusive associative prefix of the per-leaf chunk
// states, in place, plus the inclusive total exported as the final state.
//
// The hardware section of the gist.science summary of "Kernelized Linear Attention"
// (arXiv 2607.17419, section 2.3) and the paper's abstract state that the inter-chunk
// state propagation is an associative scan (parallel prefix sum) of depth
// O(log(T/C)).  The combine operator on states [S | z] is elementwise addition.
//
// Layout: ws[bh][leaf][e], e < E = 144*dv + 256 (packed S then Z, see kata_chunk.h).  One
// workgroup owns 32 consecutive elements e of one (b, h) and walks the leaves in
// passes of blockDim.x rows: lane = leaf row, so every lane moves 128 contiguous
// bytes per pass.  Within a pass the prefix across rows is a log-depth
// Hillis-Steele scan over the wavefront (DPP lane shifts, 6 levels) followed by a
// scan of the per-wave totals through LDS; passes are chained by a carry.  The
// exclusive prefix written for leaf g is S0 + sum_{g' < g} state_g'.
#pragma once

#include "kata_common.h"

namespace kata {

constexpr int SCAN_COLS = 32;

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

// Wavefront inclusive prefix sum by DPP (log depth, no LDS traffic): Hillis-Steele
// inside each 16-lane row with row_shr:1,2,4,8, then the row totals are carried
// with row_bcast:15 (row r-1's last lane into row r, rows 1 and 3) and
// row_bcast:31 (lane 31 into rows 2 and 3).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or_zero(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, true));
}
__device__ __forceinline__ float wave_inclusive_scan(float x) {
  x += dpp_or_zero<0x111, 0xf>(x);   // row_shr:1
  x += dpp_or_zero<0x112, 0xf>(x);   // row_shr:2
  x += dpp_or_zero<0x114, 0xf>(x);   // row_shr:4
  x += dpp_or_zero<0x118, 0xf>(x);   // row_shr:8
  x += dpp_or_zero<0x142, 0xa>(x);   // row_bcast:15
  x += dpp_or_zero<0x143, 0xc>(x);   // row_bcast:31
  return x;
}
// lane i receives lane i-1's value, lane 0 receives 0 (wave_shr:1)
__device__ __forceinline__ float wave_shift_up1(float x) { return dpp_or_zero<0x138, 0xf>(x); }

// grid (ceil(E/32), B*H), block = 64 * ceil(min(n_leaf, 256)/64) threads.
__global__ void __launch_bounds__(256)
kata_state_scan(float* __restrict__ ws, int64_t n_leaf, int E, int dv,
                const float* __restrict__ S0, const float* __restrict__ z0,
                float* __restrict__ ST, float* __restrict__ zT) {
  __shared__ float wtot[4][SCAN_COLS];
  __shared__ float carry[SCAN_COLS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nwaves = blockDim.x >> 6;
  const int64_t bh = blockIdx.y;
  const int e0 = blockIdx.x * SCAN_COLS;
  const int64_t pp = (int64_t)P_DIM * P_DIM;

  if (tid < SCAN_COLS) {
    float c0 = 0.f;
    const int e = e0 + tid;
    int a, b, col;
    bool is_z, mirror;
    if (e < E && packed_to_pair(e, dv, a, b, col, is_z, mirror)) {
      const int lo = a < b ? a : b, hi = a < b ? b : a;   // read the upper triangle
      if (!is_z && S0) c0 = S0[(bh * pp + lo * P_DIM + hi) * dv + col];
      if (is_z && z0) c0 = z0[bh * pp + lo * P_DIM + hi];
    }
    carry[tid] = c0;
  }
  __syncthreads();

  float* base = ws + bh * n_leaf * (int64_t)E;
  const bool full = (e0 + SCAN_COLS <= E);
  for (int64_t r0 = 0; r0 < n_leaf; r0 += blockDim.x) {
    const int64_t row = r0 + tid;
    const bool rok = row < n_leaf;
    float x[SCAN_COLS];
    float* rp = base + row * E + e0;
    if (rok && full) {
#pragma unroll
      for (int c = 0; c < SCAN_COLS; c += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(rp + c);
        x[c] = v[0]; x[c + 1] = v[1]; x[c + 2] = v[2]; x[c + 3] = v[3];
      }
    } else {
#pragma unroll
      for (int c = 0; c < SCAN_COLS; ++c) x[c] = (rok && e0 + c < E) ? rp[c] : 0.f;
    }
    float ex[SCAN_COLS];
#pragma unroll
    for (int c = 0; c < SCAN_COLS; ++c) {
      const float inc = wave_inclusive_scan(x[c]);
      ex[c] = wave_shift_up1(inc);
      if (lane == WAVE - 1) wtot[wave][c] = inc;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < SCAN_COLS; ++c) {
      float pre = carry[c];
      for (int w = 0; w < wave; ++w) pre += wtot[w][c];
      ex[c] += pre;
    }
    if (rok && full) {
#pragma unroll
      for (int c = 0; c < SCAN_COLS; c += 4)
        *reinterpret_cast<f32x4*>(rp + c) = f32x4{ex[c], ex[c + 1], ex[c + 2], ex[c + 3]};
    } else if (rok) {
#pragma unroll
      for (int c = 0; c < SCAN_COLS; ++c)
        if (e0 + c < E) rp[c] = ex[c];
    }
    __syncthreads();
    if (tid < SCAN_COLS) {
      float s = carry[tid];
      for (int w = 0; w < nwaves; ++w) s += wtot[w][tid];
      carry[tid] = s;
    }
    __syncthreads();
  }

  // carry now holds S0 + sum of every leaf state: export in the canonical layout
  if (tid < SCAN_COLS && (ST || zT)) {
    const int e = e0 + tid;
    int a, b, col;
    bool is_z, mirror;
    if (e < E && packed_to_pair(e, dv, a, b, col, is_z, mirror)) {
      const float val = carry[tid];
      if (!is_z && ST) {
        ST[(bh * pp + a * P_DIM + b) * dv + col] = val;
        if (mirror) ST[(bh * pp + b * P_DIM + a) * dv + col] = val;
      }
      if (is_z && zT) zT[bh * pp + a * P_DIM + b] = val;
    }
  }
}

}  // namespace kata
