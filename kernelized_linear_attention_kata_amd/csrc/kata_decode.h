// kata_decode.h - kata_decode_step (recurrent constant-time step) and the debug
// feature map kernel.
//
// Recurrent form of normalised linear attention with a fixed-size state: the
// gist.science summary of "Kernelized Linear Attention" (arXiv 2607.17419), section 1,
// and the paper's abstract ("constant-time recurrent inference").  Rank-one PSD
// feature phi(x) = vec((Px)(Px)^T): same summary, section 2.2.
//
// One workgroup (256 threads) per (stream, head).  The 256 x dv fp32 state is
// streamed once in and once out with 16-byte accesses that cover contiguous 1 KB
// per wavefront instruction; the readout partial sums are reduced with lane
// shuffles and LDS.  The work is bound by HBM bandwidth (~0.5 flop per byte).
#pragma once

#include "kata_common.h"

namespace kata {

// u = P x for one vector: 256 threads, thread t computes the partial dot product of
// row a = t/16 over the d/16 input columns j = (t%16) + 16 i, then 16-lane reduction.
template <typename TIn>
__device__ __forceinline__ float project_row(const TIn* __restrict__ x, const float* __restrict__ Ph, int d, int tid) {
  const int a = tid >> 4, j0 = tid & 15;
  float s = 0.f;
  for (int j = j0; j < d; j += 16) s += Ph[a * d + j] * (float)x[j];
  s += __shfl_xor(s, 8);
  s += __shfl_xor(s, 4);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 1);
  return s;   // valid in every lane of the 16-lane group of row a
}

// grid N*H, block 256.  dv in {16, 64}: each thread owns one 4-column quad.  DECAY: the
// state is first multiplied by gamma = exp(lam[stream, head]) (decay-gated state:
// S <- gamma S + phi(k) v^T, z <- gamma z + phi(k)).
template <typename TIn, typename TOut, int DV, bool DECAY = false>
__global__ void __launch_bounds__(256)
kata_decode_step(float* __restrict__ S, float* __restrict__ z, const TIn* __restrict__ q,
                 const TIn* __restrict__ k, const TIn* __restrict__ v, const float* __restrict__ P,
                 TOut* __restrict__ y, int H, int d, const float* __restrict__ lam) {
  constexpr int D = P_DIM * P_DIM;
  constexpr int QPR = DV / 4;               // float4 quads per state row
  constexpr int ROWS_PER_IT = 256 / QPR;    // rows covered per pass of the block
  constexpr int NIT = D / ROWS_PER_IT;
  __shared__ float su[P_DIM], sw[P_DIM];
  __shared__ float fu[D], fw[D];
  __shared__ float red[4][DV];
  __shared__ float dred[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nh = blockIdx.x;
  const int h = (int)(nh % H);
  const float* Ph = P + (int64_t)h * P_DIM * d;
  float gam = 1.f;
  if constexpr (DECAY) gam = __expf(lam[nh]);

  const float u = project_row<TIn>(q + nh * d, Ph, d, tid);
  const float w = project_row<TIn>(k + nh * d, Ph, d, tid);
  if ((tid & 15) == 0) { su[tid >> 4] = u; sw[tid >> 4] = w; }
  __syncthreads();
  {
    const int a = tid >> 4, b = tid & 15;
    fu[tid] = su[a] * su[b];
    fw[tid] = sw[a] * sw[b];
  }
  __syncthreads();

  const int c4 = tid % QPR;
  f32x4 vv;
#pragma unroll
  for (int i = 0; i < 4; ++i) vv[i] = (float)v[nh * DV + 4 * c4 + i];
  float* Sh = S + nh * (int64_t)D * DV;
  f32x4 acc = zero4();
#pragma unroll 4
  for (int it = 0; it < NIT; ++it) {
    const int row = it * ROWS_PER_IT + tid / QPR;
    f32x4* p = reinterpret_cast<f32x4*>(Sh + row * DV + 4 * c4);
    f32x4 s = *p;
    const float fwr = fw[row], fur = fu[row];
    if constexpr (DECAY) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = gam * s[i] + fwr * vv[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] += fwr * vv[i];
    }
    *p = s;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += fur * s[i];
  }
  // z (one feature per thread) and the denominator
  float* zh = z + nh * D;
  const float zn = DECAY ? gam * zh[tid] + fw[tid] : zh[tid] + fw[tid];
  zh[tid] = zn;
  float dp = fu[tid] * zn;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) dp += __shfl_xor(dp, off);
  // reduce acc over threads sharing the quad c4 (lanes equal mod QPR)
#pragma unroll
  for (int off = 32; off >= QPR; off >>= 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += __shfl_xor(acc[i], off);
  }
  if (lane < QPR) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][4 * lane + i] = acc[i];
  }
  if (lane == 0) dred[wave] = dp;
  __syncthreads();
  if (tid < DV) {
    const float num = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
    const float den = dred[0] + dred[1] + dred[2] + dred[3];
    Elem<TOut>::store(y, nh * DV + tid, den != 0.f ? num / den : 0.f);
  }
}

// ---- packed state ------------------------------------------------------------------
// Every update adds phi(k) = vec(w w^T), a symmetric 16 x 16 matrix, so a state built by
// the steps (or exported by kata_forward) has equal mirror rows (a, b) and (b, a), and
// every read phi(q) . S sees only their sum.  The packed layout keeps one row per pair
// {a, b}, in the circulant order of the chunked kernels: row 16 delta + a (delta = 0..7,
// a = 0..15) and row 128 + a (delta = 8, a = 0..7) stand for the pair {a, (a + delta) mod 16}:
// 136 rows instead of 256, so a step moves 1.88x fewer bytes.
constexpr int DPK = 136;
__host__ __device__ constexpr int packed_delta(int r) { return r < 128 ? r >> 4 : 8; }
__host__ __device__ constexpr int packed_a(int r) { return r < 128 ? r & 15 : r - 128; }

// grid N*H, block 256.  The packed step: Sp += phi_p(k) v^T, zp += phi_p(k) with
// phi_p(k)[r] = w_a w_b, then y = sum_r c_r phi_p(q)[r] Sp[r] / sum_r c_r phi_p(q)[r] zp[r]
// with c_r = 1 on the diagonal (delta = 0) and 2 off it (each pair stands for two mirror
// rows of the canonical state).  Equal to kata_decode_step on the canonical state.
// DECAY: the state is first multiplied by gamma = exp(lam[stream, head]), as in
// kata_decode_step<..., DECAY>.  G > 1 (P [H, G, p, d]): KATA-Mg (G packed blocks,
// factor-major, each updated by its factor's feature) or SUMG (KATA-Sigma-g: one packed
// block, the features summed over the factors), as in kata_decode_step_factors.
template <typename TIn, typename TOut, int DV, int G = 1, bool SUMG = false, bool DECAY = false>
__global__ void __launch_bounds__(256)
kata_decode_step_packed(float* __restrict__ S, float* __restrict__ z, const TIn* __restrict__ q,
                        const TIn* __restrict__ k, const TIn* __restrict__ v, const float* __restrict__ P,
                        TOut* __restrict__ y, int H, int d, const float* __restrict__ lam) {
  static_assert(!(DECAY && G > 1), "decay gates with one PSD factor only");
  constexpr int NF = SUMG ? 1 : G;          // packed state blocks
  constexpr int ROWS = NF * DPK;
  constexpr int QPR = DV / 4;               // float4 quads per state row
  constexpr int ROWS_PER_IT = 256 / QPR;    // rows covered per pass of the block
  constexpr int NIT = (ROWS + ROWS_PER_IT - 1) / ROWS_PER_IT;
  __shared__ float su[G][P_DIM], sw[G][P_DIM];
  __shared__ float fu[ROWS], fw[ROWS];
  __shared__ float red[4][DV];
  __shared__ float dred[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nh = blockIdx.x;
  const int h = (int)(nh % H);
  float gam = 1.f;
  if constexpr (DECAY) gam = __expf(lam[nh]);
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const float* Ph = P + ((int64_t)h * G + i) * P_DIM * d;
    const float u = project_row<TIn>(q + nh * d, Ph, d, tid);
    const float w = project_row<TIn>(k + nh * d, Ph, d, tid);
    if ((tid & 15) == 0) {
      su[i][tid >> 4] = u;
      sw[i][tid >> 4] = w;
    }
  }
  __syncthreads();
  for (int r = tid; r < ROWS; r += 256) {
    const int blk = r / DPK, rr = r - blk * DPK;
    const int dl = packed_delta(rr), a = packed_a(rr), b = (a + dl) & 15;
    float xu = 0.f, xw = 0.f;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if (SUMG || i == blk) {
        xu += su[i][a] * su[i][b];
        xw += sw[i][a] * sw[i][b];
      }
    }
    fu[r] = (dl == 0 ? 1.f : 2.f) * xu;
    fw[r] = xw;
  }
  __syncthreads();

  const int c4 = tid % QPR;
  f32x4 vv;
#pragma unroll
  for (int i = 0; i < 4; ++i) vv[i] = (float)v[nh * DV + 4 * c4 + i];
  float* Sh = S + nh * (int64_t)ROWS * DV;
  f32x4 acc = zero4();
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int row = it * ROWS_PER_IT + tid / QPR;
    if (row < ROWS) {
      f32x4* ptr = reinterpret_cast<f32x4*>(Sh + row * DV + 4 * c4);
      f32x4 sv = *ptr;
      const float fwr = fw[row], fur = fu[row];
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[i] = (DECAY ? gam * sv[i] : sv[i]) + fwr * vv[i];
      *ptr = sv;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += fur * sv[i];
    }
  }
  float dp = 0.f;
  float* zh = z + nh * (int64_t)ROWS;
  for (int r = tid; r < ROWS; r += 256) {
    const float zn = (DECAY ? gam * zh[r] : zh[r]) + fw[r];
    zh[r] = zn;
    dp += fu[r] * zn;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) dp += __shfl_xor(dp, off);
#pragma unroll
  for (int off = 32; off >= QPR; off >>= 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += __shfl_xor(acc[i], off);
  }
  if (lane < QPR) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][4 * lane + i] = acc[i];
  }
  if (lane == 0) dred[wave] = dp;
  __syncthreads();
  if (tid < DV) {
    const float num = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
    const float den = dred[0] + dred[1] + dred[2] + dred[3];
    Elem<TOut>::store(y, nh * DV + tid, den != 0.f ? num / den : 0.f);
  }
}

// grid n*DPK, block 64 (thread c: value column c < dv).  Canonical -> packed: row r of
// the pair {a, b} takes (S[16a + b] + S[16b + a]) / 2 (exact when the mirror rows are
// equal, as they are for every state the steps or kata_forward produce); z likewise.
__global__ void __launch_bounds__(64)
kata_state_pack(const float* __restrict__ S, const float* __restrict__ z, float* __restrict__ Sp,
                float* __restrict__ zp, int dv) {
  const int r = (int)(blockIdx.x % DPK), c = threadIdx.x;
  const int64_t n = blockIdx.x / DPK;
  const int dl = packed_delta(r), a = packed_a(r), b = (a + dl) & 15;
  const int64_t f1 = 16 * a + b, f2 = 16 * b + a;
  const float* Sn = S + n * (int64_t)(P_DIM * P_DIM) * dv;
  if (c < dv) Sp[(n * DPK + r) * dv + c] = 0.5f * (Sn[f1 * dv + c] + Sn[f2 * dv + c]);
  if (z && c == 0) zp[n * DPK + r] = 0.5f * (z[n * (P_DIM * P_DIM) + f1] + z[n * (P_DIM * P_DIM) + f2]);
}

// grid n*256, block 64.  Packed -> canonical: both mirror rows (a, b) and (b, a) take the
// pair's row.
__global__ void __launch_bounds__(64)
kata_state_unpack(const float* __restrict__ Sp, const float* __restrict__ zp, float* __restrict__ S,
                  float* __restrict__ z, int dv) {
  const int f = (int)(blockIdx.x & 255), c = threadIdx.x;
  const int64_t n = blockIdx.x >> 8;
  const int a = f >> 4, b = f & 15;
  const int dab = (b - a) & 15;
  // the pair's row: distance dab <= 8 from a (for 8, a < 8 holds the pair), else from b
  int r;
  if (dab <= 7) r = 16 * dab + a;
  else if (dab == 8) r = 128 + (a & 7);
  else r = 16 * (16 - dab) + b;
  if (c < dv) S[(n * (P_DIM * P_DIM) + f) * dv + c] = Sp[(n * DPK + r) * dv + c];
  if (z && c == 0) z[n * (P_DIM * P_DIM) + f] = zp[n * DPK + r];
}

// One decode step of KATA-Mg (several concatenated PSD factors) or KATA-Sigma-g (summed
// factors): the item "Variantes" of section 2.3 of the gist.science summary, read as the
// forward's kata_forward_factors reads it.  grid N*H, block 256.  P [H, G, p, d].
//  * concat: state S [N,H,G*256,dv], z [N,H,G*256], factor-major; every factor's feature
//    updates its own block and the read-out sums over the blocks (one division);
//  * SUMG: state [N,H,256,dv]; the features are summed over the factors first, then the
//    step is the one-factor one.
// The state is streamed once in and once out, as in kata_decode_step.
template <typename TIn, typename TOut, int DV, int G, bool SUMG>
__global__ void __launch_bounds__(256)
kata_decode_step_factors(float* __restrict__ S, float* __restrict__ z, const TIn* __restrict__ q,
                         const TIn* __restrict__ k, const TIn* __restrict__ v, const float* __restrict__ P,
                         TOut* __restrict__ y, int H, int d) {
  constexpr int D = P_DIM * P_DIM;
  constexpr int NF = SUMG ? 1 : G;          // feature (and state) blocks
  constexpr int QPR = DV / 4;
  constexpr int ROWS_PER_IT = 256 / QPR;
  constexpr int NIT = D / ROWS_PER_IT;
  __shared__ float su[G][P_DIM], sw[G][P_DIM];
  __shared__ float fu[NF][D], fw[NF][D];
  __shared__ float red[4][DV];
  __shared__ float dred[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nh = blockIdx.x;
  const int h = (int)(nh % H);
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const float* Ph = P + ((int64_t)h * G + i) * P_DIM * d;
    const float u = project_row<TIn>(q + nh * d, Ph, d, tid);
    const float w = project_row<TIn>(k + nh * d, Ph, d, tid);
    if ((tid & 15) == 0) {
      su[i][tid >> 4] = u;
      sw[i][tid >> 4] = w;
    }
  }
  __syncthreads();
  {
    const int a = tid >> 4, b = tid & 15;
    if constexpr (SUMG) {
      float xu = 0.f, xw = 0.f;
#pragma unroll
      for (int i = 0; i < G; ++i) {
        xu += su[i][a] * su[i][b];
        xw += sw[i][a] * sw[i][b];
      }
      fu[0][tid] = xu;
      fw[0][tid] = xw;
    } else {
#pragma unroll
      for (int i = 0; i < G; ++i) {
        fu[i][tid] = su[i][a] * su[i][b];
        fw[i][tid] = sw[i][a] * sw[i][b];
      }
    }
  }
  __syncthreads();

  const int c4 = tid % QPR;
  f32x4 vv;
#pragma unroll
  for (int i = 0; i < 4; ++i) vv[i] = (float)v[nh * DV + 4 * c4 + i];
  float* Sh = S + nh * (int64_t)(NF * D) * DV;
  f32x4 acc = zero4();
#pragma unroll
  for (int f = 0; f < NF; ++f) {
#pragma unroll 4
    for (int it = 0; it < NIT; ++it) {
      const int row = it * ROWS_PER_IT + tid / QPR;
      f32x4* p = reinterpret_cast<f32x4*>(Sh + (f * D + row) * DV + 4 * c4);
      f32x4 s = *p;
      const float fwr = fw[f][row], fur = fu[f][row];
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] += fwr * vv[i];
      *p = s;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += fur * s[i];
    }
  }
  float* zh = z + nh * (int64_t)(NF * D);
  float dp = 0.f;
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const float zn = zh[f * D + tid] + fw[f][tid];
    zh[f * D + tid] = zn;
    dp += fu[f][tid] * zn;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) dp += __shfl_xor(dp, off);
#pragma unroll
  for (int off = 32; off >= QPR; off >>= 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += __shfl_xor(acc[i], off);
  }
  if (lane < QPR) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][4 * lane + i] = acc[i];
  }
  if (lane == 0) dred[wave] = dp;
  __syncthreads();
  if (tid < DV) {
    const float num = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
    const float den = dred[0] + dred[1] + dred[2] + dred[3];
    Elem<TOut>::store(y, nh * DV + tid, den != 0.f ? num / den : 0.f);
  }
}

// Debug feature map: grid n*H, block 256.  layout 0 = full (256), 1 = packed key
// side (144), 2 = packed query side (144).
template <typename TIn>
__global__ void __launch_bounds__(256)
kata_feature(const TIn* __restrict__ x, const float* __restrict__ P, float* __restrict__ phi,
             int H, int d, int layout) {
  __shared__ float su[P_DIM];
  const int tid = threadIdx.x;
  const int64_t vi = blockIdx.x;
  const int h = (int)(vi % H);
  const float u = project_row<TIn>(x + vi * d, P + (int64_t)h * P_DIM * d, d, tid);
  if ((tid & 15) == 0) su[tid >> 4] = u;
  __syncthreads();
  if (layout == 0) {
    phi[vi * 256 + tid] = su[tid >> 4] * su[tid & 15];
  } else if (tid < DPACK) {
    const int delta = tid >> 4, a = tid & 15, b = (a + delta) & 15;
    const float wgt = layout == 2 ? query_weight(delta, a) : key_weight(delta, a);
    phi[vi * DPACK + tid] = wgt * su[a] * su[b];
  }
}

}  // namespace kata
