// kata_delta.h - DeltaKATA: the delta rule over KATA's rank-one PSD feature.
//
// The gist.science summary of "Kernelized Linear Attention" (arXiv 2607.17419) names
// DeltaKATA, the delta-rule variant that corrects stale bindings when a key is written
// again (section 4, repeated-key overwrite; section 1 on content-directed erasure), and
// the abstract lists delta rules among the mechanisms studied with KATA's features.
// Neither defines it.  The reading implemented: DeltaNet's delta rule with KATA's
// feature normalised to unit norm,
//
//   phi^(x) = vec(u u^T) / |u|^2,  u = P x       (|phi^(x)| = 1; 0 where u = 0)
//   S_t = S_{t-1} + beta_t phi^(k_t) (v_t - S_{t-1}^T phi^(k_t))^T
//   y_t = S_t^T phi^(q_t)                         (no denominator)
//
// One workgroup (256 threads) per (sequence, head) walks the tokens with the whole
// 256 x dv fp32 state in registers: thread t owns the float4 column quad c4 = t % (dv/4)
// of the rows it * (1024/dv) + t / (dv/4).  Per token: the projections u, w (each
// thread one partial row of P . x held in registers, 16-lane reduction), then the two
// state read-outs S^T phi^(k) and S^T phi^(q) (lane shuffles, then LDS across the four
// waves), the error e = v - S^T phi^(k), the rank-one update and
//   y = S^T phi^(q) + beta (phi^(q) . phi^(k)) e,  phi^(q) . phi^(k) = (u.w)^2 / (|u|^2 |w|^2).
// Two barriers per token; the LDS words of consecutive tokens alternate between two
// buffers so no third barrier is needed.  The state is read once and written once.
#pragma once

#include "kata_common.h"

namespace kata {

template <int DV>
struct DeltaLayout {
  static constexpr int D = P_DIM * P_DIM;
  static constexpr int QPR = DV / 4;     // float4 quads per state row
  static constexpr int RPI = 256 / QPR;  // rows covered by the block per register quad
  static constexpr int NIT = D / RPI;    // register quads per thread
  static_assert(DV == 16 || DV == 64, "dv 16 or 64");
};

// grid B*H, block 256.  S0 (nullable) is read before anything is written and ST
// (nullable) written at the end, so S0 == ST (an in-place decode step) is allowed.
// q, k [B*H, T, d]; v [B*H, T, DV]; beta [B*H, T]; y [B*H, T, DV].
template <typename TIn, typename TOut, int DV>
__global__ void __launch_bounds__(256)
kata_delta_recurrent(const float* S0, float* ST, const TIn* __restrict__ q, const TIn* __restrict__ k,
                     const TIn* __restrict__ v, const float* __restrict__ beta, const float* __restrict__ P,
                     TOut* __restrict__ y, int H, int d, int64_t T) {
  using L = DeltaLayout<DV>;
  __shared__ __align__(16) float su[2][P_DIM];
  __shared__ __align__(16) float sw[2][P_DIM];
  __shared__ __align__(16) float red[2][2][4][DV];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t bh = blockIdx.x;
  const int h = (int)(bh % H);
  const int c4 = tid % L::QPR, r0 = tid / L::QPR;
  // this thread's share of the projection: row pa of P, columns pj + 16 i (d <= 64)
  const int pa = tid >> 4, pj = tid & 15;
  const int nj = d >> 4;
  float pr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pr[i] = i < nj ? P[((int64_t)h * P_DIM + pa) * d + pj + 16 * i] : 0.f;

  f32x4 s[L::NIT];
  const int64_t sbase = bh * (int64_t)L::D * DV;
#pragma unroll
  for (int it = 0; it < L::NIT; ++it) {
    const int row = it * L::RPI + r0;
    s[it] = S0 ? *reinterpret_cast<const f32x4*>(S0 + sbase + row * DV + 4 * c4) : zero4();
  }

  for (int64_t t = 0; t < T; ++t) {
    const int buf = (int)(t & 1);
    const int64_t tok = bh * T + t;
    const TIn* qt = q + tok * d;
    const TIn* kt = k + tok * d;
    float pu = 0.f, pw = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < nj) {
        pu += pr[i] * Elem<TIn>::load(qt, pj + 16 * i);
        pw += pr[i] * Elem<TIn>::load(kt, pj + 16 * i);
      }
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) {
      pu += __shfl_xor(pu, off);
      pw += __shfl_xor(pw, off);
    }
    if (pj == 0) {
      su[buf][pa] = pu;
      sw[buf][pa] = pw;
    }
    f32x4 vq;
#pragma unroll
    for (int i = 0; i < 4; ++i) vq[i] = Elem<TIn>::load(v, tok * DV + 4 * c4 + i);
    const float bt = beta[tok];
    __syncthreads();

    float nu = 0.f, nw = 0.f, uw = 0.f;
#pragma unroll
    for (int a4 = 0; a4 < P_DIM / 4; ++a4) {
      const f32x4 ua = *reinterpret_cast<const f32x4*>(&su[buf][4 * a4]);
      const f32x4 wa = *reinterpret_cast<const f32x4*>(&sw[buf][4 * a4]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        nu += ua[i] * ua[i];
        nw += wa[i] * wa[i];
        uw += ua[i] * wa[i];
      }
    }
    const float iu = nu > 0.f ? 1.f / nu : 0.f;
    const float iw = nw > 0.f ? 1.f / nw : 0.f;
    float fk[L::NIT];
    f32x4 ak = zero4(), aq = zero4();
#pragma unroll
    for (int it = 0; it < L::NIT; ++it) {
      const int row = it * L::RPI + r0;
      const int a = row >> 4, b = row & 15;
      fk[it] = sw[buf][a] * sw[buf][b] * iw;
      const float fq = su[buf][a] * su[buf][b] * iu;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ak[i] += fk[it] * s[it][i];
        aq[i] += fq * s[it][i];
      }
    }
    // sum over the lanes of this wave that own the same column quad
#pragma unroll
    for (int off = 32; off >= L::QPR; off >>= 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ak[i] += __shfl_xor(ak[i], off);
        aq[i] += __shfl_xor(aq[i], off);
      }
    }
    if (lane < L::QPR) {
      *reinterpret_cast<f32x4*>(&red[buf][0][wave][4 * lane]) = ak;
      *reinterpret_cast<f32x4*>(&red[buf][1][wave][4 * lane]) = aq;
    }
    __syncthreads();

    f32x4 e;
    {
      const f32x4 k0 = *reinterpret_cast<const f32x4*>(&red[buf][0][0][4 * c4]);
      const f32x4 k1 = *reinterpret_cast<const f32x4*>(&red[buf][0][1][4 * c4]);
      const f32x4 k2 = *reinterpret_cast<const f32x4*>(&red[buf][0][2][4 * c4]);
      const f32x4 k3 = *reinterpret_cast<const f32x4*>(&red[buf][0][3][4 * c4]);
#pragma unroll
      for (int i = 0; i < 4; ++i) e[i] = bt * (vq[i] - ((k0[i] + k1[i]) + (k2[i] + k3[i])));
    }
#pragma unroll
    for (int it = 0; it < L::NIT; ++it) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s[it][i] += fk[it] * e[i];
    }
    if (tid < DV) {
      const float kv = (red[buf][0][0][tid] + red[buf][0][1][tid]) + (red[buf][0][2][tid] + red[buf][0][3][tid]);
      const float qv = (red[buf][1][0][tid] + red[buf][1][1][tid]) + (red[buf][1][2][tid] + red[buf][1][3][tid]);
      const float c2 = uw * uw * iu * iw;
      const float vt = Elem<TIn>::load(v, tok * DV + tid);
      Elem<TOut>::store(y, tok * DV + tid, qv + bt * c2 * (vt - kv));
    }
  }

  if (ST) {
#pragma unroll
    for (int it = 0; it < L::NIT; ++it) {
      const int row = it * L::RPI + r0;
      *reinterpret_cast<f32x4*>(ST + sbase + row * DV + 4 * c4) = s[it];
    }
  }
}

}  // namespace kata
