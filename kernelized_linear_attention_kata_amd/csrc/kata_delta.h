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

#include "kata_chunk.h"   // kata_common.h, and row_plus (DPP row rotation)
#include "kata_decode.h"  // the packed state rows (DPK, packed_delta, packed_a)

namespace kata {

// PACKED: the state in the packed symmetric layout of kata_decode_step_packed (136 rows,
// one per pair {a, b}): every delta-rule update adds beta phi^(k) e^T with phi^(k)
// symmetric, and the reads S^T phi^(x) see only the sum of the mirror rows, so the step
// updates a pair's row with the unweighted feature and reads it with weight 2 off the
// diagonal.
template <int DV, bool PACKED = false>
struct DeltaLayout {
  static constexpr int D = PACKED ? DPK : P_DIM * P_DIM;
  static constexpr int QPR = DV / 4;     // float4 quads per state row
  static constexpr int RPI = 256 / QPR;  // rows covered by the block per register quad
  static constexpr int NIT = (D + RPI - 1) / RPI;   // register quads per thread (last one partial)
  static_assert(DV == 16 || DV == 64, "dv 16 or 64");
};

// grid B*H, block 256.  S0 (nullable) is read before anything is written and ST
// (nullable) written at the end, so S0 == ST (an in-place decode step) is allowed.
// q, k [B*H, T, d]; v [B*H, T, DV]; beta [B*H, T]; y [B*H, T, DV].
template <typename TIn, typename TOut, int DV, bool PACKED = false>
__global__ void __launch_bounds__(256)
kata_delta_recurrent(const float* S0, float* ST, const TIn* __restrict__ q, const TIn* __restrict__ k,
                     const TIn* __restrict__ v, const float* __restrict__ beta, const float* __restrict__ P,
                     TOut* __restrict__ y, int H, int d, int64_t T) {
  using L = DeltaLayout<DV, PACKED>;
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
    s[it] = (S0 && row < L::D) ? *reinterpret_cast<const f32x4*>(S0 + sbase + row * DV + 4 * c4) : zero4();
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
      int a, b;
      float c = 1.f;                   // read weight of the row
      if constexpr (PACKED) {
        const bool live = row < L::D;  // the rows past the packed state (last quad) read as zero
        const int dl = live ? packed_delta(row) : 0;
        a = live ? packed_a(row) : 0;
        b = (a + dl) & 15;
        c = live ? (dl == 0 ? 1.f : 2.f) : 0.f;
      } else {
        a = row >> 4;
        b = row & 15;
      }
      fk[it] = (PACKED && row >= L::D) ? 0.f : sw[buf][a] * sw[buf][b] * iw;
      const float fq = su[buf][a] * su[buf][b] * iu * c;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ak[i] += c * fk[it] * s[it][i];
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
      if (row < L::D) *reinterpret_cast<f32x4*>(ST + sbase + row * DV + 4 * c4) = s[it];
    }
  }
}

// ---- chunked DeltaKATA forward ----------------------------------------------------------
// The chunked form of the delta rule (the WY / UT form of chunked DeltaNet): with the
// chunk's unit key features K^ (C x 256), query features Q^, write strengths beta and
//   A = I + tril(diag(beta) K^ K^^T, -1),   T = A^{-1}      (unit lower triangular)
// the chunk's corrections are E = T diag(beta) (V - K^ S), and
//   Y = Q^ S + (Q^ K^^T o M) E   (M: s <= t),      S <- S + K^^T E.
// K^ K^^T and Q^ K^^T are cos^2 tiles of the 16-dim normalised projections, so the
// features are only built for the contractions with S.  T depends on the chunk's keys
// alone, so kata_delta_prep forms it (and the normalised projections) for all chunks in
// parallel; kata_delta_chunk then walks the chunks of one sequence in order.  The value
// columns of S are independent (E's column block j needs S's column block j only), so
// a sequence's walk is split over dv/16 workgroups, one per 16-column block.
constexpr int DC = 64;          // chunk length of the chunked delta forward

// One element through a range-checked buffer (0 past its end), as float.
template <typename TIn> __device__ __forceinline__ float buf_elem(__amdgpu_buffer_rsrc_t r, int idx);
template <> __device__ __forceinline__ float buf_elem<float>(__amdgpu_buffer_rsrc_t r, int idx) {
  return __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, idx * 4, 0, 0));
}
template <> __device__ __forceinline__ float buf_elem<bf16>(__amdgpu_buffer_rsrc_t r, int idx) {
  return bf16_bits_to_float((u16)__builtin_amdgcn_raw_buffer_load_b16(r, idx * 2, 0, 0));
}

// The raw bits of one element (0 past the buffer's end), and their value: a prefetch keeps
// the bits and converts them where they are used, so the load is not waited for at issue.
template <typename TIn> __device__ __forceinline__ uint32_t buf_bits(__amdgpu_buffer_rsrc_t r, int idx);
template <> __device__ __forceinline__ uint32_t buf_bits<float>(__amdgpu_buffer_rsrc_t r, int idx) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, idx * 4, 0, 0);
}
template <> __device__ __forceinline__ uint32_t buf_bits<bf16>(__amdgpu_buffer_rsrc_t r, int idx) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, idx * 2, 0, 0);
}
template <typename TIn> __device__ __forceinline__ float bits_value(uint32_t b) {
  return __uint_as_float(sizeof(TIn) == 2 ? b << 16 : b);
}

// grid (n_chunks, B*H), block 256.  Writes for every token of the chunk u^ = Pq/|Pq| and
// w^ = Pk/|Pk| (0 where the projection is 0, and past T) to Uo, Wo [B*H, n_chunks*64, 16],
// and T of the chunk to Tf [B*H, n_chunks, 4, 2, 64, 2, 8] bf16, already in the form the
// walk feeds the matrix cores: for query block mb, token K-block kk and lane (n, g), the 8
// entries T[16 mb + n][s] of the lane's K slots (permuted token order, see the walk) as
// hi and lo bf16 halves.  The first chunk's workgroup of each sequence also zeroes that
// sequence's progress counters prog[bh][d/16] for the walk (dv = d).
// Projection: the 4 threads of a token each take 16 input columns (two 16-byte loads of q
// and of k), form the partial dot products of all 16 rows of P (staged in LDS) and sum
// them with two lane shuffles.  Inversion: one column of T per lane of wave 0, the sum
// over s split into 4 interleaved partial sums to shorten the dependency chain.
template <typename TIn, int DIN>
__global__ void __launch_bounds__(256)
kata_delta_prep(const TIn* __restrict__ q, const TIn* __restrict__ k, const float* __restrict__ beta,
                const float* __restrict__ P, float* __restrict__ Uo, float* __restrict__ Wo,
                bf16* __restrict__ Tf, int* __restrict__ prog, int64_t T, int H) {
  constexpr int d = DIN;
  __shared__ __align__(16) float Ps[P_DIM][64 + 4];
  __shared__ __align__(16) float ws[DC][P_DIM];
  __shared__ __align__(16) float G[DC][DC + 4];
  __shared__ float bs[DC];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c = blockIdx.x, bh = blockIdx.y;
  const int h = (int)(bh % H);
  const int64_t n_chunks = gridDim.x;
  for (int i = tid; i < P_DIM * d; i += 256) Ps[i / d][i % d] = P[(int64_t)h * P_DIM * d + i];
  if (c == 0 && tid < DIN / 16) prog[bh * (DIN / 16) + tid] = 0;   // the walk's progress counters (dv = d)
  const int tl = tid >> 2, qq = tid & 3;           // token of the chunk, quarter of the columns
  const int64_t t = c * DC + tl;
  const bool live = t < T;
  constexpr int cw = d >> 2;                       // columns per quarter (16 or 4)
  float xq[16], xk[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    xq[i] = 0.f;
    xk[i] = 0.f;
  }
  if (live) {
    const TIn* qr = q + (bh * T + t) * d + qq * cw;
    const TIn* kr = k + (bh * T + t) * d + qq * cw;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i < cw) {
        xq[i] = Elem<TIn>::load(qr, i);
        xk[i] = Elem<TIn>::load(kr, i);
      }
    }
  }
  __syncthreads();   // P staged
  float u[P_DIM], w[P_DIM];
#pragma unroll
  for (int a = 0; a < P_DIM; ++a) {
    float su = 0.f, sw = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i < cw) {
        const float pv = Ps[a][qq * cw + i];
        su += pv * xq[i];
        sw += pv * xk[i];
      }
    }
    su += __shfl_xor(su, 1); su += __shfl_xor(su, 2);
    sw += __shfl_xor(sw, 1); sw += __shfl_xor(sw, 2);
    u[a] = su;
    w[a] = sw;
  }
  float nu = 0.f, nw = 0.f;
#pragma unroll
  for (int a = 0; a < P_DIM; ++a) {
    nu += u[a] * u[a];
    nw += w[a] * w[a];
  }
  const float iu = nu > 0.f ? 1.f / sqrtf(nu) : 0.f;
  const float iw = nw > 0.f ? 1.f / sqrtf(nw) : 0.f;
  f32x4 uh, wh;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uh[i] = u[4 * qq + i] * iu;   // this thread writes components 4qq .. 4qq+3
    wh[i] = w[4 * qq + i] * iw;
  }
  const int64_t row = (bh * n_chunks + c) * DC + tl;
  *reinterpret_cast<f32x4*>(Uo + row * P_DIM + 4 * qq) = uh;
  *reinterpret_cast<f32x4*>(Wo + row * P_DIM + 4 * qq) = wh;
  *reinterpret_cast<f32x4*>(&ws[tl][4 * qq]) = wh;
  if (qq == 0) bs[tl] = live ? beta[bh * T + t] : 0.f;
  __syncthreads();
  // 16 x 16 blocks of the chunk's 64 x 64 matrices on the fp32 matrix cores
  // (v_mfma_f32_16x16x4_f32, wave64: A lane l holds A[l%16][k = l/16], B lane l holds
  // B[k = l/16][l%16], D lane l holds D[4(l/16) + i][l%16], i = 0..3).
  const int m16 = lane & 15, k4 = lane >> 4;
  // G[t][s] = beta_t (w^_t . w^_s)^2 for s < t, the ten blocks (bt, bs), bt >= bs, over the
  // four waves (the blocks above the diagonal are not read as G)
  for (int tile = wave; tile < 10; tile += 4) {
    const int bt = tile < 1 ? 0 : (tile < 3 ? 1 : (tile < 6 ? 2 : 3));
    const int bsb = tile - bt * (bt + 1) / 2;
    f32x4 acc = zero4();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ws[16 * bt + m16][4 * kk + k4], ws[16 * bsb + m16][4 * kk + k4],
                                                 acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tr = 16 * bt + 4 * k4 + i, sc = 16 * bsb + m16;
      G[tr][sc] = sc < tr ? bs[tr] * acc[i] * acc[i] : 0.f;
    }
  }
  __syncthreads();
  // T = (I + G)^{-1} by blocks (I + G is unit lower triangular).  Diagonal blocks by forward
  // substitution, one column per lane of wave 0 (lane (b, c): column c of block b), written
  // over their G blocks.  Then T_ij = -T_ii (sum_{k = j}^{i-1} G_ik T_kj) for i - j = 1, 2, 3
  // on the matrix cores; T_ij (i > j) is kept in block (j, i) above the diagonal, which G
  // does not use, until the last level.
  if (wave == 0) {
    const int b = lane >> 4, cc = lane & 15;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc0 = r == cc ? 1.f : 0.f, acc1 = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < r; ++s2) {
        if (s2 & 1) acc1 -= G[16 * b + r][16 * b + s2] * x[s2];
        else acc0 -= G[16 * b + r][16 * b + s2] * x[s2];
      }
      x[r] = acc0 + acc1;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) G[16 * b + r][16 * b + cc] = x[r];
  }
  __syncthreads();
  // element (r, c) of block matrix X_ij: G_ij (i > j) at [16i + r][16j + c]; T_ij (i > j) at
  // [16j + r][16i + c]; T_ii at [16i + r][16i + c]
  auto gref = [&](int i, int j, int r, int c) -> float& { return G[16 * i + r][16 * j + c]; };
  auto tref = [&](int i, int j, int r, int c) -> float& {
    return i > j ? G[16 * j + r][16 * i + c] : G[16 * i + r][16 * i + c];
  };
  for (int lev = 1; lev < 4; ++lev) {
    const int i = lev + wave, j = wave;           // wave w: block (w + lev, w)
    if (i < 4) {
      f32x4 xacc = zero4();
      for (int kb = j; kb < i; ++kb) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          xacc = __builtin_amdgcn_mfma_f32_16x16x4f32(gref(i, kb, m16, 4 * kk + k4), tref(kb, j, 4 * kk + k4, m16),
                                                      xacc, 0, 0, 0);
      }
      // X as the B operand: lane l needs X[4kk + l/16][l%16], held by lane 16kk + l%16 in its
      // accumulator entry l/16
      f32x4 tacc = zero4();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int src = (16 * kk + m16) * 4;
        float xb = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(xacc[e])));
          xb = e == k4 ? v : xb;
        }
        tacc = __builtin_amdgcn_mfma_f32_16x16x4f32(tref(i, i, m16, 4 * kk + k4), xb, tacc, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) tref(i, j, 4 * k4 + e, m16) = -tacc[e];
    }
    __syncthreads();
  }
  // T_ij (i > j) from block (j, i) to block (i, j); block (j, i) becomes 0
  for (int e = tid; e < 6 * 256; e += 256) {
    const int blk = e >> 8, r = (e >> 4) & 15, cc = e & 15;
    const int i = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3), j = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
    const float v = G[16 * j + r][16 * i + cc];
    G[16 * i + r][16 * j + cc] = v;
    G[16 * j + r][16 * i + cc] = 0.f;
  }
  __syncthreads();
  // fragments: thread handles (mb, kk, lane') for two of the 4 x 2 x 64 combinations
  bf16* out = Tf + (bh * n_chunks + c) * (DC * DC * 2);
#pragma unroll
  for (int rep = 0; rep < 2; ++rep) {
    const int idx = tid + 256 * rep;          // = (mb * 2 + kk) * 64 + lane'
    const int lf = idx & 63, kk = (idx >> 6) & 1, mb = idx >> 7;
    const int nn = lf & 15, gg = lf >> 4;
    const int row = 16 * mb + nn;
    const f32x4 a = *reinterpret_cast<const f32x4*>(&G[row][32 * kk + 4 * gg]);
    const f32x4 b = *reinterpret_cast<const f32x4*>(&G[row][32 * kk + 16 + 4 * gg]);
    const float xv[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    const Op8<true> f = make8<true>(xv);
    *reinterpret_cast<bf16x8*>(out + idx * 16) = f.hi;
    *reinterpret_cast<bf16x8*>(out + idx * 16 + 8) = f.lo;
  }
}

// Packed state.  Every update adds phi^(k) e^T with phi^(k) = vec(u u^T)/|u|^2 a
// symmetric 16 x 16 matrix, and every read S^T phi^(x) sees only the symmetric part of S
// (phi^(x) is symmetric).  The walk therefore keeps that part in the packed circulant
// order of the one-factor kernels: slot (delta, a) = 16 delta + a stands for the pair
// {a, (a + delta) mod 16}, delta = 0..8 (for delta = 8 the slots a >= 8 repeat a < 8).
// Writes add the packed feature w_a w_(a+delta) unweighted; reads weight it by 1 on the
// diagonal, 2 off it, and 0 for the repeated slots, so the packed inner product equals
// the full one.  That is 144 rows instead of 256 (136 distinct): the state contractions
// shrink from 8 to 5 K-blocks and from 16 to 9 state tiles.  The walk starts from the
// symmetric part of S0 and exports ST = S0 + (packed change) at both entries of each
// pair, so S0's antisymmetric part, which no read sees, reaches ST unchanged (and a walk
// that writes nothing returns S0 bit for bit).
//
// grid (dv/16, B*H), block 512: 8 waves in two roles that share the staged fragments.
//  * state waves (0..3): wave w owns the 16-token block w of every chunk and the packed
//    state tiles delta = w and w + 4 (wave 0 also delta = 8) of the column block; per chunk
//    R = V - K^ S, X = diag(beta) R, E = T X, S += K^^T E - the chain from one chunk's
//    state to the next;
//  * output waves (4..7): wave 4 + m computes, for token block m, Q^ S, the causal score
//    tiles (Q^ K^^T o M) and y = Q^ S + (Q^ K^^T o M) E, off that chain.
// Each SIMD runs one wave of each role, so the output work overlaps the state chain, and
// two walks share a CU (at most 128 VGPRs).  Four barriers per chunk: S and the inputs staged | X written | E written | chunk done.
// Token-K fragments use the permuted order of the accumulator tiles: slot i < 4 of
// K-block kk, lane group g is token 32kk + 4g + i, slot 4 + i is token 32kk + 16 + 4g + i
// (and slot i < 4 of the feature K-block kk is (2kk, 4g + i), slot 4 + i is
// (2kk + 1, 4g + i)), so accumulator tiles are stored as fragments with one 8-byte store
// per lane.  Precision: the state, the corrections X and E, T and the 16-dim cosine tiles
// are hi/lo bf16 operands (~16 significant bits: these are where sums cancel); the
// packed feature fragments (products of unit-vector components) are hi/lo only for fp32
// inputs (SPLIT) and single bf16 for bf16 inputs, as the one-factor kernels round theirs.
// S0/ST [B*H, 256, dv] (nullable; S0 == ST allowed), y [B*H, T, dv].
//
// Segments (nseg > 1).  Walk w = blockIdx.y (after the XCD remap) covers the chunks
// [(w % nseg) seg_chunks, + seg_chunks) of sequence w / nseg, and S0 is that walk's start
// state, [B*H*nseg, 256, dv].  The walk of the last segment exports ST (S0x: the
// sequence's own initial state, whose antisymmetric part passes through).  The chunk
// transition is affine in S, S <- (I - K^^T T diag(beta) K^) S + K^^T T diag(beta) V, so
// a segment maps its start state to S_end = M S_start + b.  AFFINE walks (state waves
// only, 256 threads) compute that map for every segment but the last (nseg = segments
// - 1 there): the value columns from a zero start (b), and DPACK more columns with V = 0
// that start from the packed unit vectors (column DV + i starts as slot i; M's column i),
// and write the packed result, aff [B*H*nseg, DPACK, DV + DPACK].  S0 is then only a flag:
// without an initial state, segment 0's start is 0, so its M is never used and its M
// column blocks return at once.  kata_delta_seg_combine then chains the maps into every
// segment's start state, and the segments' walks (y) run side by side instead of one
// after another.
constexpr int DKB = 5;   // feature K-blocks of the packed state: delta pairs (0,1) .. (8, 9 = none)

template <typename TIn, typename TOut, int DV, bool AFFINE = false>
__global__ void __launch_bounds__(AFFINE ? 256 : 512, AFFINE ? 4 : 2)
kata_delta_chunk(int* __restrict__ prog, const float* __restrict__ Uh, const float* __restrict__ Wh,
                 const bf16* __restrict__ Tf,
                 const TIn* __restrict__ v, const float* __restrict__ beta, const float* S0, float* ST,
                 const float* S0x, TOut* __restrict__ y, int64_t T, int64_t n_chunks, int nseg,
                 int64_t seg_chunks, float* __restrict__ aff) {
  constexpr bool SPLIT = sizeof(TIn) == 4;   // feature fragments split
  __shared__ __align__(16) float Us[DC][P_DIM];
  __shared__ __align__(16) float Wsm[DC][P_DIM];
  __shared__ __align__(16) bf16 SB[2][DKB][WAVE][8];   // packed S as B-fragments, hi / lo
  __shared__ __align__(16) bf16 XB[2][2][WAVE][8];     // diag(beta) R
  __shared__ __align__(16) bf16 EB[2][2][WAVE][8];     // E
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool state_role = AFFINE || wave < 4;
  const int mb = wave & 3;                            // 16-token block of this wave
  const int n = lane & 15, g = lane >> 4;
  // The dv/16 workgroups of a sequence read the same u^, w^ and T.  Workgroups go to the
  // 8 XCDs (each with its own L2) round-robin by linear id, so when B*H is a multiple of 8
  // the ids are remapped to place all column blocks of a sequence on one XCD:
  // id = 8 slot + xcd, sequence = xcd + 8 (slot / NBLK), column block = slot % NBLK.
  constexpr int NCOL = AFFINE ? DV + DPACK : DV;    // state columns of the walk
  constexpr int NBLK = NCOL / 16;
  int j = blockIdx.x;                                 // value column block
  int64_t bw = blockIdx.y;                            // walk: (sequence, segment)
  if ((gridDim.y & 7) == 0) {
    const int64_t id = (int64_t)blockIdx.y * NBLK + blockIdx.x;
    const int64_t xcd = id & 7, slot = id >> 3;
    bw = xcd + 8 * (slot / NBLK);
    j = (int)(slot % NBLK);
  }
  const int64_t bh = bw / nseg;                       // sequence
  const int64_t seg = bw % nseg;                      // segment
  const int64_t c0 = seg * seg_chunks;                // its first chunk
  const int64_t nch = min<int64_t>(seg_chunks, n_chunks - c0);   // chunks of this walk
  const int64_t tok0 = c0 * DC;
  const bool couple_on = !AFFINE && nseg == 1;        // progress coupling: whole-sequence walks
  constexpr int PF = 1;                               // chunks of input prefetch (one set)
  const int col = 16 * j + n;                         // state column of this lane
  const bool vcols = !AFFINE || j < DV / 16;          // (workgroup-uniform) a value column block
  if (AFFINE && !vcols && seg == 0 && !S0) return;    // segment 0 starts from 0: M unused
  // v and beta of this walk's tokens through range-checked buffers: rows past T read 0
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + (bh * T + tok0) * DV, (T - tok0) * DV * (int64_t)sizeof(TIn));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(beta + bh * T + tok0, (T - tok0) * 4);

  auto put = [&](auto& dst, int kk, int slot, const float (&x)[4]) {   // dst [2][K-blocks][WAVE][8]
    bf16x4 hi, lo;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      hi[r] = (bf16)x[r];
      lo[r] = (bf16)(x[r] - (float)hi[r]);
    }
    *reinterpret_cast<bf16x4*>(&dst[0][kk][lane][slot]) = hi;
    *reinterpret_cast<bf16x4*>(&dst[1][kk][lane][slot]) = lo;
  };
  auto frag = [&](const auto& src, int kk) {
    Op8<true> f;
    f.hi = *reinterpret_cast<const bf16x8*>(&src[0][kk][lane][0]);
    f.lo = *reinterpret_cast<const bf16x8*>(&src[1][kk][lane][0]);
    return f;
  };

  // Packed state tiles (state waves): tile jt is diagonal dl(jt) = w, w + 4, and 8 (wave 0
  // only); lane (n, g) holds slots (dl, a = 4g + r), column col.  sym0 gives the symmetric
  // part of S0 at the lane's pair {a, b} (full row indices 16 a + b and 16 b + a).
  const bool own8 = state_role && wave == 0;
  auto dl = [&](int jt) { return jt == 2 ? 8 : wave + 4 * jt; };
  auto s0_at = [&](int a, int b) { return S0[(bw * P_DIM * P_DIM + 16 * a + b) * DV + col]; };
  auto sym0 = [&](int a, int b) { return 0.5f * (s0_at(a, b) + s0_at(b, a)); };
  f32x4 Sacc[3];
#pragma unroll
  for (int jt = 0; jt < 3; ++jt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int a = 4 * g + r, b = (a + dl(jt)) & 15;
      if constexpr (AFFINE)   // value columns from 0, column DV + i from packed slot i
        Sacc[jt][r] = ((jt < 2 || own8) && col >= DV && 16 * dl(jt) + a == col - DV) ? 1.f : 0.f;
      else
        Sacc[jt][r] = (S0 && state_role && (jt < 2 || own8)) ? sym0(a, b) : 0.f;
    }
  }
  // the K-block 4 slots 4..7 stand for delta = 9, which does not exist: zero once
  if (tid < 2 * WAVE) {
    const bf16x4 z = {(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
    *reinterpret_cast<bf16x4*>(&SB[tid >> 6][DKB - 1][lane][4]) = z;
  }

  // per-chunk inputs, prefetched one chunk ahead into one register set (a second set, two
  // chunks ahead, would cost the registers that let two walks, or four AFFINE walks, share
  // a CU).  Threads 0..255 stage u^, threads 256..511 w^ (AFFINE: threads 0..255 w^, no
  // u^); the state waves also take T (their own hi/lo A-fragments), v and beta.
  struct Inputs {
    f32x4 puw;
    Op8<true> pt[2];
    uint32_t pv[4];   // raw bits of v (converted at use)
    float pb[4];
  };
  // T is fetched apart from the rest (fetch_t), after its one use in the step, so the
  // step reads it from the register set itself with no copy.
  auto fetch_t = [&](Inputs& in, int64_t c) {
    const bf16* tf = Tf + (bh * n_chunks + c0 + c) * (DC * DC * 2) + ((mb * 2) * WAVE + lane) * 16;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      in.pt[kk].hi = *reinterpret_cast<const bf16x8*>(tf + kk * WAVE * 16);
      in.pt[kk].lo = *reinterpret_cast<const bf16x8*>(tf + kk * WAVE * 16 + 8);
    }
  };
  auto fetch = [&](Inputs& in, int64_t c) {
    const int64_t rbase = (bh * n_chunks + c0 + c) * DC;
    in.puw = *reinterpret_cast<const f32x4*>(((AFFINE || !state_role) ? Wh : Uh) + rbase * P_DIM + 4 * (tid & 255));
    if (state_role) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = (int)(c * DC) + 16 * mb + 4 * g + r;
        in.pv[r] = vcols ? buf_bits<TIn>(rv, t * DV + col) : 0u;
        in.pb[r] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, t * 4, 0, 0));
      }
    }
  };

  const int rot = (lane & ~15) | ((n + wave) & 15);   // lane of the row rotated by w

  auto step = [&](Inputs& in, int64_t c) {
    // ---- stage: inputs to LDS, packed S to B-fragments (K-block dl / 2, half dl % 2)
    *reinterpret_cast<f32x4*>(((AFFINE || !state_role) ? &Wsm[0][0] : &Us[0][0]) + 4 * (tid & 255)) = in.puw;
    float vv[4], bb[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      vv[r] = bits_value<TIn>(in.pv[r]);
      bb[r] = in.pb[r];
    }
    if (state_role) {
      // published with the read weights (1 on the diagonal, 2 off it, 0 for the repeated
      // delta = 8 slots a >= 8): powers of two, so the products equal weighted features
      // times S exactly
#pragma unroll
      for (int jt = 0; jt < 3; ++jt) {
        if (jt < 2 || own8) {
          const int d = dl(jt);
          const float wt = d == 0 ? 1.f : (d == 8 ? (g < 2 ? 2.f : 0.f) : 2.f);
          const float sx[4] = {Sacc[jt][0] * wt, Sacc[jt][1] * wt, Sacc[jt][2] * wt, Sacc[jt][3] * wt};
          put(SB, d >> 1, (d & 1) * 4, sx);
        }
      }
    }
    __syncthreads();
    if (c + PF < nch) fetch(in, c + PF);

    // ---- R = V - K^ S (state waves) or Q^ S (output waves), tokens 16 mb + n, K = packed
    // slot.  xr[m] = components 4g + 4m .. 4g + 4m + 3 (mod 16) of the token's projection,
    // so component (4g + i + delta) mod 16 is xr[(i + delta) / 4 % 4][(i + delta) % 4].
    const int tt = 16 * mb + n;
    const float* xs = state_role ? &Wsm[tt][0] : &Us[tt][0];
    f32x4 xr[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) xr[m] = *reinterpret_cast<const f32x4*>(xs + ((4 * g + 4 * m) & 15));
    auto comp = [&](int e) { return xr[(e >> 2) & 3][e & 3]; };
    f32x4 acc = zero4();
#pragma unroll
    for (int kk = 0; kk < DKB; ++kk) {   // (the read weights ride on the published S)
      const int d0 = 2 * kk, d1 = 2 * kk + 1;
      float xf[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xf[i] = comp(i) * comp(i + d0);
        xf[4 + i] = d1 == 9 ? 0.f : comp(i) * comp(i + d1);
      }
      acc = mma<SPLIT, true>(make8<SPLIT>(xf), frag(SB, kk), acc);
    }
    // accumulator lane (n, g) holds token 16 mb + 4g + r, column col
    if (state_role) {
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = bb[r] * (vv[r] - acc[r]);
      put(XB, mb >> 1, (mb & 1) * 4, x);
    }
    // output waves: the causal score tiles of key K-block kk against this query block as an
    // A-fragment, built off the state chain (kk = 0 beside E = T X, kk = 1 beside the state
    // update).  X = W^_sb U^_mb^T (K = 16), lane (t = n, g) holds s = 16 sb + 4g + r:
    // (u^_t . w^_s)^2, masked s <= t.
    auto score_frag = [&](int kk) {
      const float ubv[4] = {xr[0][0], xr[0][1], xr[0][2], xr[0][3]};
      const Op4<true> uf = make4<true>(ubv);
      float xa[8];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int sb = 2 * kk + hb;
        if (sb <= mb) {
          const f32x4 wb = *reinterpret_cast<const f32x4*>(&Wsm[16 * sb + n][4 * g]);
          float wbv[4] = {wb[0], wb[1], wb[2], wb[3]};
          const f32x4 X = mma<true, true>(make4<true>(wbv), uf, zero4());
#pragma unroll
          for (int r = 0; r < 4; ++r) xa[4 * hb + r] = (sb < mb || 4 * g + r <= n) ? X[r] * X[r] : 0.f;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) xa[4 * hb + r] = 0.f;
        }
      }
      return make8<SPLIT>(xa);
    };
    __syncthreads();

    // ---- E = T X (state waves), tokens 16 mb + n (A rows of T), K = token
    Op8<SPLIT> sc0;
    if (state_role) {
      f32x4 accE = zero4();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) accE = mma<true, true>(in.pt[kk], frag(XB, kk), accE);
      if (c + PF < nch) fetch_t(in, c + PF);
      const float ex[4] = {accE[0], accE[1], accE[2], accE[3]};
      put(EB, mb >> 1, (mb & 1) * 4, ex);
    } else {
      sc0 = score_frag(0);
    }
    __syncthreads();

    if (state_role) {
      // ---- S += K^^T E on the owned diagonals: as an A operand, row n of tile delta is
      // slot (delta, a = n), so slot i of K-block kk carries w^_s[n] w^_s[(n + delta) % 16]
      // of token s.  wn: component n; wr: component (n + w) % 16 (a rotated LDS read), so
      // delta = w is wn wr, delta = w + 4 rotates wr by 4 lanes, delta = 8 rotates wn by 8.
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const Op8<true> eb = frag(EB, kk);
        float wn[8], wr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int sidx = 32 * kk + (i < 4 ? 4 * g + i : 16 + 4 * g + i - 4);
          wn[i] = Wsm[sidx][n];
          wr[i] = Wsm[sidx][rot & 15];
        }
        float xa[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) xa[i] = wn[i] * wr[i];
        Sacc[0] = mma<SPLIT, true>(make8<SPLIT>(xa), eb, Sacc[0]);
#pragma unroll
        for (int i = 0; i < 8; ++i) xa[i] = wn[i] * row_plus<4>(wr[i]);
        Sacc[1] = mma<SPLIT, true>(make8<SPLIT>(xa), eb, Sacc[1]);
        if (own8) {
#pragma unroll
          for (int i = 0; i < 8; ++i) xa[i] = wn[i] * row_plus<8>(wn[i]);
          Sacc[2] = mma<SPLIT, true>(make8<SPLIT>(xa), eb, Sacc[2]);
        }
      }
    } else {
      // ---- y = Q^ S + (Q^ K^^T o M) E: A = score rows t over key tokens s, B = E (K = s)
      acc = mma<SPLIT, true>(sc0, frag(EB, 0), acc);
      if (mb >= 2) acc = mma<SPLIT, true>(score_frag(1), frag(EB, 1), acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = tok0 + c * DC + 16 * mb + 4 * g + r;
        if (t < T) Elem<TOut>::store(y, (bh * T + t) * DV + col, acc[r]);
      }
    }
    __syncthreads();
  };

  // Progress coupling of the NBLK column-block workgroups of a sequence.  They read the
  // same u^, w^ and T of every chunk from their XCD's L2; left alone they drift apart over
  // the chunks, and a workgroup far behind the first misses in L2 and reads them again from
  // memory (1.45-1.56x the algorithmic bytes).  Every COUPLE_EVERY chunks a workgroup
  // publishes its progress, and while it is more than COUPLE_LAG chunks ahead of the
  // slowest workgroup of its sequence it sleeps and polls again, at most COUPLE_POLLS
  // times.  The wait only orders memory traffic (results do not depend on it), and the
  // poll bound ends it even if a partner never ran.
  constexpr int COUPLE_EVERY = 32, COUPLE_LAG = 32, COUPLE_POLLS = 2048;
  int* myprog = prog + bh * NBLK;   // (only whole-sequence walks couple: bw == bh there)
  auto couple = [&](int64_t cc) {
    if (tid == 0) {
      __hip_atomic_store(myprog + j, (int)cc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int it = 0; it < COUPLE_POLLS; ++it) {
        int slowest = (int)cc;
#pragma unroll
        for (int o = 0; o < NBLK; ++o)
          slowest = min(slowest, __hip_atomic_load(myprog + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        if (cc - slowest <= COUPLE_LAG) break;
        __builtin_amdgcn_s_sleep(8);
      }
    }
    __syncthreads();
  };

  Inputs in{};   // zeroed: the output waves load only puw and never read the rest
  if (nch > 0) {
    fetch(in, 0);
    if (state_role) fetch_t(in, 0);
  }
  for (int64_t c = 0; c < nch; ++c) {
    if (couple_on && c % COUPLE_EVERY == 0) couple(c);
    step(in, c);
  }
  if (couple_on && tid == 0)   // done: nobody waits for this workgroup any more
    __hip_atomic_store(myprog + j, (int)(nch + COUPLE_LAG), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if constexpr (AFFINE) {
    // the packed state of every owned slot (the repeated delta = 8 slots too), column col
#pragma unroll
    for (int jt = 0; jt < 3; ++jt) {
      if (jt < 2 || own8) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          aff[(bw * DPACK + 16 * dl(jt) + 4 * g + r) * NCOL + col] = Sacc[jt][r];
      }
    }
    return;
  }
  // ST = S0x + the change of the packed state since the sequence's start, at both entries
  // (a, b) and (b, a) of each pair, written by the one lane that owns its slot (for
  // delta = 8 the lanes a < 8) in the walk of the last segment.  That lane is also the
  // only reader of these S0x entries, so S0x == ST is safe.
  auto s0x_at = [&](int a, int b) { return S0x[(bh * P_DIM * P_DIM + 16 * a + b) * DV + col]; };
  if (ST && state_role && seg == nseg - 1) {
#pragma unroll
    for (int jt = 0; jt < 3; ++jt) {
      if (jt < 2 || own8) {
        const int d = dl(jt);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int a = 4 * g + r, b = (a + d) & 15;
          if (d == 8 && a >= 8) continue;
          float sab = 0.f, sba = 0.f, ch = Sacc[jt][r];
          if (S0x) {
            sab = s0x_at(a, b);
            sba = s0x_at(b, a);
            ch -= 0.5f * (sab + sba);
          }
          ST[(bh * P_DIM * P_DIM + 16 * a + b) * DV + col] = sab + ch;
          if (d != 0) ST[(bh * P_DIM * P_DIM + 16 * b + a) * DV + col] = sba + ch;
        }
      }
    }
  }
}

// grid (dv/16, B*H), block SEG_THREADS: the start state of every segment of a sequence
// from the affine maps of the segments before it (kata_delta_chunk<..., AFFINE>, aff
// [B*H*(nseg - 1), DPACK, dv + DPACK]), in order:
//   S_0 = the symmetric part of S0 (or 0),  S_{s+1} = M_s S_s + b_s   (packed, fp32),
// written canonically (both mirror entries of each pair hold the packed value, which is
// what the walk's initial read takes) to S0seg [B*H*nseg, 256, dv] for the segments'
// walks.  Without S0, M_0 is not formed (S_1 = b_0).  The walk of the last segment
// exports the final state.  M_s S_s runs on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32: fp32 products and sums): wave w forms rows 16w .. 16w+15 of
// the 16 columns, with its rows of M_s in registers (loaded one segment ahead) and S_s in
// LDS, column-major.
__device__ __forceinline__ int pair_slot(int a, int b) {   // packed slot of the pair {a, b}
  int dlt = (b - a) & 15, aa = a;
  if (dlt > 8) {
    dlt = 16 - dlt;
    aa = b;
  } else if (dlt == 8) {
    aa = a < b ? a : b;                                   // the used slot of delta = 8
  }
  return 16 * dlt + aa;
}

constexpr int SEG_WAVES = DPACK / 16;         // 9: one 16-row block of the packed state each
constexpr int SEG_THREADS = SEG_WAVES * WAVE;
constexpr int SEG_STR = DPACK + 4;            // LDS column stride of the state (floats)
constexpr int SEG_KB = DPACK / 16;            // 16-column groups of M per lane row

template <int DV>
__global__ void __launch_bounds__(SEG_THREADS)
kata_delta_seg_combine(const float* __restrict__ aff, const float* __restrict__ S0, float* __restrict__ S0seg,
                       int nseg) {
  constexpr int NCOL = DV + DPACK;
  __shared__ __align__(16) float Sp[16 * SEG_STR];   // [16 columns][DPACK slots] (padded)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = tid >> 6;
  const int j = blockIdx.x;
  const int64_t bh = blockIdx.y;
  // MFMA lanes: A lane l holds A[l%16][k = l/16], B lane l holds B[k = l/16][l%16], D lane l
  // holds D[4(l/16) + i][l%16].  Lane (n, g) holds M's row 16 wave + n at columns
  // 16 kb + 4g .. +3; the MFMA (kb, i) takes its column 16 kb + 4g + i as K index g, and
  // the state column n at the same slot as the B operand.
  const int n = lane & 15, g = lane >> 4;
  auto s0_at = [&](int a, int b, int cc) { return S0[(bh * P_DIM * P_DIM + 16 * a + b) * DV + 16 * j + cc]; };
  for (int e = tid; e < DPACK * 16; e += SEG_THREADS) {
    const int slot = e >> 4, cc = e & 15;
    const int a = slot & 15, b = (a + (slot >> 4)) & 15;
    Sp[cc * SEG_STR + slot] = S0 ? 0.5f * (s0_at(a, b, cc) + s0_at(b, a, cc)) : 0.f;
  }
  // the maps are loaded two segments ahead into two register sets, which alternate
  f32x4 ma[SEG_KB], mb[SEG_KB], ba, bb;
  auto load_map = [&](int sg, f32x4 (&mr)[SEG_KB], f32x4& br) {
    const float* blk = aff + (bh * (nseg - 1) + sg) * DPACK * NCOL;
#pragma unroll
    for (int kb = 0; kb < SEG_KB; ++kb)
      mr[kb] = *reinterpret_cast<const f32x4*>(blk + (16 * wave + n) * NCOL + DV + 16 * kb + 4 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) br[i] = blk[(16 * wave + 4 * g + i) * NCOL + 16 * j + n];   // b
  };
  // one segment: write its start state; unless it is the last, S <- M S + b (then the
  // register set is free for the map two segments on)
  auto step = [&](int sg, f32x4 (&mr)[SEG_KB], f32x4& br) {
    const int64_t bw = bh * nseg + sg;
    __syncthreads();   // the previous step's state written
    for (int e = tid; e < 256 * 16; e += SEG_THREADS) {
      const int ab = e >> 4, cc = e & 15;
      S0seg[(bw * 256 + ab) * DV + 16 * j + cc] = Sp[cc * SEG_STR + pair_slot(ab >> 4, ab & 15)];
    }
    if (sg + 1 >= nseg) return false;   // the last segment has no map
    f32x4 acc = br;
    if (sg > 0 || S0) {   // S_0 = 0 without S0: M_0 was not formed
#pragma unroll
      for (int kb = 0; kb < SEG_KB; ++kb) {
        const f32x4 sv = *reinterpret_cast<const f32x4*>(&Sp[n * SEG_STR + 16 * kb + 4 * g]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(mr[kb][i], sv[i], acc, 0, 0, 0);
      }
    }
    if (sg + 3 < nseg) load_map(sg + 2, mr, br);   // segments 0 .. nseg - 2 have maps
    __syncthreads();   // every wave has read the state
    *reinterpret_cast<f32x4*>(&Sp[n * SEG_STR + 16 * wave + 4 * g]) = acc;
    return true;
  };
  load_map(0, ma, ba);   // (nseg >= 2: segment 0 has a map)
  if (nseg > 2) load_map(1, mb, bb);
  for (int sg = 0;; sg += 2) {
    if (!step(sg, ma, ba) || !step(sg + 1, mb, bb)) break;
  }
}

}  // namespace kata
