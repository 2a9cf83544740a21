// kata_bwd.h - backward pass of the KATA causal forward in the chunked-state form on
// gfx950: gradients of q, k, v, the projection P and the initial state (S0, z0).
//
// The pages describe the forward only (gist.science summary of "Kernelized Linear
// Attention", arXiv 2607.17419, section 2.3: chunked state, associative scan over chunk
// states; the paper's abstract: exact O(T) form).  Its gradient follows from the
// forward by the chain rule.  With u = P q, w = P k, a_ts = (u_t . w_s)^2 (s <= t):
//
//   g_t = gy_t / den_t,  h_t = -(gy_t . y_t) / den_t           (gradient of [num_t | den_t])
//   ga_ts = g_t . v_s + h_t,  B_ts = 2 (u_t . w_s) ga_ts
//   du_t = sum_{s<=t} B_ts w_s + 2 F_t u_t,   F_t = mat([S_t | z_t] [g_t | h_t])  (prefix state)
//   dw_s = sum_{t>=s} B_ts u_t + 2 G_s w_s,   G_s = mat([R_s | r_s] [v_s | 1])    (suffix state)
//   dv_s = sum_{t>=s} a_ts g_t  (= R_s^T phi(w_s) for the later chunks)
//
// where [R | r] = sum_{t} phi(u_t) [g_t | h_t]^T over the later tokens (plus the
// gradient of the final state) is the backward's own state: a reverse (suffix) prefix
// of chunk states of exactly the forward's form with (q, [g | h]) in place of
// (k, [v | 1]).  So the backward is two chunk walks:
//   kata_bwd_query : forward order over the chunks of a leaf, from the forward's scanned
//                    prefix state: den, g, h, du -> dq, and the dP share of du q^T;
//                    writes 1/den_t and h_t (8 bytes per token) for the later kernels,
//                    which form g_t = gy_t (1/den_t) again, bit for bit
//   kata_bwd_rstate: per leaf, sum of phi(U_c)^T [G_c | h_c]   (Z part: U^T diag(h) U)
//   kata_state_scan: (reverse) exclusive suffix of those leaf states; its total is dS0, dz0
//   kata_bwd_key   : reverse order over the chunks of a leaf, from the suffix state:
//                    dv, dw -> dk, and the dP share of dw k^T
//   kata_bwd_dp_reduce: dP = sum of the per-workgroup partials over batch rows and leaves
//
// Contractions of a state with a vector of value columns (F_t above) need the state
// with the value column as the MFMA K index, the transpose of the readout's layout: the
// owners publish it as "HT" fragments, HT[delta][kc][lane = (a, g)][i] =
// H[(delta, a)][32 kc + 8 g + i].  The packed slot (delta, a) holds u_a u_{a+delta}, so
// the gradient of slot (delta, a) reaches both u_a and u_{a+delta}; reading the HT
// fragment of row (a - delta) mod 16 in lane a (a permuted LDS read) lines up the
// second term with lane a, so every lane accumulates its own 4 entries of du_t with
// no cross-lane reduction.
#pragma once

#include "kata_chunk.h"

namespace kata {

// The backward instance: C = 64, d = dv = 64, bf16 q/k/v.
using BS = Shape<64, 64, 64, false>;
constexpr int BW_GSTR = 72;                          // bf16 row stride of token rows staged in LDS
constexpr int BW_ROWS_BYTES = BS::C * BW_GSTR * 2;   // 9216
constexpr int BW_HT_BYTES = NDELTA * 2 * WAVE * 16;  // 18432: HT fragments of one state
constexpr int BW_DP = P_DIM * 64;                    // floats of one dP partial (16 x 64)

// kata_bwd_query LDS (bytes)
constexpr int QA_OFF_VF = 0;
constexpr int QA_OFF_VR = QA_OFF_VF + BS::VF_BYTES;
constexpr int QA_OFF_U = QA_OFF_VR + BW_ROWS_BYTES;
constexpr int QA_OFF_W = QA_OFF_U + BS::U_BYTES;
constexpr int QA_OFF_WACC = QA_OFF_W + BS::U_BYTES;
constexpr int QA_OFF_WZ = QA_OFF_WACC + BS::WACC_BYTES;
constexpr int QA_OFF_HT = QA_OFF_WZ + BS::WZ_BYTES;
constexpr int QA_OFF_Z = QA_OFF_HT + BW_HT_BYTES;
constexpr int QA_OFF_PF = QA_OFF_Z + BS::Z_BYTES;
constexpr int QA_OFF_PT = QA_OFF_PF + BS::PF_BYTES;
constexpr int QA_OFF_GY = QA_OFF_PT + 4 * 2 * WAVE * 8;
// gy rows of the chunk (row stride keeps 16-byte alignment and spreads the banks)
template <typename TY> struct QaGy {
  static constexpr int STR = sizeof(TY) == 2 ? 72 : 68;
  static constexpr int SMEM = QA_OFF_GY + BS::C * STR * (int)sizeof(TY);
};
static_assert(QaGy<bf16>::SMEM * 2 <= 156 * 1024, "two query workgroups per CU (bf16 gy)");

// kata_bwd_key LDS (bytes)
constexpr int KB_OFF_HX = 0;
constexpr int KB_OFF_HT = KB_OFF_HX + BS::HX_BYTES;
constexpr int KB_OFF_Z = KB_OFF_HT + BW_HT_BYTES;
constexpr int KB_OFF_GF = KB_OFF_Z + BS::Z_BYTES;
constexpr int KB_OFF_GRH = KB_OFF_GF + BS::VF_BYTES;
constexpr int KB_OFF_GRL = KB_OFF_GRH + BW_ROWS_BYTES;
constexpr int KB_OFF_U = KB_OFF_GRL + BW_ROWS_BYTES;
constexpr int KB_OFF_W = KB_OFF_U + BS::U_BYTES;
constexpr int KB_OFF_UACC = KB_OFF_W + BS::U_BYTES;
constexpr int KB_OFF_HS = KB_OFF_UACC + BS::WACC_BYTES;
constexpr int KB_OFF_PF = KB_OFF_HS + BS::C * 4;
constexpr int KB_OFF_PT = KB_OFF_PF + BS::PF_BYTES;
constexpr int KB_OFF_DW = KB_OFF_PT + 4 * 2 * WAVE * 8;
constexpr int KB_SMEM = KB_OFF_DW + 2 * BS::C * P_DIM * 4;   // dw of two chunks (role 1 -> role 0)
static_assert(KB_SMEM <= 156 * 1024, "key workgroup LDS");
static_assert(4 * 4 * WAVE * 16 <= BS::HX_BYTES && 4 * 4 * WAVE * 16 <= BW_HT_BYTES, "dP reduction fits");

// kata_bwd_rstate LDS (bytes)
constexpr int RS_OFF_VF = 0;
constexpr int RS_OFF_WACC = RS_OFF_VF + BS::VF_BYTES;
constexpr int RS_OFF_WZ = RS_OFF_WACC + BS::WACC_BYTES;
constexpr int RS_OFF_PF = RS_OFF_WZ + BS::WZ_BYTES;
constexpr int RS_OFF_HS = RS_OFF_PF + BS::PF_BYTES;
constexpr int RS_SMEM = RS_OFF_HS + BS::C * 4;

__device__ __forceinline__ int ht_index(int delta, int kc, int l) { return ((delta * 2 + kc) * WAVE + l) * 8; }

// Scatter accumulator tile (delta, nb) of a state held in the readout orientation (lane
// (n, g) holds rows (delta, 4g + r) of column 16 nb + n) into the HT fragments.
__device__ __forceinline__ void put_ht(bf16* HT, int delta, int nb, const f32x4& acc, int lane) {
  const int n = lane & 15, g = lane >> 4;
  const int kc = nb >> 1;
  const int cp = 16 * (nb & 1) + n;     // column within the 32-column K-block
  const int gp = cp >> 3, i = cp & 7;
#pragma unroll
  for (int r = 0; r < 4; ++r) HT[ht_index(delta, kc, 4 * g + r + 16 * gp) + i] = (bf16)acc[r];
}

// The same tile as bf16 readout fragments (the forward's layout): kb = delta / 2,
// slots 4 (delta & 1) .. +3.
__device__ __forceinline__ void put_hx(bf16* hx, int delta, int nb, const f32x4& a, int lane) {
  const int idx = (((delta >> 1) * BS::NB + nb) * WAVE + lane) * 8 + (delta & 1) * 4;
  bf16x4 hi;
#pragma unroll
  for (int i = 0; i < 4; ++i) hi[i] = (bf16)a[i];
  *reinterpret_cast<bf16x4*>(hx + idx) = hi;
}

// The 16 x 16 z-matrix of a state (symmetric; its accumulator tile is its own
// 16x16x16 A-fragment) split into hi/lo bf16.
__device__ __forceinline__ void put_z(bf16* Zs, const f32x4& Z, int lane) {
  float zv[4] = {Z[0], Z[1], Z[2], Z[3]};
  const Op4<true> z = make4<true>(zv);
  bf16x8 zz;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    zz[i] = z.hi[i];
    zz[4 + i] = z.lo[i];
  }
  *reinterpret_cast<bf16x8*>(Zs + lane * 8) = zz;
}
__device__ __forceinline__ Op4<true> get_z(const bf16* Zs, int lane) {
  const bf16x8 zz = *reinterpret_cast<const bf16x8*>(Zs + lane * 8);
  Op4<true> zf;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    zf.hi[i] = zz[i];
    zf.lo[i] = zz[4 + i];
  }
  return zf;
}

// ---- input-space gradient and the projection's gradient ----------------------------

// P^T as 16x16x16 A-fragments (M = input column within block db, K = projection index):
// lane (n, g) holds P[4g + i][16 db + n], split hi/lo.  Loop-invariant: written to LDS
// once (PTs[db][hi/lo][lane], 8 bytes each, 4 KiB) and read back per use.
constexpr int BW_PT_BYTES = 4 * 2 * WAVE * 8;
__device__ __forceinline__ void write_pt(bf16* PTs, const float* __restrict__ P, int h, int lane) {
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = P[((int64_t)h * P_DIM + 4 * g + i) * 64 + 16 * db + n];
    const Op4<true> f = make4<true>(x);
    *reinterpret_cast<bf16x4*>(PTs + ((2 * db) * WAVE + lane) * 4) = f.hi;
    *reinterpret_cast<bf16x4*>(PTs + ((2 * db + 1) * WAVE + lane) * 4) = f.lo;
  }
}
__device__ __forceinline__ Op4<true> read_pt(const bf16* PTs, int db, int lane) {
  Op4<true> f;
  f.hi = *reinterpret_cast<const bf16x4*>(PTs + ((2 * db) * WAVE + lane) * 4);
  f.lo = *reinterpret_cast<const bf16x4*>(PTs + ((2 * db + 1) * WAVE + lane) * 4);
  return f;
}

// Given the projected-space gradient of one 16-token block (lane (t, g) holds
// d_t[4g + r], t = the block's token n): store P^T d_t (input-space gradient, bf16; lane
// (t, g) forms columns 16 db + 4g + r, which store_row sends out as whole 128-byte rows)
// and add d x^T to this wave's dP accumulators.
// xr are the block's input rows as loaded for the projection (lane (t, g) holds
// x_t[16 g + 8 kk + i]).  d^T comes from one identity MFMA per hi/lo half (exact), x^T
// from column-selector MFMAs (exact), so dP takes one MFMA per half.
struct DPAcc { f32x4 t[4]; };   // lane (a, g) holds dP[a][16 db + 4g + r]

__device__ __forceinline__ void grad_head(const f32x4& d, const bf16* PTs, const bf16x8 (&xr)[2],
                                          __amdgpu_buffer_rsrc_t out, int row_byte, DPAcc& acc, int lane) {
  const int n = lane & 15, g = lane >> 4;
  float dv4[4] = {d[0], d[1], d[2], d[3]};
  const Op4<true> df = make4<true>(dv4);
  f32x4 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = mma<true, true>(read_pt(PTs, db, lane), df, zero4());   // column 16db + 4g + r
  store_row<BS, bf16>(o, 1.f, out, row_byte / 2, n, g);
  // d^T: C[t][a] = sum_k d_t[k] [k == a]; lane (a, g) then holds d_{4g + r}[a]
  bf16x4 eye;
#pragma unroll
  for (int i = 0; i < 4; ++i) eye[i] = (bf16)((4 * g + i == n) ? 1.f : 0.f);
  f32x4 tr = mfma16(df.hi, eye, zero4());
  tr = mfma16(df.lo, eye, tr);
  float tv[4] = {tr[0], tr[1], tr[2], tr[3]};
  const Op4<true> tf = make4<true>(tv);
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    // x^T block db: C[t][n'] = x_t[16 db + n'], lane (n', g) holds token 4g + r; the
    // selector picks input column 16 db + n' out of this lane group's 8 columns
    f32x4 xt = zero4();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 hot;
#pragma unroll
      for (int i = 0; i < 8; ++i) hot[i] = (bf16)((g == db && 8 * kk + i == n) ? 1.f : 0.f);
      xt = mfma32(xr[kk], hot, xt);
    }
    Op4<false> xa;
#pragma unroll
    for (int i = 0; i < 4; ++i) xa.hi[i] = (bf16)xt[i];
    acc.t[db] = mma<false, true>(xa, tf, acc.t[db]);    // lane (a, g): += sum_t x_t[16db + 4g + r] d_t[a]
  }
}

// Sum the dP accumulators of the 4 waves that hold them, in a fixed order (through `red`,
// 16 KiB of LDS free at this point), and write the workgroup's partial ([a][col]).
__device__ __forceinline__ void write_dp_partial(const DPAcc& acc, bool holder, int hw, float* red,
                                                 float* __restrict__ out, int tid, int lane) {
  if (holder) {
#pragma unroll
    for (int db = 0; db < 4; ++db) *reinterpret_cast<f32x4*>(red + ((hw * 4 + db) * WAVE + lane) * 4) = acc.t[db];
  }
  __syncthreads();
  if (tid < 256) {
    const int db = tid >> 6, l = tid & 63;
    f32x4 s = zero4();
#pragma unroll
    for (int w = 0; w < 4; ++w) s += *reinterpret_cast<const f32x4*>(red + ((w * 4 + db) * WAVE + l) * 4);
    const int a = l & 15, g = l >> 4;
    *reinterpret_cast<f32x4*>(out + a * 64 + 16 * db + 4 * g) = s;
  }
}

// Contraction of the HT-published state with one value-column vector per token:
// du_t[b] += qw(delta, b) F[(delta, b)] u_t[b + delta] + qw(delta, b - delta) F[(delta,
// b - delta)] u_t[b - delta] (indices mod 16), F = H x_t, summed over delta; lane (t, g)
// accumulates b = 4g + r.  xf: x_t as natural K-order fragments (lane (t, g) holds
// x_t[32 kc + 8 g + i]); Q: rotated quads of u_t (Q[m] = u_t[4((g + m) & 3) .. + 3]).
// With GN, also adds this lane's share of phi(u_t) . (H x_t) (query weights included) to
// *gn: summed over the lane groups it is x_t . (the inter-chunk part of the numerator).
// Only the diagonals DLO <= delta < DHI are taken (the contraction may be split
// between waves).
template <bool GN, int DLO = 0, int DHI = NDELTA>
__device__ __forceinline__ void ht_contract(f32x4& du, float* gn, const bf16* HT, const bf16x8 (&xf)[2],
                                            const f32x4 (&Q)[4], int lane) {
  const int n = lane & 15, g = lane >> 4;
  auto u_rot = [&](int delta, int i) -> float {   // u_t[(4g + i + delta) & 15]
    const int m = delta >> 2, e = delta & 3;
    const int j = i + e;
    return j < 4 ? Q[m & 3][j] : Q[(m + 1) & 3][j - 4];
  };
#pragma unroll
  for (int delta = DLO; delta < DHI; ++delta) {
    f32x4 f = zero4(), f2 = zero4();
    const int lrot = ((n - delta) & 15) + 16 * g;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      f = mfma32(*reinterpret_cast<const bf16x8*>(HT + ht_index(delta, kc, lane)), xf[kc], f);
      if (delta != 0) f2 = mfma32(*reinterpret_cast<const bf16x8*>(HT + ht_index(delta, kc, lrot)), xf[kc], f2);
    }
    if (delta == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        du[r] += 2.f * f[r] * Q[0][r];
        if constexpr (GN) *gn += f[r] * Q[0][r] * Q[0][r];
      }
    } else {
      const float w1 = delta == 8 ? (g < 2 ? 2.f : 0.f) : 2.f;    // slot (delta, b) valid
      const float w2 = delta == 8 ? (g >= 2 ? 2.f : 0.f) : 2.f;   // slot (delta, b - delta) valid
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float up = u_rot(delta, r);
        du[r] += w1 * f[r] * up + w2 * f2[r] * u_rot(16 - delta, r);
        if constexpr (GN) *gn += w1 * f[r] * Q[0][r] * up;
      }
    }
    // keep the fragment reads of at most three diagonals in flight (register pressure)
    if (delta % 3 == 2) asm volatile("" ::: "memory");
  }
}

// ---- kata_bwd_query ------------------------------------------------------------------

template <typename TY>
struct QaIn {
  ChunkIn<BS, bf16> c;   // q, k, v rows of the wave's 16 tokens
  Vec8<TY> gy[2];        // natural column order: lane (t, g) holds columns 32 kk + 8 g + i
};

struct QaRsrc {
  SeqRsrc s;
  __amdgpu_buffer_rsrc_t gy, ih, dq;
};

template <typename TY>
__device__ __forceinline__ void load_qa(QaIn<TY>& r, const QaRsrc& rs, int t0, int wave, int lane) {
  load_chunk<BS, bf16, true>(r.c, rs.s, t0, wave, lane);
  const int n = lane & 15, g = lane >> 4;
  const int t = t0 + wave * 16 + n;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    r.gy[kk].load(rs.gy, (t * 64 + 32 * kk + 8 * g) * (int)sizeof(TY));
  }
}

// grid (n_leaf, B*H), block 256; ws holds each leaf's exclusive prefix of the forward
// state (kata_chunk_state + kata_state_scan).
//
// h_t needs gy_t . y_t = g_t . num_t.  It is formed here from the quantities the walk
// already has, rather than from the forward's rounded y: the inter-chunk part is
// phi(u_t) . (H g_t), the contraction F = H g_t that du needs anyway, and the
// intra-chunk part is sum_s a_ts (g_t . v_s), from the score tile and g_t . v_s.  The
// cancellation in g_t . (v_s - y_t) then happens between consistently rounded terms
// (with the forward's bf16-rounded y the gradient of a short sequence was off by tens of
// percent on some inputs; formed here it stays at the bf16 level for every T).
template <typename TY>
__global__ void __launch_bounds__(256, 2)
kata_bwd_query(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
               const TY* __restrict__ gy, const float* __restrict__ P,
               const float* __restrict__ ws, float* __restrict__ ih, bf16* __restrict__ dq,
               float* __restrict__ dpart, int64_t T, int H,
               int leaf_chunks, int64_t n_chunks) {
  using S = BS;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* vf = reinterpret_cast<bf16*>(smem + QA_OFF_VF);
  bf16* vr = reinterpret_cast<bf16*>(smem + QA_OFF_VR);
  float* Us = reinterpret_cast<float*>(smem + QA_OFF_U);
  float* Ws = reinterpret_cast<float*>(smem + QA_OFF_W);
  float* Wacc = reinterpret_cast<float*>(smem + QA_OFF_WACC);
  bf16* Wz = reinterpret_cast<bf16*>(smem + QA_OFF_WZ);
  bf16* HT = reinterpret_cast<bf16*>(smem + QA_OFF_HT);
  bf16* Zs = reinterpret_cast<bf16*>(smem + QA_OFF_Z);
  bf16* Pf = reinterpret_cast<bf16*>(smem + QA_OFF_PF);
  bf16* PTs = reinterpret_cast<bf16*>(smem + QA_OFF_PT);
  TY* gys = reinterpret_cast<TY*>(smem + QA_OFF_GY);
  constexpr int GYS = QaGy<TY>::STR;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int64_t bh = blockIdx.y;
  const int h = (int)(bh % H);
  const int64_t leaf = blockIdx.x;
  const int64_t c0 = leaf * leaf_chunks;
  const int nch = (int)min<int64_t>(leaf_chunks, n_chunks - c0);
  const int64_t base_tok = bh * T;
  const bool zrole = wave == 0;

  if (wave == 0) write_P<S>(Pf, P, h, lane);
  if (wave == 1) write_pt(PTs, P, h, lane);
  StateAcc<S> st;
  load_state<S>(st, ws + (bh * (int64_t)gridDim.x + leaf) * S::E, wave, zrole, lane);
  auto publish = [&]() {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int nb = 0; nb < S::NB; ++nb) put_ht(HT, wave + 4 * j, nb, st.s[j][nb], lane);
    }
    put_ht(HT, 8, wave, st.s8[0], lane);
    if (zrole) put_z(Zs, st.Z, lane);
  };
  publish();

  QaRsrc rs;
  const int64_t tb = T * 64 * 2;
  rs.s.q = make_rsrc(q + base_tok * 64, tb);
  rs.s.k = make_rsrc(k + base_tok * 64, tb);
  rs.s.v = make_rsrc(v + base_tok * 64, tb);
  rs.gy = make_rsrc(gy + base_tok * 64, T * 64 * (int64_t)sizeof(TY));
  rs.ih = make_rsrc(ih + base_tok * 2, T * 8);
  rs.dq = make_rsrc(dq + base_tok * 64, tb);
  const int tc0 = (int)(c0 * S::C);
  QaIn<TY> cur;
  load_qa<TY>(cur, rs, tc0, wave, lane);
  DPAcc dpa;
#pragma unroll
  for (int db = 0; db < 4; ++db) dpa.t[db] = zero4();
  __syncthreads();   // P fragments, P^T fragments and the first HT / Z written

  for (int c = 0; c < nch; ++c) {
    const int t0 = tc0 + c * S::C;
    progress_priority(c, nch);
    // Lane-derived constants (selectors, masks, addresses) are rebuilt in every chunk
    // from an opaque copy of the lane index: hoisted out of the loop they would not fit
    // in registers next to the state and the prefetched inputs, and spilled values come
    // back from scratch memory with its full latency.
    int lane_o = lane;
    asm volatile("" : "+v"(lane_o));
    const int lane = lane_o;
    const int n = lane & 15, g = lane >> 4;
    {
      const bf16x8 sel[2] = {column_selector(0, lane), column_selector(1, lane)};
      stage_chunk<S, bf16, true>(cur.c, Pf, sel, Us, Ws, Wacc, Wz, vf, nullptr, wave, lane);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      *reinterpret_cast<bf16x8*>(vr + (wave * 16 + n) * BW_GSTR + 32 * kk + 8 * g) = cur.c.v[0][kk].x;
      // this lane's gy columns, read back by the same lane once den_t is known
      TY* gp = gys + (wave * 16 + n) * GYS + 32 * kk + 8 * g;
      if constexpr (sizeof(TY) == 2) {
        *reinterpret_cast<bf16x8*>(gp) = cur.gy[kk].x;
      } else {
        *reinterpret_cast<f32x4*>(gp) = cur.gy[kk].a;
        *reinterpret_cast<f32x4*>(gp + 4) = cur.gy[kk].b;
      }
    }
    const bf16x8 qr[2] = {cur.c.q[0][0].x, cur.c.q[0][1].x};
    if (c + 1 < nch) load_qa<TY>(cur, rs, t0 + S::C, wave, lane);
    __syncthreads();

    // ---- token block mb = wave: den, g, h, du -----------------------------------------
    const int mb = wave;
    const int t = mb * 16 + n;
    f32x4 Q[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) Q[m] = *reinterpret_cast<const f32x4*>(Us + t * S::USTR + 4 * ((g + m) & 3));
    const Op4<true> zf = get_z(Zs, lane);
    float uv[4] = {Q[0][0], Q[0][1], Q[0][2], Q[0][3]};
    const Op4<true> uf = make4<true>(uv);
    const f32x4 zu = mma<true, true>(zf, uf, zero4());      // lane (t, g): (Z u_t)[4g + r]
    float den = zu[0] * Q[0][0] + zu[1] * Q[0][1] + zu[2] * Q[0][2] + zu[3] * Q[0][3];
    f32x4 X[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      X[j] = zero4();
      if (j <= mb) {
        const f32x4 wb = *reinterpret_cast<const f32x4*>(Ws + (j * 16 + n) * S::USTR + 4 * g);
        float wv[4] = {wb[0], wb[1], wb[2], wb[3]};
        X[j] = mma<true, true>(make4<true>(wv), uf, zero4());   // lane (t, g): X[s = 16j + 4g + r][t]
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ok = j < mb || 4 * g + r <= n;
          den += ok ? X[j][r] * X[j][r] : 0.f;
        }
      }
    }
    den = row_pair_sum<16>(den);
    den = row_pair_sum<32>(den);
    const float inv = den != 0.f ? __builtin_amdgcn_rcpf(den) : 0.f;
    float gv[2][8];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const TY* gp = gys + t * GYS + 32 * kk + 8 * g;
      if constexpr (sizeof(TY) == 2) {
        const bf16x8 x = *reinterpret_cast<const bf16x8*>(gp);
#pragma unroll
        for (int i = 0; i < 8; ++i) gv[kk][i] = (float)x[i] * inv;
      } else {
        const f32x4 a = *reinterpret_cast<const f32x4*>(gp), b = *reinterpret_cast<const f32x4*>(gp + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          gv[kk][i] = a[i] * inv;
          gv[kk][4 + i] = b[i] * inv;
        }
      }
    }
    Op8<true> G[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) G[kk] = make8<true>(gv[kk]);

    // g_t . v_s for the chunk's s <= t, and its a_ts-weighted sum (intra part of g_t . num_t)
    f32x4 D[4];
    float gn = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      D[j] = zero4();
      if (j <= mb) {
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          Op8<false> va;
          va.hi = *reinterpret_cast<const bf16x8*>(vr + (j * 16 + n) * BW_GSTR + 32 * kc + 8 * g);
          D[j] = mma<false, true>(va, G[kc], D[j]);    // lane (t, g): g_t . v_{16j + 4g + r}
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ok = j < mb || 4 * g + r <= n;
          gn += ok ? X[j][r] * X[j][r] * D[j][r] : 0.f;
        }
      }
    }
    // inter-chunk S part of du through the HT fragments, and phi(u_t) . (H g_t) into gn
    f32x4 du = zero4();
    const bf16x8 gh[2] = {G[0].hi, G[1].hi};
    ht_contract<true>(du, &gn, HT, gh, Q, lane);
    gn = row_pair_sum<16>(gn);
    gn = row_pair_sum<32>(gn);
    const float hh = -gn * inv;                          // h_t = -(g_t . num_t) / den_t
    if (g == 0) {
      const i32x2 ihv = {__float_as_int(inv), __float_as_int(hh)};
      __builtin_amdgcn_raw_buffer_store_b64(ihv, rs.ih, (t0 + t) * 8, 0, 0);
    }

    // intra-chunk: B_ts = 2 X_ts (g_t . v_s + h_t) for s <= t; du_t += sum_s B_ts w_s
    f32x4 Bm[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = j < mb || (j == mb && 4 * g + r <= n);
        Bm[j][r] = ok ? 2.f * (D[j][r] + hh) * X[j][r] : 0.f;
      }
    }
#pragma unroll
    for (int jj = 0; jj < S::NJ; ++jj) {
      if (2 * jj <= mb) {
        Op8<true> wz;
        wz.hi = *reinterpret_cast<const bf16x8*>(Wz + (jj * WAVE + lane) * 8);
        wz.lo = *reinterpret_cast<const bf16x8*>(Wz + ((S::NJ + jj) * WAVE + lane) * 8);
        float bx[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          bx[r] = Bm[2 * jj][r];
          bx[4 + r] = Bm[2 * jj + 1][r];
        }
        du = mma<true, false>(wz, make8<false>(bx), du);   // lane (t, g): du_t[4g + r]
      }
    }
    // inter-chunk z part: 2 h_t Z u_t
#pragma unroll
    for (int r = 0; r < 4; ++r) du[r] += 2.f * hh * zu[r];

    grad_head(du, PTs, qr, rs.dq, ((t0 + t) * 64) * 2, dpa, lane);

    const bool more = c + 1 < nch;
    if (more) state_update<S>(st, Wacc, Wz, vf, nullptr, wave, zrole, lane);
    __syncthreads();
    if (more) publish();
  }
  float* red = reinterpret_cast<float*>(smem + QA_OFF_HT);   // HT is no longer read
  write_dp_partial(dpa, true, wave, red, dpart + (bh * (int64_t)gridDim.x + leaf) * BW_DP, tid, lane);
}

// ---- kata_bwd_rstate ----------------------------------------------------------------
// grid (n_leaf, B*H), block 256.  Per leaf, sum over its tokens of phi(u_t) [g_t | h_t]:
// the packed S part accumulates phi(u) g^T exactly as kata_chunk_state accumulates
// phi(w) v^T (u plays the key, the hi plane of g the value), and the z part is the
// 16 x 16 matrix sum_t h_t u_t u_t^T.  g_t = gy_t (1/den_t) is formed from gy and the
// (1/den_t, h_t) pairs of kata_bwd_query, as that kernel formed it.  Layout of ws as for
// kata_chunk_state.
template <typename TY>
__global__ void __launch_bounds__(256, 3)
kata_bwd_rstate(const bf16* __restrict__ q, const TY* __restrict__ gy, const float* __restrict__ ih,
                const float* __restrict__ P, float* __restrict__ ws, int64_t T, int H, int leaf_chunks,
                int64_t n_chunks) {
  using S = BS;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* vf = reinterpret_cast<bf16*>(smem + RS_OFF_VF);
  float* Wacc = reinterpret_cast<float*>(smem + RS_OFF_WACC);
  bf16* Wz = reinterpret_cast<bf16*>(smem + RS_OFF_WZ);
  bf16* Pf = reinterpret_cast<bf16*>(smem + RS_OFF_PF);
  float* hs = reinterpret_cast<float*>(smem + RS_OFF_HS);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int64_t bh = blockIdx.y;
  const int h = (int)(bh % H);
  const int64_t leaf = blockIdx.x;
  const int64_t c0 = leaf * leaf_chunks;
  const int nch = (int)min<int64_t>(leaf_chunks, n_chunks - c0);
  const int64_t base_tok = bh * T;

  if (wave == 0) write_P<S>(Pf, P, h, lane);
  const bf16x8 sel[2] = {column_selector(0, lane), column_selector(1, lane)};
  StateAcc<S> st;
  state_zero<S>(st);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + base_tok * 64, T * 64 * 2);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(gy + base_tok * 64, T * 64 * (int64_t)sizeof(TY));
  const __amdgpu_buffer_rsrc_t rih = make_rsrc(ih + base_tok * 2, T * 8);
  struct In {
    Vec8<bf16> x[2];   // q rows, projection column order
    Vec8<TY> gy[2];    // gy rows, natural column order
    i32x2 ih;          // (1/den, h) of token n
  };
  auto load_in = [&](In& r, int t0) {
    const int t = t0 + wave * 16 + n;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      r.x[kk].load(rq, (t * 64 + 16 * g + 8 * kk) * 2);
      r.gy[kk].load(rg, (t * 64 + 32 * kk + 8 * g) * (int)sizeof(TY));
    }
    r.ih = __builtin_amdgcn_raw_buffer_load_b64(rih, t * 8, 0, 0);
  };
  const int tc0 = (int)(c0 * S::C);
  In in;
  load_in(in, tc0);
  __syncthreads();   // P fragments written
  for (int c = 0; c < nch; ++c) {
    const int t0 = tc0 + c * S::C;
    ChunkIn<S, bf16> cur;   // u plays the key, the hi part of g the value
    const float inv = __int_as_float(in.ih[0]);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      cur.k[0][kk] = in.x[kk];
#pragma unroll
      for (int i = 0; i < 8; ++i) cur.v[0][kk].x[i] = (bf16)(in.gy[kk][i] * inv);
    }
    stage_chunk<S, bf16, false>(cur, Pf, sel, nullptr, nullptr, Wacc, Wz, vf, nullptr, wave, lane);
    if (g == 0) hs[wave * 16 + n] = __int_as_float(in.ih[1]);
    if (c + 1 < nch) load_in(in, t0 + S::C);
    __syncthreads();
    state_update<S>(st, Wacc, Wz, vf, nullptr, wave, false, lane);
    if (wave == 0) {   // Z += U^T diag(h) U, hi/lo operands
#pragma unroll
      for (int jj = 0; jj < S::NJ; ++jj) {
        const f32x4 u0 = *reinterpret_cast<const f32x4*>(Wacc + ((2 * jj) * WAVE + lane) * 4);
        const f32x4 u1 = *reinterpret_cast<const f32x4*>(Wacc + ((2 * jj + 1) * WAVE + lane) * 4);
        const f32x4 h0 = *reinterpret_cast<const f32x4*>(hs + 32 * jj + 4 * g);
        const f32x4 h1 = *reinterpret_cast<const f32x4*>(hs + 32 * jj + 16 + 4 * g);
        float ua[8], uh[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          ua[r] = u0[r];
          ua[4 + r] = u1[r];
          uh[r] = u0[r] * h0[r];
          uh[4 + r] = u1[r] * h1[r];
        }
        st.Z = mma<true, true>(make8<true>(ua), make8<true>(uh), st.Z);
      }
    }
    __syncthreads();
  }
  float* out = ws + (bh * (int64_t)gridDim.x + leaf) * S::E;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int delta = wave + 4 * j;
#pragma unroll
    for (int nb = 0; nb < S::NB; ++nb)
      *reinterpret_cast<f32x4*>(out + ws_tile_offset<S>(delta, nb, lane)) = st.s[j][nb];
  }
  *reinterpret_cast<f32x4*>(out + ws_tile_offset<S>(8, wave, lane)) = st.s8[0];
  if (wave == 0) *reinterpret_cast<f32x4*>(out + DPACK * S::DV + lane * 4) = st.Z;
}

// ---- kata_bwd_key --------------------------------------------------------------------
// grid (n_leaf, B*H), block 512 (8 waves).  ws holds each leaf's exclusive SUFFIX of the
// backward state [R | Zr] (kata_bwd_rstate + reverse kata_state_scan).  Waves 0..3
// (role 0) compute dv of the 16-token key block mb = wave, waves 4..7 (role 1) dw of key
// block mb = 7 - wave.  dk = P^T dw and the dP share dw k^T are formed by role 0 one
// chunk later, from dw handed over in LDS (two buffers), which balances the two roles
// without another barrier.  The state is owned by diagonal: wave w holds delta = w for
// all column blocks, waves 4..7 also delta = 8 for column block w - 4, wave 0 the
// z-matrix.  Chunks are walked from the leaf's last to its first.
struct KbState {
  f32x4 s[4];
  f32x4 s8;
  f32x4 Z;
};

template <typename TY>
__global__ void __launch_bounds__(512, 2)
kata_bwd_key(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
             const TY* __restrict__ gy, const float* __restrict__ ih,
             const float* __restrict__ P, const float* __restrict__ ws, bf16* __restrict__ dk,
             bf16* __restrict__ dv, float* __restrict__ dpart, int64_t T, int H, int leaf_chunks,
             int64_t n_chunks) {
  using S = BS;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* hx = reinterpret_cast<bf16*>(smem + KB_OFF_HX);
  bf16* HT = reinterpret_cast<bf16*>(smem + KB_OFF_HT);
  bf16* Zs = reinterpret_cast<bf16*>(smem + KB_OFF_Z);
  bf16* gf = reinterpret_cast<bf16*>(smem + KB_OFF_GF);
  bf16* grh = reinterpret_cast<bf16*>(smem + KB_OFF_GRH);
  bf16* grl = reinterpret_cast<bf16*>(smem + KB_OFF_GRL);
  float* Us = reinterpret_cast<float*>(smem + KB_OFF_U);
  float* Ws = reinterpret_cast<float*>(smem + KB_OFF_W);
  float* Uacc = reinterpret_cast<float*>(smem + KB_OFF_UACC);
  float* hs = reinterpret_cast<float*>(smem + KB_OFF_HS);
  bf16* Pf = reinterpret_cast<bf16*>(smem + KB_OFF_PF);
  bf16* PTs = reinterpret_cast<bf16*>(smem + KB_OFF_PT);
  float* dWs = reinterpret_cast<float*>(smem + KB_OFF_DW);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // key block of the wave: role 0 takes block w, role 1 block 3 - (w - 4), so that each
  // SIMD (waves w and w + 4) pairs a block with many later query tiles with one with few
  const int role = wave >> 2, mb = role == 0 ? wave : 3 - (wave & 3);
  const int n = lane & 15, g = lane >> 4;
  const int64_t bh = blockIdx.y;
  const int h = (int)(bh % H);
  const int64_t leaf = blockIdx.x;
  const int64_t c0 = leaf * leaf_chunks;
  const int nch = (int)min<int64_t>(leaf_chunks, n_chunks - c0);
  const int64_t base_tok = bh * T;

  // the readout K-block 4 holds delta = 8 in slots 0..3; slots 4..7 stay zero
  for (int i = tid; i < S::NB * WAVE; i += 512) {
    const int idx = ((4 * S::NB) * WAVE + i) * 8 + 4;
    *reinterpret_cast<bf16x4*>(hx + idx) = bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
  }
  if (wave == 0) write_P<S>(Pf, P, h, lane);
  if (wave == 1) write_pt(PTs, P, h, lane);

  KbState st;
  {
    const float* in = ws + (bh * (int64_t)gridDim.x + leaf) * S::E;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) st.s[nb] = *reinterpret_cast<const f32x4*>(in + ws_tile_offset<S>(wave, nb, lane));
    st.s8 = wave >= 4 ? *reinterpret_cast<const f32x4*>(in + ws_tile_offset<S>(8, wave - 4, lane)) : zero4();
    st.Z = wave == 0 ? *reinterpret_cast<const f32x4*>(in + DPACK * S::DV + lane * 4) : zero4();
  }
  auto publish = [&]() {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      put_hx(hx, wave, nb, st.s[nb], lane);
      put_ht(HT, wave, nb, st.s[nb], lane);
    }
    if (wave >= 4) {
      put_hx(hx, 8, wave - 4, st.s8, lane);
      put_ht(HT, 8, wave - 4, st.s8, lane);
    }
    if (wave == 0) put_z(Zs, st.Z, lane);
  };
  publish();

  // role 0 loads k (-> w; kept for dk and dP), role 1 q (-> u); both load v, gy and the
  // (1/den, h) pairs and form g = gy (1/den) as kata_bwd_query did: role 0 stages its hi
  // part (G^T fragments, G rows) and h, role 1 the lo part (G rows).
  const int64_t tb = T * 64 * 2;
  const __amdgpu_buffer_rsrc_t r_x = make_rsrc((role == 0 ? k : q) + base_tok * 64, tb);
  const __amdgpu_buffer_rsrc_t r_g = make_rsrc(gy + base_tok * 64, T * 64 * (int64_t)sizeof(TY));
  const __amdgpu_buffer_rsrc_t r_v = make_rsrc(v + base_tok * 64, tb);
  const __amdgpu_buffer_rsrc_t r_ih = make_rsrc(ih + base_tok * 2, T * 8);
  const __amdgpu_buffer_rsrc_t r_dv = make_rsrc(dv + base_tok * 64, tb);
  const __amdgpu_buffer_rsrc_t r_dk = make_rsrc(dk + base_tok * 64, tb);
  struct In {
    Vec8<bf16> x[2];   // k or q rows, projection column order
    Vec8<TY> gg[2];    // gy rows, natural column order
    Vec8<bf16> vv[2];  // v rows, natural column order
    i32x2 ih;          // (1/den, h) of token n
  };
  auto load_in = [&](In& r, int t0) {
    const int t = t0 + mb * 16 + n;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      r.x[kk].load(r_x, (t * 64 + 16 * g + 8 * kk) * 2);
      r.gg[kk].load(r_g, (t * 64 + 32 * kk + 8 * g) * (int)sizeof(TY));
        r.vv[kk].load(r_v, (t * 64 + 32 * kk + 8 * g) * 2);
    }
    r.ih = __builtin_amdgcn_raw_buffer_load_b64(r_ih, t * 8, 0, 0);
  };
  DPAcc dpa;
#pragma unroll
  for (int db = 0; db < 4; ++db) dpa.t[db] = zero4();
  // role 0: dk = P^T dw and dP += dw k^T for the key block of an earlier chunk; dw is
  // role 1's part (LDS) plus the part of the state contraction role 0 took itself
  auto key_grad = [&](int tprev, int buf, const bf16x8 (&krows)[2], const f32x4& own) {
    const int s_loc = mb * 16 + n;
    f32x4 dwv = *reinterpret_cast<const f32x4*>(dWs + (buf * S::C + s_loc) * P_DIM + 4 * g);
    dwv += own;
    grad_head(dwv, PTs, krows, r_dk, ((tprev + s_loc) * 64) * 2, dpa, lane);
  };
  // split of the dw state contraction over the diagonals: role 1 takes delta < KB_DSPLIT
  constexpr int KB_DSPLIT = 6;
  const int tc0 = (int)(c0 * S::C);
  auto chunk_t0 = [&](int c) { return tc0 + (nch - 1 - c) * S::C; };   // last chunk first
  In cur;
  load_in(cur, chunk_t0(0));
  bf16x8 kprev[2];   // role 0: k rows of the previous chunk
  f32x4 dwprev = zero4();   // role 0: its share of the previous chunk's dw
  __syncthreads();   // P and P^T fragments, hx zeros, first publish

  for (int c = 0; c < nch; ++c) {
    const int t0 = chunk_t0(c);
    progress_priority(c, nch);
    // lane-derived constants rebuilt per chunk (not hoisted and spilled), as in the query walk
    int lane_o = lane;
    asm volatile("" : "+v"(lane_o));
    const int lane = lane_o;
    const int n = lane & 15, g = lane >> 4;
    // ---- stage ----
    ProjP<S> pp;
    read_P<S>(pp, Pf, lane);
    const f32x4 x = project_tile<S, bf16>(cur.x, pp);      // lane (a, g): x-projection of token 4g + r
    const bf16x8 kcur[2] = {cur.x[0].x, cur.x[1].x};
    Vec8<bf16> vcur[2] = {cur.vv[0], cur.vv[1]};
    Op8<true> gsp[2];   // g = gy (1/den) of this lane's token and columns, hi/lo
    {
      const float inv = __int_as_float(cur.ih[0]);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float gv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) gv[i] = cur.gg[kk][i] * inv;
        gsp[kk] = make8<true>(gv);
      }
    }
    const float hcur = __int_as_float(cur.ih[1]);
    if (role == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) Ws[(mb * 16 + 4 * g + r) * S::USTR + n] = x[r];
      Vec8<bf16> gh[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        gh[kk].x = gsp[kk].hi;
        *reinterpret_cast<bf16x8*>(grh + (mb * 16 + n) * BW_GSTR + 32 * kk + 8 * g) = gsp[kk].hi;
      }
      const bf16x8 sel[2] = {column_selector(0, lane), column_selector(1, lane)};
      stage_v<S, bf16>(gh, mb, sel, gf, nullptr, lane);
      if (g == 0) hs[mb * 16 + n] = hcur;
    } else {
      *reinterpret_cast<f32x4*>(Uacc + (mb * WAVE + lane) * 4) = x;
#pragma unroll
      for (int r = 0; r < 4; ++r) Us[(mb * 16 + 4 * g + r) * S::USTR + n] = x[r];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        *reinterpret_cast<bf16x8*>(grl + (mb * 16 + n) * BW_GSTR + 32 * kk + 8 * g) = gsp[kk].lo;
    }
    if (c + 1 < nch) load_in(cur, chunk_t0(c + 1));
    __syncthreads();

    // ---- key block mb ----
    const int s_loc = mb * 16 + n;
    f32x4 Q[4];   // rotated quads of w_s
#pragma unroll
    for (int m = 0; m < 4; ++m) Q[m] = *reinterpret_cast<const f32x4*>(Ws + s_loc * S::USTR + 4 * ((g + m) & 3));
    float wv[4] = {Q[0][0], Q[0][1], Q[0][2], Q[0][3]};
    const Op4<true> wf = make4<true>(wv);
    f32x4 X[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      X[j] = zero4();
      if (j >= mb) {
        const f32x4 ub = *reinterpret_cast<const f32x4*>(Us + (j * 16 + n) * S::USTR + 4 * g);
        float uvv[4] = {ub[0], ub[1], ub[2], ub[3]};
        X[j] = mma<true, true>(make4<true>(uvv), wf, zero4());   // lane (s, g): X[t = 16j + 4g + r][s]
      }
    }
    if (role == 0) {
      // dv_s = R^T phi(w_s) (readout of the later chunks) + sum_{t >= s} a_ts g_t
      auto w_rot = [&](int delta, int i) -> float {
        const int m = delta >> 2, e = delta & 3;
        const int j = i + e;
        return j < 4 ? Q[m & 3][j] : Q[(m + 1) & 3][j - 4];
      };
      f32x4 wa2, wa8;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wa2[i] = 2.f * Q[0][i];
        wa8[i] = g < 2 ? wa2[i] : 0.f;
      }
      f32x4 O[S::NB];
#pragma unroll
      for (int nb = 0; nb < S::NB; ++nb) O[nb] = zero4();
#pragma unroll
      for (int kb = 0; kb < READ_KB; ++kb) {
        float xx[8];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int delta = 2 * kb + half;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (delta <= 8) {
              const f32x4& wa = delta == 0 ? Q[0] : (delta == 8 ? wa8 : wa2);
              xx[half * 4 + i] = wa[i] * w_rot(delta, i);
            } else {
              xx[half * 4 + i] = 0.f;
            }
          }
        }
        const Op8<false> qf = make8<false>(xx);
#pragma unroll
        for (int nb = 0; nb < S::NB; ++nb) {
          Op8<false> hf;
          hf.hi = *reinterpret_cast<const bf16x8*>(hx + ((kb * S::NB + nb) * WAVE + lane) * 8);
          O[nb] = mma<false, false>(hf, qf, O[nb]);
        }
      }
      f32x4 A2[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ok = j > mb || (j == mb && 4 * g + r >= n);
          A2[j][r] = ok ? X[j][r] * X[j][r] : 0.f;
        }
      }
#pragma unroll
      for (int jj = 0; jj < S::NJ; ++jj) {
        if (2 * jj + 1 >= mb) {
          float xx[8];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            xx[r] = A2[2 * jj][r];
            xx[4 + r] = A2[2 * jj + 1][r];
          }
          const Op8<false> af = make8<false>(xx);
#pragma unroll
          for (int nb = 0; nb < S::NB; ++nb)
            O[nb] = mma<false, false>(load_vf<S>(gf, nullptr, jj, nb, lane), af, O[nb]);
        }
      }
      store_row<S, bf16>(O, 1.f, r_dv, (t0 + s_loc) * 64, s_loc, g);   // whole 128-byte rows
      if (c > 0) key_grad(chunk_t0(c - 1), (c - 1) & 1, kprev, dwprev);
      kprev[0] = kcur[0];
      kprev[1] = kcur[1];
      // this chunk's share of the dw state contraction (diagonals KB_DSPLIT..8)
      dwprev = zero4();
      const bf16x8 vx[2] = {vcur[0].x, vcur[1].x};
      ht_contract<false, KB_DSPLIT, NDELTA>(dwprev, nullptr, HT, vx, Q, lane);
    } else {
      // dw_s = sum_{t >= s} B_ts u_t + 2 (mat(R v_s) + Zr) w_s; dk = P^T dw; dP += dw k^T
      f32x4 Bm[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        Bm[j] = zero4();
        if (j >= mb) {
          f32x4 d = zero4();
#pragma unroll
          for (int kc = 0; kc < 2; ++kc) {
            Op8<true> ga;
            ga.hi = *reinterpret_cast<const bf16x8*>(grh + (j * 16 + n) * BW_GSTR + 32 * kc + 8 * g);
            ga.lo = *reinterpret_cast<const bf16x8*>(grl + (j * 16 + n) * BW_GSTR + 32 * kc + 8 * g);
            Op8<false> vb;
            vb.hi = vcur[kc].x;
            d = mma<true, false>(ga, vb, d);           // lane (s, g): g_{16j + 4g + r} . v_s
          }
          const f32x4 hv = *reinterpret_cast<const f32x4*>(hs + j * 16 + 4 * g);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool ok = j > mb || 4 * g + r >= n;
            Bm[j][r] = ok ? 2.f * (d[r] + hv[r]) * X[j][r] : 0.f;
          }
        }
      }
      f32x4 dw = zero4();
#pragma unroll
      for (int jj = 0; jj < S::NJ; ++jj) {
        if (2 * jj + 1 >= mb) {
          const f32x4 u0 = *reinterpret_cast<const f32x4*>(Uacc + ((2 * jj) * WAVE + lane) * 4);
          const f32x4 u1 = *reinterpret_cast<const f32x4*>(Uacc + ((2 * jj + 1) * WAVE + lane) * 4);
          float ua[8], bx[8];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            ua[r] = u0[r];
            ua[4 + r] = u1[r];
            bx[r] = Bm[2 * jj][r];
            bx[4 + r] = Bm[2 * jj + 1][r];
          }
          dw = mma<true, false>(make8<true>(ua), make8<false>(bx), dw);   // lane (s, g): dw_s[4g + r]
        }
      }
      const f32x4 zw = mma<true, true>(get_z(Zs, lane), wf, zero4());   // (Zr w_s)[4g + r]
#pragma unroll
      for (int r = 0; r < 4; ++r) dw[r] += 2.f * zw[r];
      const bf16x8 vx[2] = {vcur[0].x, vcur[1].x};
      ht_contract<false, 0, KB_DSPLIT>(dw, nullptr, HT, vx, Q, lane);
      *reinterpret_cast<f32x4*>(dWs + ((c & 1) * S::C + s_loc) * P_DIM + 4 * g) = dw;
    }

    // ---- state update: R += phi(U_c)^T G_c, Zr += U_c^T diag(h_c) U_c ----
    const bool more = c + 1 < nch;
    if (more) {
      const int rot_lane = (lane & ~15) | ((lane + wave) & 15);
#pragma unroll
      for (int jj = 0; jj < S::NJ; ++jj) {
        const f32x4 wa0 = *reinterpret_cast<const f32x4*>(Uacc + ((2 * jj) * WAVE + lane) * 4);
        const f32x4 wa1 = *reinterpret_cast<const f32x4*>(Uacc + ((2 * jj + 1) * WAVE + lane) * 4);
        const f32x4 wr0 = *reinterpret_cast<const f32x4*>(Uacc + ((2 * jj) * WAVE + rot_lane) * 4);
        const f32x4 wr1 = *reinterpret_cast<const f32x4*>(Uacc + ((2 * jj + 1) * WAVE + rot_lane) * 4);
        Op8<false> vfr[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) vfr[nb] = load_vf<S>(gf, nullptr, jj, nb, lane);
        {
          const Op8<false> kf = key_frag<S, 0>(wa0, wa1, wr0, wr1);      // delta = wave
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) st.s[nb] = mma<false, false>(kf, vfr[nb], st.s[nb]);
        }
        if (wave >= 4) {
          const Op8<false> kf = key_frag<S, 8>(wa0, wa1, wa0, wa1);      // delta = 8
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            if (nb == wave - 4) st.s8 = mma<false, false>(kf, vfr[nb], st.s8);
        }
        if (wave == 0) {
          const f32x4 h0 = *reinterpret_cast<const f32x4*>(hs + 32 * jj + 4 * g);
          const f32x4 h1 = *reinterpret_cast<const f32x4*>(hs + 32 * jj + 16 + 4 * g);
          float ua[8], uh[8];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            ua[r] = wa0[r];
            ua[4 + r] = wa1[r];
            uh[r] = wa0[r] * h0[r];
            uh[4 + r] = wa1[r] * h1[r];
          }
          st.Z = mma<true, true>(make8<true>(ua), make8<true>(uh), st.Z);
        }
      }
    }
    __syncthreads();
    if (more) publish();
  }
  // the last chunk's dk (its dw was written before the loop's final barrier)
  if (role == 0) key_grad(chunk_t0(nch - 1), (nch - 1) & 1, kprev, dwprev);
  float* red = reinterpret_cast<float*>(smem + KB_OFF_HX);   // hx is no longer read
  write_dp_partial(dpa, role == 0, mb, red, dpart + (bh * (int64_t)gridDim.x + leaf) * BW_DP, tid, lane);
}

// ---- kata_bwd_dp_reduce --------------------------------------------------------------
// grid (H, 4), block 256: dP[h][e] = sum over batch rows b and leaves of both partials.
__global__ void __launch_bounds__(256)
kata_bwd_dp_reduce(const float* __restrict__ pa, const float* __restrict__ pb, float* __restrict__ dP, int64_t B,
                   int H, int64_t n_leaf) {
  const int h = blockIdx.x;
  const int e = blockIdx.y * 256 + threadIdx.x;
  float s = 0.f;
  for (int64_t b = 0; b < B; ++b) {
    const int64_t base = ((b * H + h) * n_leaf) * BW_DP + e;
    for (int64_t l = 0; l < n_leaf; ++l) s += pa[base + l * BW_DP] + pb[base + l * BW_DP];
  }
  dP[(int64_t)h * BW_DP + e] = s;
}

}  // namespace kata
