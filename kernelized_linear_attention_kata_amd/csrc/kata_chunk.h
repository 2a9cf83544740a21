// kata_chunk.h - chunk-level kernels of the KATA causal forward on gfx950:
//   kata_chunk_state  : per leaf of chunks, sum of the chunk states phi(K_c)^T [V_c | 1]
//   kata_chunk_intra  : per leaf, for every chunk: prefix-state readout phi(Q_c) H_c,
//                       masked squared score tile (U_c W_c^T)^2 times [V_c | 1], output
//                       gate (the division), and the running state update H += phi(K_c)^T [V_c|1]
// The chunked-state decomposition follows the hardware section of the gist.science
// summary of "Kernelized Linear Attention" (arXiv 2607.17419, section 2.3: intra-chunk
// work on matrix cores, inter-chunk state propagated by an associative scan) and the
// exactness of that O(T) form stated in the paper's abstract.
//
// Work decomposition of one 256-thread workgroup (4 waves) over a chunk of C tokens:
//  * token split  : wave w owns the 16-token M-blocks mb = w, w+4, ... < C/16 for the
//                   projection u = P q, w = P k, the readout, the intra tile and y.
//  * feature split: the packed state H (144 feature rows x dv columns, see below) is
//                   held in MFMA accumulators; wave w owns rows of diagonals delta = w
//                   and w+4 for every column block and, for delta = 8, the column blocks
//                   nb = w (mod 4).  After each update the owners publish H as bf16 MFMA
//                   B-fragments in LDS for the next chunk's readout.
//
// Packed symmetric feature ("circulant" order): slot (delta, a) = 16*delta + a holds
// u_a * u_{(a+delta) mod 16} for delta = 0..8 (for delta = 8 only a < 8 is distinct;
// slots a >= 8 are zero).  The 136 distinct entries of the symmetric u u^T are thus
// stored once; the query side carries weight 2 off the diagonal so the packed inner
// product equals the full one.  The rotation structure lets every lane build its
// fragment from four 16-byte reads of its own token's u (no per-lane gathers).
#pragma once

#include "kata_common.h"
#include "kata_scan.h"

namespace kata {

// Compile-time shape of one kernel instance.
// SPLIT (fp32 inputs): every operand hi/lo bf16, V included.  PREC (bf16 inputs): the
// feature operands phi(k), phi(q) and the published state H hi/lo (V, exact in bf16, and
// the squared scores stay single): the readout phi(q)^T H of a query whose denominator is
// a small fraction of sum_s |u|^2 |w_s|^2 then keeps about 16 significant bits instead of 8.
template <int C_, int DIN_, int DV_, bool SPLIT_, bool PREC_ = false>
struct Shape {
  static constexpr int C = C_;          // chunk length (32, 64, 128)
  static constexpr int DIN = DIN_;      // q/k head dim (16 or 64)
  static constexpr int DV = DV_;        // value head dim (16 or 64)
  static constexpr bool SPLIT = SPLIT_; // fp32 inputs: hi/lo bf16 operands
  static constexpr bool FSPLIT = SPLIT_ || PREC_;   // hi/lo features and published state
  static constexpr int NB = DV / 16;    // value column blocks
  static constexpr int NMB = C / 16;    // 16-token M-blocks per chunk
  static constexpr int NJ = C / 32;     // 32-token K-blocks per chunk
  static constexpr int KD = DIN >= 32 ? DIN / 32 : 1;   // projection K-blocks
  static constexpr int KV = DV >= 32 ? DV / 32 : 1;     // value-row K-blocks (transpose)
  static constexpr int MBW = (NMB + 3) / 4;             // M-blocks per wave (max)
  static constexpr int USTR = 20;       // LDS row stride (floats) of U and W rows
  // LDS footprint (bytes)
  static constexpr int VF_BYTES = C * DV * 2;                 // V as bf16 B-fragments
  static constexpr int HX_BYTES = READ_KB * NB * WAVE * 16;   // H as bf16 readout fragments
  static constexpr int U_BYTES = C * USTR * 4;                // u rows (fp32), W rows likewise
  static constexpr int WACC_BYTES = NMB * WAVE * 16;          // w tiles in accumulator layout
  static constexpr int WZ_BYTES = 2 * NJ * WAVE * 16;         // w tiles as hi/lo bf16 K-block fragments
  static constexpr int Z_BYTES = WAVE * 16;                   // Z (16 x 16) as hi/lo bf16 A-fragments
  static constexpr int PF_BYTES = KD * 2 * WAVE * 16;         // P as hi/lo projection B-fragments
  static constexpr int NSPLIT = SPLIT ? 2 : 1;      // planes of V
  static constexpr int NFSPLIT = FSPLIT ? 2 : 1;    // planes of H
  static constexpr int OFF_VF = 0;
  static constexpr int OFF_HX = OFF_VF + NSPLIT * VF_BYTES;
  static constexpr int OFF_U = OFF_HX + NFSPLIT * HX_BYTES;
  static constexpr int OFF_W = OFF_U + U_BYTES;
  static constexpr int OFF_WACC = OFF_W + U_BYTES;
  static constexpr int OFF_WZ = OFF_WACC + WACC_BYTES;
  static constexpr int OFF_Z = OFF_WZ + WZ_BYTES;
  static constexpr int OFF_PF = OFF_Z + Z_BYTES;
  static constexpr int SMEM = OFF_PF + PF_BYTES;
  // kata_chunk_state needs only the V fragments, the w tiles and the constants
  static constexpr int ST_OFF_WACC = NSPLIT * VF_BYTES;
  static constexpr int ST_OFF_WZ = ST_OFF_WACC + WACC_BYTES;
  static constexpr int ST_OFF_PF = ST_OFF_WZ + WZ_BYTES;
  static constexpr int SMEM_STATE = ST_OFF_PF + PF_BYTES;
  // decay-gated instances append the chunk's cumulative log-decays and the key weights
  // of the state update (two floats per token) after the layouts above
  static constexpr int DEC_BYTES = 2 * C * 4;
  // waves per SIMD each kernel is compiled for (register budget 512 / OCC): the
  // largest that fits without spilling on gfx950
  static constexpr int OCC_INTRA = DV <= 16 ? (C == 128 ? 3 : 4) : ((FSPLIT || C == 128) ? 2 : 3);
  static constexpr int OCC_STATE = DV <= 16 ? 4 : (SPLIT ? 2 : 3);
  // workspace block per leaf: packed S in accumulator-tile order, then the 16 x 16
  // normaliser matrix Z = sum w w^T (z = vec(Z)) as one accumulator tile
  static constexpr int E = DPACK * DV + P_DIM * P_DIM;
  static_assert(C == 32 || C == 64 || C == 128, "chunk");
  static_assert(DV % 16 == 0 && DV <= 128, "dv");
  static_assert(DIN == 16 || DIN % 32 == 0, "d");
  // three workgroups of the bf16 C = 64, dv = 64 instance share a CU (156 KiB of LDS)
  static_assert(!(C == 64 && DV == 64 && !FSPLIT) || 3 * (SMEM + DEC_BYTES) <= 156 * 1024, "LDS budget");
};

// Offsets of an accumulator tile (delta, nb) inside a leaf's workspace block:
// tile index delta*NB + nb, 256 floats per tile, lane-major, 4 floats per lane.
template <class S>
__device__ __forceinline__ int ws_tile_offset(int delta, int nb, int lane) {
  return ((delta * S::NB + nb) * WAVE + lane) * 4;
}

// ---- per-chunk input staging ---------------------------------------------------

// 8 consecutive input elements, loaded as 16-byte vectors through a buffer resource.
template <typename TIn> struct Vec8;
template <> struct Vec8<bf16> {
  bf16x8 x;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int off) {
    x = __builtin_bit_cast(bf16x8, buf_load16(r, off));
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (bf16)0.f;
  }
  __device__ __forceinline__ float operator[](int i) const { return (float)x[i]; }
};
template <> struct Vec8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int off) {
    a = __builtin_bit_cast(f32x4, buf_load16(r, off));
    b = __builtin_bit_cast(f32x4, buf_load16(r, off >= BUF_OOB ? off : off + 16));
  }
  __device__ __forceinline__ void zero() { a = zero4(); b = zero4(); }
  __device__ __forceinline__ float operator[](int i) const { return i < 4 ? a[i] : b[i - 4]; }
};

// Buffer resources over one (b, h) sequence of q, k, v and y.
struct SeqRsrc {
  __amdgpu_buffer_rsrc_t q, k, v, y;
};

// Register-resident copy of one chunk's inputs for this thread: the q/k/v rows of
// the wave's 16-token M-blocks, laid out as MFMA A-fragments (lane = token row).
template <class S, typename TIn>
struct ChunkIn {
  Vec8<TIn> q[S::MBW][S::KD];
  Vec8<TIn> k[S::MBW][S::KD];
  Vec8<TIn> v[S::MBW][S::KV];
};

// projection K-slot -> input column: lane group g, K-block kk, slot i
template <class S>
__device__ __forceinline__ int proj_col(int g, int kk, int i) {
  if constexpr (S::DIN == 16) return 8 * g + i;          // one K-block, lanes g >= 2 padded
  else return 16 * g + 8 * kk + i;                        // each lane reads 16 contiguous
}
template <class S>
__device__ __forceinline__ bool proj_valid(int g) {
  if constexpr (S::DIN == 16) return g < 2;
  else return true;
}

// Load the wave's q/k/v rows of the chunk starting at token t0 (within the sequence).
// Rows at or past T fall outside the buffer and read as zero (no branches, so the
// compiler can track the outstanding loads of each prefetch buffer exactly).
template <class S, typename TIn, bool WANT_Q>
__device__ __forceinline__ void load_chunk(ChunkIn<S, TIn>& r, const SeqRsrc& rs, int t0, int tw, int lane) {
  const int n = lane & 15, g = lane >> 4;
  constexpr int ES = (int)sizeof(TIn);
#pragma unroll
  for (int m = 0; m < S::MBW; ++m) {
    const int mb = tw + 4 * m;
    if (S::NMB >= 4 * (m + 1) || mb < S::NMB) {       // wave-uniform
      const int t = t0 + mb * 16 + n;
#pragma unroll
      for (int kk = 0; kk < S::KD; ++kk) {
        const int off = proj_valid<S>(g) ? (t * S::DIN + proj_col<S>(g, kk, 0)) * ES : BUF_OOB;
        if constexpr (WANT_Q) r.q[m][kk].load(rs.q, off);
        r.k[m][kk].load(rs.k, off);
      }
#pragma unroll
      for (int kk = 0; kk < S::KV; ++kk) {
        const int off = (S::DV >= 32 || g < 2) ? (t * S::DV + 32 * kk + 8 * g) * ES : BUF_OOB;
        r.v[m][kk].load(rs.v, off);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < S::KD; ++kk) {
        if constexpr (WANT_Q) r.q[m][kk].zero();
        r.k[m][kk].zero();
      }
#pragma unroll
      for (int kk = 0; kk < S::KV; ++kk) r.v[m][kk].zero();
    }
  }
}

// V as MFMA B-fragments in LDS: Vf[jj][nb][lane][slot], lane = 16g + n holds column
// 16nb + n and, for the 32-token K-block jj, tokens 4g..4g+3 in slots 0..3 and
// 16+4g..16+4g+3 in slots 4..7.  This K order is the row order of the accumulator
// tiles of a 16-token M-block, so the squared score tiles of the intra part feed
// the next MFMA without data movement.
//
// V arrives token-major (a row per lane); the transpose into column-per-lane
// fragments is done on the matrix cores: C = V_rows x E with E a 0/1 column selector
// (exact in bf16 -> fp32), whose accumulator tile holds V[4g+r][16nb+n] in lane (n, g),
// i.e. 4 slots of the fragment, written with one 8-byte LDS store per lane.

// selector B-fragment picking columns 16*h + n of a 32-column K-block
__device__ __forceinline__ bf16x8 column_selector(int h, int lane) {
  const int n = lane & 15, g = lane >> 4;
  bf16x8 e;
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = (bf16)((8 * g + i == 16 * h + n) ? 1.f : 0.f);
  return e;
}

template <class S, typename TIn>
__device__ __forceinline__ void stage_v(const Vec8<TIn> (&vr)[S::KV], int mb, const bf16x8 (&sel)[2],
                                        bf16* vf_hi, bf16* vf_lo, int lane) {
  const int jj = mb >> 1, half = mb & 1;
  bf16x8 xh[S::KV], xl[S::KV];
#pragma unroll
  for (int kk = 0; kk < S::KV; ++kk) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = vr[kk][i];
      xh[kk][i] = (bf16)x;
      if constexpr (S::SPLIT) xl[kk][i] = (bf16)(x - (float)xh[kk][i]);
    }
  }
#pragma unroll
  for (int nb = 0; nb < S::NB; ++nb) {
    const int kk = S::DV >= 32 ? nb >> 1 : 0;
    const int h = S::DV >= 32 ? nb & 1 : 0;
    const int idx = ((jj * S::NB + nb) * WAVE + lane) * 8 + half * 4;
    const f32x4 ch = mfma32(xh[kk], sel[h], zero4());
    bf16x4 bh;
#pragma unroll
    for (int r = 0; r < 4; ++r) bh[r] = (bf16)ch[r];
    *reinterpret_cast<bf16x4*>(vf_hi + idx) = bh;
    if constexpr (S::SPLIT) {
      const f32x4 cl = mfma32(xl[kk], sel[h], zero4());
      bf16x4 bl;
#pragma unroll
      for (int r = 0; r < 4; ++r) bl[r] = (bf16)cl[r];
      *reinterpret_cast<bf16x4*>(vf_lo + idx) = bl;
    }
  }
}

template <class S>
__device__ __forceinline__ Op8<S::SPLIT> load_vf(const bf16* vf_hi, const bf16* vf_lo, int jj, int nb, int lane) {
  Op8<S::SPLIT> o;
  const int idx = ((jj * S::NB + nb) * WAVE + lane) * 8;
  o.hi = *reinterpret_cast<const bf16x8*>(vf_hi + idx);
  if constexpr (S::SPLIT) o.lo = *reinterpret_cast<const bf16x8*>(vf_lo + idx);
  return o;
}

// P as projection B-fragments (K = input column, N = projection index a = lane%16),
// always split hi/lo since P is float32.
template <class S>
struct ProjP { Op8<true> f[S::KD]; };

// The P fragments are loop-invariant and live in LDS rather than in registers:
// Pf[kk][hi/lo][lane], 16 bytes each, written by one wave before the first chunk.
// In two halves, so a kernel can issue the reads of P, then its first input loads, and
// only then wait for P (the two latencies overlap): read_P_rows takes this lane's entries
// of P into registers, store_P writes them as fragments.
template <class S>
struct PRows { float x[S::KD][8]; };

template <class S>
__device__ __forceinline__ void read_P_rows(PRows<S>& r, const float* __restrict__ P, int h, int lane) {
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int kk = 0; kk < S::KD; ++kk) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      r.x[kk][i] = proj_valid<S>(g) ? P[((int64_t)h * P_DIM + n) * S::DIN + proj_col<S>(g, kk, i)] : 0.f;
  }
}

template <class S>
__device__ __forceinline__ void store_P(bf16* Pf, const PRows<S>& r, int lane) {
#pragma unroll
  for (int kk = 0; kk < S::KD; ++kk) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = r.x[kk][i];
    const Op8<true> f = make8<true>(x);
    *reinterpret_cast<bf16x8*>(Pf + ((2 * kk) * WAVE + lane) * 8) = f.hi;
    *reinterpret_cast<bf16x8*>(Pf + ((2 * kk + 1) * WAVE + lane) * 8) = f.lo;
  }
}

template <class S>
__device__ __forceinline__ void write_P(bf16* Pf, const float* __restrict__ P, int h, int lane) {
  PRows<S> r;
  read_P_rows<S>(r, P, h, lane);
  store_P<S>(Pf, r, lane);
}

template <class S>
__device__ __forceinline__ void read_P(ProjP<S>& pp, const bf16* Pf, int lane) {
#pragma unroll
  for (int kk = 0; kk < S::KD; ++kk) {
    pp.f[kk].hi = *reinterpret_cast<const bf16x8*>(Pf + ((2 * kk) * WAVE + lane) * 8);
    pp.f[kk].lo = *reinterpret_cast<const bf16x8*>(Pf + ((2 * kk + 1) * WAVE + lane) * 8);
  }
}

// u (or w) rows of M-block m of this wave: returns the accumulator tile whose lane
// (a = lane%16, g) holds row 4g + r, column a.
template <class S, typename TIn>
__device__ __forceinline__ f32x4 project_tile(const Vec8<TIn> (&x)[S::KD], const ProjP<S>& pp) {
  f32x4 acc = zero4();
#pragma unroll
  for (int kk = 0; kk < S::KD; ++kk) {
    if constexpr (S::SPLIT) {
      float xf[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) xf[i] = x[kk][i];
      acc = mma<true, true>(make8<true>(xf), pp.f[kk], acc);
    } else {
      Op8<false> a;
      if constexpr (sizeof(TIn) == 2) {
        a.hi = x[kk].x;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) a.hi[i] = (bf16)x[kk][i];
      }
      acc = mma<false, true>(a, pp.f[kk], acc);
    }
  }
  return acc;
}

// Row rotation inside each 16-lane row: lane a receives the value of lane
// (a + DELTA) mod 16.  DPP row_ror:R moves lane i's value to lane (i + R) mod 16, so
// the rotation is row_ror:(16 - DELTA).
template <int DELTA>
__device__ __forceinline__ float row_plus(float x) {
  if constexpr (DELTA % 16 == 0) {
    return x;
  } else {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + (16 - DELTA % 16), 0xf, 0xf,
                                                      false));
  }
}

// Packed phi(K)^T A-fragment: lane (a = lane%16, g) slot i holds w_s[a] * w_s[b]
// for the token s of slot i, with b = (a + delta) % 16.  wa0/wa1 are the key
// projection tiles of the two 16-token M-blocks of the K-block in accumulator layout
// (lane (a, g) holds w_{4g+r}[a]); wb0/wb1 the same tiles with the lanes rotated so
// lane a holds w[(a + d0) % 16]; ROT (a compile-time DPP row rotation) adds the rest
// of delta = d0 + ROT.  The slots (8, a >= 8) repeat the pairs of a < 8; they are
// accumulated like the others but carry query weight 0 and are never exported.
template <class S, int ROT>
__device__ __forceinline__ Op8<S::FSPLIT> key_frag(const f32x4& wa0, const f32x4& wa1, const f32x4& wb0,
                                                   const f32x4& wb1) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = wa0[i] * row_plus<ROT>(wb0[i]);
    x[4 + i] = wa1[i] * row_plus<ROT>(wb1[i]);
  }
  return make8<S::FSPLIT>(x);
}

// Feature-split ownership of the packed state accumulators.
template <class S>
struct StateAcc {
  static constexpr int N8 = (S::NB + 3) / 4;   // delta = 8 column blocks per wave (max)
  f32x4 s[2][S::NB];     // delta = wave, wave + 4
  f32x4 s8[N8];          // delta = 8, nb = wave + 4*i
  f32x4 Z;               // normaliser matrix, Z-owning wave only: lane (b, g) holds Z[4g+r][b]
};

template <class S>
__device__ __forceinline__ void state_zero(StateAcc<S>& st) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int nb = 0; nb < S::NB; ++nb) st.s[j][nb] = zero4();
  }
#pragma unroll
  for (int i = 0; i < StateAcc<S>::N8; ++i) st.s8[i] = zero4();
  st.Z = zero4();
}

// H += phi(K_c)^T V_c for the tiles this wave owns; wave 0 also Z += W_c^T W_c.
// Wave w owns the diagonals w and w + 4 (and delta = 8 for some column blocks): it
// reads its key tiles once plainly and once with the lanes rotated by w (a permuted,
// conflict-free LDS read), after which every diagonal it needs is a fixed DPP
// rotation (0, 4 or 8) away.  The z part of the chunk state, sum_s phi(k_s), is
// vec(Z): the W fragment of a K-block is at the same time the A operand W^T (lane =
// feature row a) and the B operand W (lane = column b), so one MFMA per K-block
// updates all 256 entries; the fragment arrives already split into hi/lo bf16 (Wz).
template <class S>
__device__ __forceinline__ void state_update(StateAcc<S>& st, const float* Wacc, const bf16* Wz,
                                             const bf16* vf_hi, const bf16* vf_lo, int wave, bool zrole,
                                             int lane) {
  const int rot_lane = (lane & ~15) | ((lane + wave) & 15);
#pragma unroll
  for (int jj = 0; jj < S::NJ; ++jj) {
    const f32x4 wa0 = *reinterpret_cast<const f32x4*>(Wacc + ((2 * jj) * WAVE + lane) * 4);
    const f32x4 wa1 = *reinterpret_cast<const f32x4*>(Wacc + ((2 * jj + 1) * WAVE + lane) * 4);
    const f32x4 wr0 = *reinterpret_cast<const f32x4*>(Wacc + ((2 * jj) * WAVE + rot_lane) * 4);
    const f32x4 wr1 = *reinterpret_cast<const f32x4*>(Wacc + ((2 * jj + 1) * WAVE + rot_lane) * 4);
    Op8<S::SPLIT> vfr[S::NB];
#pragma unroll
    for (int nb = 0; nb < S::NB; ++nb) vfr[nb] = load_vf<S>(vf_hi, vf_lo, jj, nb, lane);
    {
      const Op8<S::FSPLIT> kf = key_frag<S, 0>(wa0, wa1, wr0, wr1);     // delta = w
#pragma unroll
      for (int nb = 0; nb < S::NB; ++nb) st.s[0][nb] = mma<S::FSPLIT, S::SPLIT>(kf, vfr[nb], st.s[0][nb]);
    }
    {
      const Op8<S::FSPLIT> kf = key_frag<S, 4>(wa0, wa1, wr0, wr1);     // delta = w + 4
#pragma unroll
      for (int nb = 0; nb < S::NB; ++nb) st.s[1][nb] = mma<S::FSPLIT, S::SPLIT>(kf, vfr[nb], st.s[1][nb]);
    }
    if (wave < S::NB) {
      const Op8<S::FSPLIT> kf = key_frag<S, 8>(wa0, wa1, wa0, wa1);      // delta = 8
#pragma unroll
      for (int i = 0; i < StateAcc<S>::N8; ++i) {
#pragma unroll
        for (int nb = 0; nb < S::NB; ++nb)   // static register index: nb == wave + 4i
          if (nb == wave + 4 * i) st.s8[i] = mma<S::FSPLIT, S::SPLIT>(kf, vfr[nb], st.s8[i]);
      }
    }
    if (zrole) {   // hi/lo: Z feeds the denominator
      Op8<true> wf;
      wf.hi = *reinterpret_cast<const bf16x8*>(Wz + (jj * WAVE + lane) * 8);
      wf.lo = *reinterpret_cast<const bf16x8*>(Wz + ((S::NJ + jj) * WAVE + lane) * 8);
      st.Z = mma<true, true>(wf, wf, st.Z);
    }
  }
}

// ---- decay gates ------------------------------------------------------------------
// Decay-gated state (the abstract's "decay gates", read as a scalar forget gate per token
// and head): S_t = gamma_t S_{t-1} + phi(k_t) [v_t | 1]^T with gamma_t = exp(lam_t).  Inside
// a chunk with cumulative log-decay l_t (from the chunk start) and total L_c:
//   chunk state  = sum_s exp(L_c - l_s) phi(k_s) [v_s | 1]^T     (keys weighted)
//   prefix       : H <- exp(L_c) H + chunk state                 (affine scan)
//   readout of t : exp(l_t) phi(q_t)^T H,  tile weights (u_t . w_s)^2 exp(l_t - l_s).

// Chunk-local inclusive prefix of the log-decays: lane l of the wave gets l_l, the sum
// of lam over tokens t0 .. t0 + l (x = lam of token t0 + l, 0 past the sequence); Lc is
// the chunk total.  Every wave computes it (one 256-byte load per chunk and wave).
__device__ __forceinline__ float chunk_cumlog(float x, int lane, float& Lc) {
#pragma unroll
  for (int off = 1; off < WAVE; off <<= 1) {
    const float y = __shfl_up(x, off, WAVE);
    if (lane >= off) x += y;
  }
  Lc = __shfl(x, WAVE - 1, WAVE);
  return x;
}

// The state update of a decay-gated chunk: as state_update, with the key features of
// token s weighted by es[s] (the factor its contribution keeps at the end of the chunk,
// or of the leaf) and the z-matrix updated by W^T diag(es) W.
template <class S>
__device__ __forceinline__ void state_update_decay(StateAcc<S>& st, const float* Wacc, const float* es,
                                                   const bf16* vf_hi, const bf16* vf_lo, int wave, bool zrole,
                                                   int lane) {
  const int g = lane >> 4;
  const int rot_lane = (lane & ~15) | ((lane + wave) & 15);
#pragma unroll
  for (int jj = 0; jj < S::NJ; ++jj) {
    const f32x4 wa0 = *reinterpret_cast<const f32x4*>(Wacc + ((2 * jj) * WAVE + lane) * 4);
    const f32x4 wa1 = *reinterpret_cast<const f32x4*>(Wacc + ((2 * jj + 1) * WAVE + lane) * 4);
    const f32x4 wr0 = *reinterpret_cast<const f32x4*>(Wacc + ((2 * jj) * WAVE + rot_lane) * 4);
    const f32x4 wr1 = *reinterpret_cast<const f32x4*>(Wacc + ((2 * jj + 1) * WAVE + rot_lane) * 4);
    const f32x4 e0 = *reinterpret_cast<const f32x4*>(es + 32 * jj + 4 * g);
    const f32x4 e1 = *reinterpret_cast<const f32x4*>(es + 32 * jj + 16 + 4 * g);
    // the weight goes on the plain operand: key feature (a, a + delta) of token s times es[s]
    f32x4 we0, we1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      we0[i] = wa0[i] * e0[i];
      we1[i] = wa1[i] * e1[i];
    }
    Op8<S::SPLIT> vfr[S::NB];
#pragma unroll
    for (int nb = 0; nb < S::NB; ++nb) vfr[nb] = load_vf<S>(vf_hi, vf_lo, jj, nb, lane);
    {
      const Op8<S::FSPLIT> kf = key_frag<S, 0>(we0, we1, wr0, wr1);     // delta = w
#pragma unroll
      for (int nb = 0; nb < S::NB; ++nb) st.s[0][nb] = mma<S::FSPLIT, S::SPLIT>(kf, vfr[nb], st.s[0][nb]);
    }
    {
      const Op8<S::FSPLIT> kf = key_frag<S, 4>(we0, we1, wr0, wr1);     // delta = w + 4
#pragma unroll
      for (int nb = 0; nb < S::NB; ++nb) st.s[1][nb] = mma<S::FSPLIT, S::SPLIT>(kf, vfr[nb], st.s[1][nb]);
    }
    if (wave < S::NB) {
      const Op8<S::FSPLIT> kf = key_frag<S, 8>(we0, we1, wa0, wa1);      // delta = 8
#pragma unroll
      for (int i = 0; i < StateAcc<S>::N8; ++i) {
#pragma unroll
        for (int nb = 0; nb < S::NB; ++nb)
          if (nb == wave + 4 * i) st.s8[i] = mma<S::FSPLIT, S::SPLIT>(kf, vfr[nb], st.s8[i]);
      }
    }
    if (zrole) {
      float ua[8], ue[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ua[r] = wa0[r];
        ua[4 + r] = wa1[r];
        ue[r] = we0[r];
        ue[4 + r] = we1[r];
      }
      st.Z = mma<true, true>(make8<true>(ua), make8<true>(ue), st.Z);
    }
  }
}

template <class S>
__device__ __forceinline__ void state_scale(StateAcc<S>& st, float f) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int nb = 0; nb < S::NB; ++nb) st.s[j][nb] *= f;
  }
#pragma unroll
  for (int i = 0; i < StateAcc<S>::N8; ++i) st.s8[i] *= f;
  st.Z *= f;
}

// Stage one chunk: project keys (token split) into W tiles in LDS (accumulator
// layout, one 16-byte slot per lane), queries into U rows and keys into W rows when
// WANT_Q, and transpose the wave's V rows into B-fragments.
template <class S, typename TIn, bool WANT_Q>
__device__ __forceinline__ void stage_chunk(const ChunkIn<S, TIn>& r, const bf16* Pf, const bf16x8 (&sel)[2],
                                            float* Us, float* Ws, float* Wacc, bf16* Wz, bf16* vf_hi,
                                            bf16* vf_lo, int tw, int lane) {
  const int n = lane & 15, g = lane >> 4;
  ProjP<S> pp;
  read_P<S>(pp, Pf, lane);
#pragma unroll
  for (int m = 0; m < S::MBW; ++m) {
    const int mb = tw + 4 * m;
    if (mb < S::NMB) {
      const f32x4 w = project_tile<S, TIn>(r.k[m], pp);
      *reinterpret_cast<f32x4*>(Wacc + (mb * WAVE + lane) * 4) = w;
      {   // hi/lo halves of the Z-update fragment of K-block mb/2 (slots 4*(mb&1) ..)
        float wv[4] = {w[0], w[1], w[2], w[3]};
        const Op4<true> wz = make4<true>(wv);
        const int idx = ((mb >> 1) * WAVE + lane) * 8 + (mb & 1) * 4;
        *reinterpret_cast<bf16x4*>(Wz + idx) = wz.hi;
        *reinterpret_cast<bf16x4*>(Wz + S::NJ * WAVE * 8 + idx) = wz.lo;
      }
      if constexpr (WANT_Q) {
#pragma unroll
        for (int i = 0; i < 4; ++i) Ws[(mb * 16 + 4 * g + i) * S::USTR + n] = w[i];
        const f32x4 u = project_tile<S, TIn>(r.q[m], pp);
#pragma unroll
        for (int i = 0; i < 4; ++i) Us[(mb * 16 + 4 * g + i) * S::USTR + n] = u[i];
      }
      stage_v<S, TIn>(r.v[m], mb, sel, vf_hi, vf_lo, lane);
    }
  }
}

// ---- kata_chunk_state ----------------------------------------------------------
// grid (n_leaf, B*H), block 256.  Writes the leaf's summed packed state to ws.  DECAY:
// lam [B*H, T] log-decays; each token's contribution is weighted by the decay from it to
// the leaf's end, and the leaf's total decay exp(sum lam) goes to dec[bh * n_leaf + leaf].
// G > 1 (KATA-Mg, several concatenated PSD factors): grid (n_leaf, B*H*G), P [H, G, p, d];
// the workgroup of virtual head vh = bh*G + i builds factor i's state of sequence bh into
// ws row vh (the state of each factor is that of one-factor KATA with P_i).
// G > 1 with SUMG (KATA-Sigma-g, summed PSD factors): grid (n_leaf, B*H); the workgroup adds
// the key features of all G factors into the same accumulators (their state is the sum of
// the factor states), so k and v are read once; the extra factors' key tiles and P
// fragments sit after the one-factor LDS (SgStateLayout).
template <class S, int G>
struct SgStateLayout {
  static constexpr int XB = S::WACC_BYTES + S::WZ_BYTES + S::PF_BYTES;   // per extra factor
  static constexpr int SMEM = S::SMEM_STATE + (G - 1) * XB;
  static __device__ __forceinline__ int off(int i) { return S::SMEM_STATE + (i - 1) * XB; }
};

// The key projections of one more factor (stage_chunk's key part, without V).
template <class S, typename TIn>
__device__ __forceinline__ void stage_keys(const ChunkIn<S, TIn>& r, const bf16* Pf, float* Wacc, bf16* Wz, int tw,
                                           int lane) {
  ProjP<S> pp;
  read_P<S>(pp, Pf, lane);
#pragma unroll
  for (int m = 0; m < S::MBW; ++m) {
    const int mb = tw + 4 * m;
    if (mb < S::NMB) {
      const f32x4 w = project_tile<S, TIn>(r.k[m], pp);
      *reinterpret_cast<f32x4*>(Wacc + (mb * WAVE + lane) * 4) = w;
      float wv[4] = {w[0], w[1], w[2], w[3]};
      const Op4<true> wz = make4<true>(wv);
      const int idx = ((mb >> 1) * WAVE + lane) * 8 + (mb & 1) * 4;
      *reinterpret_cast<bf16x4*>(Wz + idx) = wz.hi;
      *reinterpret_cast<bf16x4*>(Wz + S::NJ * WAVE * 8 + idx) = wz.lo;
    }
  }
}

template <class S, typename TIn, bool DECAY = false, int G = 1, bool SUMG = false>
__global__ void __launch_bounds__(256, S::OCC_STATE)
kata_chunk_state(const TIn* __restrict__ k, const TIn* __restrict__ v, const float* __restrict__ P,
                 float* __restrict__ ws, int64_t T, int H, int64_t part_tokens,
                 const float* __restrict__ lam, float* __restrict__ dec) {
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* vf_hi = reinterpret_cast<bf16*>(smem + S::OFF_VF);
  bf16* vf_lo = reinterpret_cast<bf16*>(smem + S::OFF_VF + S::VF_BYTES);
  float* Wacc = reinterpret_cast<float*>(smem + S::ST_OFF_WACC);
  bf16* Wz = reinterpret_cast<bf16*>(smem + S::ST_OFF_WZ);
  bf16* Pf = reinterpret_cast<bf16*>(smem + S::ST_OFF_PF);
  float* es = reinterpret_cast<float*>(smem + S::SMEM_STATE);   // DECAY: key weights
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  static_assert(!(DECAY && G > 1), "decay gates with one PSD factor only");
  constexpr int VG = SUMG ? 1 : G;        // workspace rows per sequence
  const int64_t bh = blockIdx.y / VG;    // sequence; blockIdx.y is the workspace row
  const int h = (int)(bh % H);
  const int64_t part = blockIdx.x;
  // the part's tokens [tb, tb + len) of the sequence; loads past them read zeros
  const int64_t tb = min<int64_t>(part * part_tokens, T);
  const int len = (int)(min<int64_t>(tb + part_tokens, T) - tb);
  const int nch = (len + S::C - 1) / S::C;
  const int64_t base_tok = bh * T + tb;
  __amdgpu_buffer_rsrc_t rl;
  if constexpr (DECAY) rl = make_rsrc(lam + base_tok, (int64_t)len * 4);
  float fdec = 1.f;   // DECAY: decay from the end of the current chunk to the part's end

  // P is read before the first chunk's loads and written to LDS after them (see store_P)
  PRows<S> prow;
  read_P_rows<S>(prow, P, G == 1 ? h : (SUMG ? h * G : h * G + (int)(blockIdx.y % G)), lane);
  if constexpr (SUMG) {
    if (wave == 0) {
#pragma unroll
      for (int i = 1; i < G; ++i)
        write_P<S>(reinterpret_cast<bf16*>(smem + SgStateLayout<S, G>::off(i) + S::WACC_BYTES + S::WZ_BYTES), P,
                   h * G + i, lane);
    }
  }
  const bf16x8 sel[2] = {column_selector(0, lane), column_selector(1, lane)};
  StateAcc<S> st;
  state_zero<S>(st);
  SeqRsrc rs;
  rs.k = make_rsrc(k + base_tok * S::DIN, (int64_t)len * S::DIN * (int64_t)sizeof(TIn));
  rs.v = make_rsrc(v + base_tok * S::DV, (int64_t)len * S::DV * (int64_t)sizeof(TIn));
  // Inputs are prefetched DEPTH chunks ahead in DEPTH register buffers: the loads of
  // chunk c+DEPTH are in flight while chunk c is processed.  Loads past the leaf
  // read zeros or unused rows.  (Two buffers measured no faster: the kernel is not
  // limited by the prefetch distance, and the extra registers cost occupancy.)
  constexpr int DEPTH = 1;
  // Chunks are summed last to first: the sum does not depend on the order, and the
  // data read last (the part's first chunks) is what kata_chunk_intra reads first,
  // so some of it is still in the last-level cache.  The prefetch past the part's
  // last chunk reads at len, outside the buffer (zeros, no memory traffic).
  auto chunk_t0 = [&](int c) { return (nch - 1 - c) * S::C; };
  ChunkIn<S, TIn> buf[DEPTH];
#pragma unroll
  for (int i = 0; i < DEPTH; ++i) load_chunk<S, TIn, false>(buf[i], rs, chunk_t0(i), wave, lane);
  float lam_next = 0.f;
  if constexpr (DECAY) lam_next = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, (chunk_t0(0) + lane) * 4, 0, 0));
  if (wave == 0) store_P<S>(Pf, prow, lane);
  __syncthreads();   // P fragments written
  auto step = [&](ChunkIn<S, TIn>& cur, int c) {
    stage_chunk<S, TIn, false>(cur, Pf, sel, nullptr, nullptr, Wacc, Wz, vf_hi, vf_lo, wave, lane);
    if constexpr (SUMG) {
#pragma unroll
      for (int i = 1; i < G; ++i) {
        unsigned char* xb = smem + SgStateLayout<S, G>::off(i);
        stage_keys<S, TIn>(cur, reinterpret_cast<const bf16*>(xb + S::WACC_BYTES + S::WZ_BYTES),
                           reinterpret_cast<float*>(xb), reinterpret_cast<bf16*>(xb + S::WACC_BYTES), wave, lane);
      }
    }
    load_chunk<S, TIn, false>(cur, rs, c + DEPTH < nch ? chunk_t0(c + DEPTH) : len, wave, lane);
    if constexpr (DECAY) {
      float Lc;
      const float l = chunk_cumlog(lam_next, lane, Lc);
      if (wave == 0) es[lane] = fdec * __expf(Lc - l);
      fdec *= __expf(Lc);
      lam_next = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          rl, ((c + 1 < nch ? chunk_t0(c + 1) : len) + lane) * 4, 0, 0));
    }
    __syncthreads();
    if constexpr (DECAY) state_update_decay<S>(st, Wacc, es, vf_hi, vf_lo, wave, wave == 0, lane);
    else state_update<S>(st, Wacc, Wz, vf_hi, vf_lo, wave, wave == 0, lane);
    if constexpr (SUMG) {
#pragma unroll
      for (int i = 1; i < G; ++i) {
        unsigned char* xb = smem + SgStateLayout<S, G>::off(i);
        state_update<S>(st, reinterpret_cast<const float*>(xb), reinterpret_cast<const bf16*>(xb + S::WACC_BYTES),
                        vf_hi, vf_lo, wave, wave == 0, lane);
      }
    }
    __syncthreads();
  };
  int c = 0;
  for (; c + DEPTH <= nch; c += DEPTH) {
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) step(buf[i], c + i);
  }
#pragma unroll
  for (int i = 0; i + 1 < DEPTH; ++i)   // fewer than DEPTH chunks left: static buffer index
    if (c + i < nch) step(buf[i], c + i);
  // write the part's state (tile-native layout) and Z
  float* out = ws + ((int64_t)blockIdx.y * gridDim.x + part) * S::E;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int delta = wave + 4 * j;
#pragma unroll
    for (int nb = 0; nb < S::NB; ++nb)
      *reinterpret_cast<f32x4*>(out + ws_tile_offset<S>(delta, nb, lane)) = st.s[j][nb];
  }
#pragma unroll
  for (int i = 0; i < StateAcc<S>::N8; ++i) {
    const int nb = wave + 4 * i;
    if (nb < S::NB) *reinterpret_cast<f32x4*>(out + ws_tile_offset<S>(8, nb, lane)) = st.s8[i];
  }
  if (wave == 0) *reinterpret_cast<f32x4*>(out + DPACK * S::DV + lane * 4) = st.Z;
  if constexpr (DECAY) {
    if (tid == 0) dec[(int64_t)blockIdx.y * gridDim.x + part] = fdec;
  }
}

// ---- kata_chunk_intra ------------------------------------------------------------

// Issue priority from the progress through the leaf.  The workgroups that share a CU
// start together, and at equal priority the oldest wave issues first, so the first
// workgroup dispatched to a CU runs ahead and the last one finishes alone, at a
// fraction of the CU's throughput.  Lowering a wave's priority as it passes 50%, 75%
// and 90% of its leaf lets the ones behind catch up at each step.
__device__ __forceinline__ void progress_priority(int c, int nch) {
  const int pm = (1000 * c) / nch;
  if (pm < 500) __builtin_amdgcn_s_setprio(3);
  else if (pm < 750) __builtin_amdgcn_s_setprio(2);
  else if (pm < 900) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Publish the state accumulators as bf16 readout fragments: Hx[kb][nb][lane][slot],
// delta = 2*kb + slot/4 (delta 8 -> kb 4, slots 0..3).  The Z owner publishes Z split into
// hi/lo bf16: Z is symmetric, so its accumulator tile (lane (b, g) holds Z[4g+r][b])
// is also its 16x16x16 A-fragment (lane (m, g) holds Z[m][4g+i]); Zs[lane] = {hi, lo}.
template <class S>
__device__ __forceinline__ void publish_state(const StateAcc<S>& st, bf16* hx_hi, bf16* hx_lo, bf16* Zs,
                                              int wave, bool zrole, int lane) {
  auto put = [&](int delta, int nb, const f32x4& a) {
    const int idx = (((delta >> 1) * S::NB + nb) * WAVE + lane) * 8 + (delta & 1) * 4;
    bf16x4 hi, lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hi[i] = (bf16)a[i];
      if constexpr (S::FSPLIT) lo[i] = (bf16)(a[i] - (float)hi[i]);
    }
    *reinterpret_cast<bf16x4*>(hx_hi + idx) = hi;
    if constexpr (S::FSPLIT) *reinterpret_cast<bf16x4*>(hx_lo + idx) = lo;
  };
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int delta = wave + 4 * j;
#pragma unroll
    for (int nb = 0; nb < S::NB; ++nb) put(delta, nb, st.s[j][nb]);
  }
#pragma unroll
  for (int i = 0; i < StateAcc<S>::N8; ++i) {
    const int nb = wave + 4 * i;
    if (nb < S::NB) put(8, nb, st.s8[i]);
  }
  if (zrole) {
    float zv[4] = {st.Z[0], st.Z[1], st.Z[2], st.Z[3]};
    const Op4<true> z = make4<true>(zv);
    bf16x8 zz;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      zz[i] = z.hi[i];
      zz[4 + i] = z.lo[i];
    }
    *reinterpret_cast<bf16x8*>(Zs + lane * 8) = zz;
  }
}

template <class S>
__device__ __forceinline__ void load_state(StateAcc<S>& st, const float* in, int wave, bool zrole, int lane) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int delta = wave + 4 * j;
#pragma unroll
    for (int nb = 0; nb < S::NB; ++nb)
      st.s[j][nb] = *reinterpret_cast<const f32x4*>(in + ws_tile_offset<S>(delta, nb, lane));
  }
#pragma unroll
  for (int i = 0; i < StateAcc<S>::N8; ++i) {
    const int nb = wave + 4 * i;
    st.s8[i] = (nb < S::NB) ? *reinterpret_cast<const f32x4*>(in + ws_tile_offset<S>(8, nb, lane)) : zero4();
  }
  st.Z = zrole ? *reinterpret_cast<const f32x4*>(in + DPACK * S::DV + lane * 4) : zero4();
}

// y is written once and not read again by the pass, so its stores are non-temporal
// (cache policy NT): the lines go out to memory instead of staying dirty in the caches,
// where the next pass (the state pass of the next batch, in a stream of forwards) would
// have to write them back while it streams its own reads.  Measured on the long shape,
// the state pass that follows takes 102 us instead of 125 us; the intra pass itself
// takes about 4 us longer.
constexpr int Y_STORE_POLICY = 2;   // NT

// Element index e (in the leaf block of the workspace) of accumulator element r of the
// tile (delta, nb) that this lane holds.
template <class S>
__device__ __forceinline__ int acc_elem(int delta, int nb, int lane, int r) {
  return ws_tile_offset<S>(delta, nb, lane) + r;
}

// Sets every accumulator element this wave holds (its diagonals, its delta = 8 column
// blocks, and Z for the Z owner) to fn(e, value), e its element index.
template <class S, typename F>
__device__ __forceinline__ void for_state_elems(StateAcc<S>& st, int wave, bool zrole, int lane, F&& fn) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int nb = 0; nb < S::NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) st.s[j][nb][r] = fn(acc_elem<S>(wave + 4 * j, nb, lane, r), st.s[j][nb][r]);
  }
#pragma unroll
  for (int i = 0; i < StateAcc<S>::N8; ++i) {
    const int nb = wave + 4 * i;
    if (nb < S::NB) {
#pragma unroll
      for (int r = 0; r < 4; ++r) st.s8[i][r] = fn(acc_elem<S>(8, nb, lane, r), st.s8[i][r]);
    }
  }
  if (zrole) {
#pragma unroll
    for (int r = 0; r < 4; ++r) st.Z[r] = fn(DPACK * S::DV + lane * 4 + r, st.Z[r]);
  }
}

template <class S>
__device__ __forceinline__ void state_add(StateAcc<S>& st, const StateAcc<S>& t) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int nb = 0; nb < S::NB; ++nb) st.s[j][nb] += t.s[j][nb];
  }
#pragma unroll
  for (int i = 0; i < StateAcc<S>::N8; ++i) st.s8[i] += t.s8[i];
  st.Z += t.Z;
}

// Vector store of 4 consecutive outputs through the y buffer resource (stores past
// the end of the sequence are dropped).
template <typename TOut> struct Store4;
template <> struct Store4<float> {
  static __device__ __forceinline__ void st(__amdgpu_buffer_rsrc_t r, int off, const f32x4& x) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, x), r, off, 0, Y_STORE_POLICY);
  }
};
template <> struct Store4<bf16> {
  static __device__ __forceinline__ void st(__amdgpu_buffer_rsrc_t r, int off, const f32x4& x) {
    bf16x4 b;
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = (bf16)x[i];
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, b), r, off, 0, Y_STORE_POLICY);
  }
};

// Score-tile operand: four consecutive fp32 projection entries (u_t or w_s, from their
// LDS rows) as a hi/lo bf16 pair.  The score X = u.w feeds the weight X^2, and where X is
// a small fraction eps of |u| |w| (a query nearly orthogonal to its keys) single bf16
// operands give X^2 a relative error of about 2^-8 / eps, so a few such weights decide
// y_t.  With hi/lo operands (three MFMAs instead of one on a K = 16 tile) the error of X
// drops to about 2^-16 |u| |w|.  The denominator sums the fp32 squares; the value MFMA
// takes them as bf16, a relative rounding of each (non-negative) weight.
__device__ __forceinline__ Op4<true> score_operand(const float* row4) {
  const f32x4 x = *reinterpret_cast<const f32x4*>(row4);
  float xv[4] = {x[0], x[1], x[2], x[3]};
  return make4<true>(xv);
}

// The gated output row of token t: lane (t, g) holds O[nb][r] = column 16nb + 4g + r.
// bf16 rows of 64 columns (128 bytes, one cache line) go out in whole lines: for each
// pair of column blocks (nb, nb + 1) one v_permlane16_swap per element between the lanes
// g and g ^ 1 (the two 16-lane rows of each 32-lane half) leaves the even lane columns
// 4g .. 4g + 7 of block nb and the odd lane columns 16 + 4(g - 1) .. 16 + 4g + 3 of
// block nb + 1, i.e. eight consecutive columns per lane; a DPP exchange between the
// lanes t and t ^ 8 of each 16-lane row then gives each of the two 16-byte stores eight
// whole token rows (tokens 0..7 of the M-block, then 8..15).  Stores of half lines take
// about 4% longer for the whole intra pass with the NT policy.  Other shapes store the
// four columns of each block directly.
template <typename T> struct IsBf16 { static constexpr bool value = false; };
template <> struct IsBf16<bf16> { static constexpr bool value = true; };

template <class S, typename TOut>
__device__ __forceinline__ void store_row(const f32x4 (&O)[S::NB], float inv, __amdgpu_buffer_rsrc_t ry,
                                          int row0, int t, int g) {
  if constexpr (IsBf16<TOut>::value && S::NB == 4) {
    i32x4 half[2];   // columns 32p + 8(g >> 1) + 16(g & 1) .. + 7 of token t
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      bf16x8 out;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(O[2 * p][r] * inv),
                                                         __float_as_uint(O[2 * p + 1][r] * inv), false, false);
        out[r] = (bf16)__uint_as_float(sw[0]);
        out[4 + r] = (bf16)__uint_as_float(sw[1]);
      }
      half[p] = __builtin_bit_cast(i32x4, out);
    }
    // lane t < 8 keeps columns 0..31 of token t and takes columns 0..31 of token t + 8;
    // lane t >= 8 takes columns 32..63 of token t - 8 and keeps columns 32..63 of token t
    // (DPP row_ror:8 swaps the two 8-lane halves of each 16-lane row)
    const bool lo = (t & 15) < 8;
    i32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rcv = __builtin_amdgcn_update_dpp(0, lo ? half[1][i] : half[0][i], 0x128, 0xf, 0xf, false);
      a[i] = lo ? half[0][i] : rcv;
      b[i] = lo ? rcv : half[1][i];
    }
    const int col = (lo ? 0 : 32) + 8 * (g >> 1) + 16 * (g & 1);
    const int rowa = row0 - (lo ? 0 : 8 * S::DV);   // token t & ~8, then t | 8
    __builtin_amdgcn_raw_buffer_store_b128(a, ry, (rowa + col) * 2, 0, Y_STORE_POLICY);
    __builtin_amdgcn_raw_buffer_store_b128(b, ry, (rowa + 8 * S::DV + col) * 2, 0, Y_STORE_POLICY);
  } else {
#pragma unroll
    for (int nb = 0; nb < S::NB; ++nb) {
      f32x4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = O[nb][r] * inv;
      Store4<TOut>::st(ry, (row0 + nb * 16 + 4 * g) * (int)sizeof(TOut), o);
    }
  }
}

// Readout + intra tile + gate for one 16-token M-block mb of the chunk; writes y.
// Everything is computed transposed, O^T = H^T phi(Q)^T + V^T (A o A o M)^T, by
// feeding the same fragments to the MFMA in swapped operand order: lane (t, g) then
// holds output columns 16nb + 4g .. 16nb + 4g + 3 of token t, so the denominator of
// token t is lane-local and y leaves as 4-element vector stores.
template <class S, typename TOut, bool DECAY = false>
__device__ __forceinline__ void chunk_outputs(int mb, const float* Us, const float* Ws, const bf16* vf_hi,
                                              const bf16* vf_lo, const bf16* hx_hi, const bf16* hx_lo,
                                              const bf16* Zs, const SeqRsrc& rs, int t0, int lane,
                                              const float* ls = nullptr) {
  const int n = lane & 15, g = lane >> 4;
  const int t = mb * 16 + n;    // token (within chunk) whose fragment column this lane builds

  // rotated quads of u_t: Q[m] = u_t[4*((g+m)&3) .. +3]
  f32x4 Q[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) Q[m] = *reinterpret_cast<const f32x4*>(Us + t * S::USTR + 4 * ((g + m) & 3));
  auto u_rot = [&](int delta, int i) -> float {   // u_t[(4g + i + delta) & 15]
    const int m = delta >> 2, e = delta & 3;
    const int j = i + e;
    return j < 4 ? Q[m & 3][j] : Q[(m + 1) & 3][j - 4];
  };
  // query-side weights folded into u_a: 1 on the diagonal, 2 off it, and for the
  // diagonal delta = 8 only the 8 distinct slots a < 8 (lane groups g < 2) count
  f32x4 ua1 = Q[0], ua2, ua8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ua2[i] = 2.f * Q[0][i];
    ua8[i] = g < 2 ? ua2[i] : 0.f;
  }

  f32x4 O[S::NB];
#pragma unroll
  for (int nb = 0; nb < S::NB; ++nb) O[nb] = zero4();

  // inter-chunk readout: O^T += H^T phi(Q)^T
#pragma unroll
  for (int kb = 0; kb < READ_KB; ++kb) {
    float x[8];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int delta = 2 * kb + half;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (delta <= 8) {
          const f32x4& ua = delta == 0 ? ua1 : (delta == 8 ? ua8 : ua2);
          x[half * 4 + i] = ua[i] * u_rot(delta, i);
        } else {
          x[half * 4 + i] = 0.f;
        }
      }
    }
    const Op8<S::FSPLIT> qf = make8<S::FSPLIT>(x);
#pragma unroll
    for (int nb = 0; nb < S::NB; ++nb) {
      const int idx = ((kb * S::NB + nb) * WAVE + lane) * 8;
      Op8<S::FSPLIT> hf;
      hf.hi = *reinterpret_cast<const bf16x8*>(hx_hi + idx);
      if constexpr (S::FSPLIT) hf.lo = *reinterpret_cast<const bf16x8*>(hx_lo + idx);
      O[nb] = mma<S::FSPLIT, S::FSPLIT>(hf, qf, O[nb]);
    }
  }
  // phi(q_t) . z = u_t^T Z u_t: (Z U^T)[4g + r][t] from one 16x16x16 MFMA (Z symmetric,
  // so its accumulator tile is its own A fragment), dotted with u_t[4g..4g+3]
  float den;
  {
    const bf16x8 zz = *reinterpret_cast<const bf16x8*>(Zs + lane * 8);
    Op4<true> zf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      zf.hi[i] = zz[i];
      zf.lo[i] = zz[4 + i];
    }
    float uv[4] = {Q[0][0], Q[0][1], Q[0][2], Q[0][3]};
    const f32x4 zu = mma<true, true>(zf, make4<true>(uv), zero4());
    den = zu[0] * Q[0][0] + zu[1] * Q[0][1] + zu[2] * Q[0][2] + zu[3] * Q[0][3];
  }
  // DECAY: the prefix state reaches token t decayed by exp(l_t)
  float lt = 0.f;
  if constexpr (DECAY) {
    lt = ls[t];
    const float f = __expf(lt);
    den *= f;
#pragma unroll
    for (int nb = 0; nb < S::NB; ++nb) O[nb] *= f;
  }

  // intra-chunk: X_j = W_j U_mb^T (16x16, K = p), lane (t, g) holds X[s = 4g + r][t].
  // u and w enter as hi/lo bf16 pairs for every input dtype: a weight (u.w)^2 of a query
  // nearly orthogonal to a key is a small difference of large products, and single bf16
  // operands would leave it an error of about 2^-8 |u| |w| (see score_operand)
  const Op4<true> uf = score_operand(Us + t * S::USTR + 4 * g);
  f32x4 A2[S::NMB];
#pragma unroll
  for (int j = 0; j < S::NMB; ++j) {
    A2[j] = zero4();
    if (j <= mb) {
      const f32x4 X = mma<true, true>(score_operand(Ws + (j * 16 + n) * S::USTR + 4 * g), uf, zero4());
      if (j < mb) {   // wave-uniform: only the diagonal tile is masked
#pragma unroll
        for (int r = 0; r < 4; ++r) A2[j][r] = X[r] * X[r];
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) A2[j][r] = (4 * g + r <= n) ? X[r] * X[r] : 0.f;
      }
      if constexpr (DECAY) {   // weight exp(l_t - l_s) of key s = 16j + 4g + r
        const f32x4 lsv = *reinterpret_cast<const f32x4*>(ls + j * 16 + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) A2[j][r] *= __expf(fminf(lt - lsv[r], 0.f));
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) den += A2[j][r];
    }
  }
  // O^T += V^T (A^2 masked)^T: K-block jj = score tiles 2jj (slots 0..3), 2jj+1 (slots 4..7)
#pragma unroll
  for (int jj = 0; jj < S::NJ; ++jj) {
    if (2 * jj <= mb) {
      float x[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = A2[2 * jj][i];
        x[4 + i] = (2 * jj + 1 < S::NMB) ? A2[2 * jj + 1][i] : 0.f;
      }
      const Op8<S::SPLIT> af = make8<S::SPLIT>(x);
#pragma unroll
      for (int nb = 0; nb < S::NB; ++nb)
        O[nb] = mma<S::SPLIT, S::SPLIT>(load_vf<S>(vf_hi, vf_lo, jj, nb, lane), af, O[nb]);
    }
  }

  // den(t) = sum over the 4 lane groups of this token's partial sums: each permlane
  // swap exchanges rows between its two outputs, whose sum is the pair sum in every lane
  den = row_pair_sum<16>(den);
  den = row_pair_sum<32>(den);
  // output gate: y = O / den (0 where the denominator is 0); v_rcp_f32 is within 1 ulp
  const float inv = den != 0.f ? __builtin_amdgcn_rcpf(den) : 0.f;
  store_row<S, TOut>(O, inv, rs.y, (t0 + t) * S::DV, t, g);
}

// ---- the same three steps, separated -------------------------------------------------
// chunk_outputs above fuses, for one PSD factor, the prefix readout, the intra tile and the
// gate.  With several concatenated PSD factors (KATA-Mg) every factor adds its readout and
// its intra tile to one output tile and one denominator before the single division, so
// the steps are also available separately (same arithmetic, same fragment layouts).

// Inter-chunk readout of token t = 16 mb + lane % 16 through the published state:
// O^T += H^T phi(Q)^T, and den += phi(q_t) . z = u_t^T Z u_t (den = ... when FIRST).
template <class S, bool FIRST>
__device__ __forceinline__ void readout_acc(int t, const float* Us, const bf16* hx_hi, const bf16* hx_lo,
                                            const bf16* Zs, int lane, f32x4 (&O)[S::NB], float& den) {
  const int g = lane >> 4;
  // rotated quads of u_t: Q[m] = u_t[4*((g+m)&3) .. +3]
  f32x4 Q[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) Q[m] = *reinterpret_cast<const f32x4*>(Us + t * S::USTR + 4 * ((g + m) & 3));
  auto u_rot = [&](int delta, int i) -> float {   // u_t[(4g + i + delta) & 15]
    const int m = delta >> 2, e = delta & 3;
    const int j = i + e;
    return j < 4 ? Q[m & 3][j] : Q[(m + 1) & 3][j - 4];
  };
  // query-side weights folded into u_a: 1 on the diagonal, 2 off it, and for the
  // diagonal delta = 8 only the 8 distinct slots a < 8 (lane groups g < 2) count
  f32x4 ua1 = Q[0], ua2, ua8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ua2[i] = 2.f * Q[0][i];
    ua8[i] = g < 2 ? ua2[i] : 0.f;
  }
#pragma unroll
  for (int kb = 0; kb < READ_KB; ++kb) {
    float x[8];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int delta = 2 * kb + half;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (delta <= 8) {
          const f32x4& ua = delta == 0 ? ua1 : (delta == 8 ? ua8 : ua2);
          x[half * 4 + i] = ua[i] * u_rot(delta, i);
        } else {
          x[half * 4 + i] = 0.f;
        }
      }
    }
    const Op8<S::FSPLIT> qf = make8<S::FSPLIT>(x);
#pragma unroll
    for (int nb = 0; nb < S::NB; ++nb) {
      const int idx = ((kb * S::NB + nb) * WAVE + lane) * 8;
      Op8<S::FSPLIT> hf;
      hf.hi = *reinterpret_cast<const bf16x8*>(hx_hi + idx);
      if constexpr (S::FSPLIT) hf.lo = *reinterpret_cast<const bf16x8*>(hx_lo + idx);
      O[nb] = mma<S::FSPLIT, S::FSPLIT>(hf, qf, O[nb]);
    }
  }
  // (Z U^T)[4g + r][t] from one 16x16x16 MFMA (Z symmetric, so its accumulator tile is
  // its own A fragment), dotted with u_t[4g..4g+3]
  const bf16x8 zz = *reinterpret_cast<const bf16x8*>(Zs + lane * 8);
  Op4<true> zf;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    zf.hi[i] = zz[i];
    zf.lo[i] = zz[4 + i];
  }
  float uv[4] = {Q[0][0], Q[0][1], Q[0][2], Q[0][3]};
  const f32x4 zu = mma<true, true>(zf, make4<true>(uv), zero4());
  const float zd = zu[0] * Q[0][0] + zu[1] * Q[0][1] + zu[2] * Q[0][2] + zu[3] * Q[0][3];
  if constexpr (FIRST) den = zd;
  else den += zd;
}

// Intra-chunk part of M-block mb: X_j = W_j U_mb^T (16x16, K = p), lane (t, g) holds
// X[s = 4g + r][t]; the masked squares (times exp(l_t - l_s) under DECAY) add to den and,
// through O^T += V^T (A^2 masked)^T, to the output tile.
template <class S, bool DECAY>
__device__ __forceinline__ void intra_acc(int mb, int t, const float* Us, const float* Ws, const bf16* vf_hi,
                                          const bf16* vf_lo, int lane, float lt, const float* ls,
                                          f32x4 (&O)[S::NB], float& den) {
  const int n = lane & 15, g = lane >> 4;
  const Op4<true> uf = score_operand(Us + t * S::USTR + 4 * g);   // hi/lo, as in chunk_outputs
  f32x4 A2[S::NMB];
#pragma unroll
  for (int j = 0; j < S::NMB; ++j) {
    A2[j] = zero4();
    if (j <= mb) {
      const f32x4 X = mma<true, true>(score_operand(Ws + (j * 16 + n) * S::USTR + 4 * g), uf, zero4());
      if (j < mb) {   // wave-uniform: only the diagonal tile is masked
#pragma unroll
        for (int r = 0; r < 4; ++r) A2[j][r] = X[r] * X[r];
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) A2[j][r] = (4 * g + r <= n) ? X[r] * X[r] : 0.f;
      }
      if constexpr (DECAY) {   // weight exp(l_t - l_s) of key s = 16j + 4g + r
        const f32x4 lsv = *reinterpret_cast<const f32x4*>(ls + j * 16 + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) A2[j][r] *= __expf(fminf(lt - lsv[r], 0.f));
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) den += A2[j][r];
    }
  }
  // O^T += V^T (A^2 masked)^T: K-block jj = score tiles 2jj (slots 0..3), 2jj+1 (slots 4..7)
#pragma unroll
  for (int jj = 0; jj < S::NJ; ++jj) {
    if (2 * jj <= mb) {
      float x[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = A2[2 * jj][i];
        x[4 + i] = (2 * jj + 1 < S::NMB) ? A2[2 * jj + 1][i] : 0.f;
      }
      const Op8<S::SPLIT> af = make8<S::SPLIT>(x);
#pragma unroll
      for (int nb = 0; nb < S::NB; ++nb)
        O[nb] = mma<S::SPLIT, S::SPLIT>(load_vf<S>(vf_hi, vf_lo, jj, nb, lane), af, O[nb]);
    }
  }
}

// Output gate of token t: den summed over the 4 lane groups (each permlane swap
// exchanges rows between its two outputs, whose sum is the pair sum in every lane),
// y = O / den (0 where the denominator is 0; v_rcp_f32 is within 1 ulp).
template <class S, typename TOut>
__device__ __forceinline__ void gate_store(const f32x4 (&O)[S::NB], float den, const SeqRsrc& rs, int t0, int t,
                                           int lane) {
  const int g = lane >> 4;
  den = row_pair_sum<16>(den);
  den = row_pair_sum<32>(den);
  const float inv = den != 0.f ? __builtin_amdgcn_rcpf(den) : 0.f;
  store_row<S, TOut>(O, inv, rs.y, (t0 + t) * S::DV, t, g);
}

// grid (n_leaf, B*H), block 256.  ws holds each leaf's exclusive prefix state.  DECAY:
// lam [B*H, T] log-decays (see the decay-gate notes above).
// direct (not with DECAY): ws holds the leaf states themselves (no scan ran), and the
// workgroup of leaf g forms its prefix as the symmetric part of S0/z0 (or 0) plus the
// states of leaves 0 .. g-1; the workgroup of the last leaf also adds its own leaf's
// state to that prefix and exports the sum, the final state, to ST/zT (when not NULL) as
// the scan would, before its chunks (the stores drain while it works).
template <class S, typename TIn, typename TOut, bool DECAY = false>
__global__ void __launch_bounds__(256, S::OCC_INTRA)
kata_chunk_intra(const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
                 const float* __restrict__ P, const float* __restrict__ ws, TOut* __restrict__ y,
                 int64_t T, int H, int leaf_chunks, int64_t n_chunks, const float* __restrict__ lam,
                 int direct, const float* __restrict__ S0, const float* __restrict__ z0, float* __restrict__ ST,
                 float* __restrict__ zT) {
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* vf_hi = reinterpret_cast<bf16*>(smem + S::OFF_VF);
  bf16* vf_lo = reinterpret_cast<bf16*>(smem + S::OFF_VF + S::VF_BYTES);
  bf16* hx_hi = reinterpret_cast<bf16*>(smem + S::OFF_HX);
  bf16* hx_lo = reinterpret_cast<bf16*>(smem + S::OFF_HX + S::HX_BYTES);
  float* Us = reinterpret_cast<float*>(smem + S::OFF_U);
  float* Ws = reinterpret_cast<float*>(smem + S::OFF_W);
  float* Wacc = reinterpret_cast<float*>(smem + S::OFF_WACC);
  bf16* Wz = reinterpret_cast<bf16*>(smem + S::OFF_WZ);
  bf16* Zs = reinterpret_cast<bf16*>(smem + S::OFF_Z);
  bf16* Pf = reinterpret_cast<bf16*>(smem + S::OFF_PF);
  float* ls = reinterpret_cast<float*>(smem + S::SMEM);        // DECAY: cumulative log-decays
  float* es = ls + S::C;                                         // DECAY: key weights exp(L_c - l_s)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bh = blockIdx.y;
  const int h = (int)(bh % H);
  const int64_t leaf = blockIdx.x;
  const int64_t c0 = leaf * leaf_chunks;
  const int nch = (int)min<int64_t>(leaf_chunks, n_chunks - c0);
  const int64_t base_tok = bh * T;
  __amdgpu_buffer_rsrc_t rl;
  if constexpr (DECAY) rl = make_rsrc(lam + base_tok, T * 4);

  // the readout K-block 4 holds delta = 8 in slots 0..3; slots 4..7 stay zero
  for (int i = tid; i < S::NB * WAVE; i += 256) {
    const int idx = ((4 * S::NB) * WAVE + i) * 8 + 4;
    *reinterpret_cast<bf16x4*>(hx_hi + idx) = bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
    if constexpr (S::FSPLIT) *reinterpret_cast<bf16x4*>(hx_lo + idx) = bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
  }
  // Roles: wave w takes the M-blocks w, w + 4, ... (token split) and the Z update
  // goes to wave 0, whose M-block has the least intra-chunk work.
  const int tw = wave;
  const bool zrole = wave == 0;
  const bf16x8 sel[2] = {column_selector(0, lane), column_selector(1, lane)};
  // P, the leaf's prefix state and the first chunk's inputs are loaded in this order before
  // any of them is waited for, so the three latencies overlap (loads complete in issue
  // order: P is waited for with the state and chunk loads still in flight, and so on).
  PRows<S> prow;
  read_P_rows<S>(prow, P, h, lane);
  StateAcc<S> st;
  if (!DECAY && direct) {
    state_zero<S>(st);
    if (S0) for_state_elems<S>(st, wave, zrole, lane, [&](int e, float) { return scan_initial(e, S::DV, bh, S0, z0); });
    for (int64_t g = 0; g < leaf; ++g) {
      StateAcc<S> t;
      load_state<S>(t, ws + (bh * (int64_t)gridDim.x + g) * S::E, wave, zrole, lane);
      state_add<S>(st, t);
    }
    if (ST && leaf + 1 == (int64_t)gridDim.x) {   // S0 + every leaf: the canonical final state
      StateAcc<S> t;
      load_state<S>(t, ws + (bh * (int64_t)gridDim.x + leaf) * S::E, wave, zrole, lane);
      state_add<S>(t, st);
      const int64_t pp = (int64_t)P_DIM * P_DIM;
      for_state_elems<S>(t, wave, zrole, lane, [&](int e, float x) {
        int a, b, col;
        bool is_z, mirror;
        if (packed_to_pair(e, S::DV, a, b, col, is_z, mirror)) {
          if (!is_z) {
            ST[(bh * pp + a * P_DIM + b) * S::DV + col] = x;
            if (mirror) ST[(bh * pp + b * P_DIM + a) * S::DV + col] = x;
          } else {
            zT[bh * pp + a * P_DIM + b] = x;
          }
        }
        return x;
      });
    }
  } else {
    load_state<S>(st, ws + (bh * (int64_t)gridDim.x + leaf) * S::E, wave, zrole, lane);
  }

  SeqRsrc rs;
  rs.q = make_rsrc(q + base_tok * S::DIN, T * S::DIN * (int64_t)sizeof(TIn));
  rs.k = make_rsrc(k + base_tok * S::DIN, T * S::DIN * (int64_t)sizeof(TIn));
  rs.v = make_rsrc(v + base_tok * S::DV, T * S::DV * (int64_t)sizeof(TIn));
  rs.y = make_rsrc(y + base_tok * S::DV, T * S::DV * (int64_t)sizeof(TOut));
  const int tc0 = (int)(c0 * S::C);
  ChunkIn<S, TIn> cur;
  load_chunk<S, TIn, true>(cur, rs, tc0, tw, lane);
  if (wave == 0) store_P<S>(Pf, prow, lane);
  publish_state<S>(st, hx_hi, hx_lo, Zs, wave, zrole, lane);
  float lam_next = 0.f;
  if constexpr (DECAY) lam_next = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, (tc0 + lane) * 4, 0, 0));
  __syncthreads();   // P fragments written
  for (int c = 0; c < nch; ++c) {
    const int t0 = tc0 + c * S::C;
    progress_priority(c, nch);
    stage_chunk<S, TIn, true>(cur, Pf, sel, Us, Ws, Wacc, Wz, vf_hi, vf_lo, tw, lane);
    if (c + 1 < nch) load_chunk<S, TIn, true>(cur, rs, t0 + S::C, tw, lane);
    float Lc = 0.f;
    if constexpr (DECAY) {
      const float l = chunk_cumlog(lam_next, lane, Lc);
      if (wave == 0) {
        ls[lane] = l;
        es[lane] = __expf(Lc - l);
      }
      lam_next = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, (t0 + S::C + lane) * 4, 0, 0));
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < S::MBW; ++m) {
      const int mb = tw + 4 * m;
      if (mb < S::NMB) chunk_outputs<S, TOut, DECAY>(mb, Us, Ws, vf_hi, vf_lo, hx_hi, hx_lo, Zs, rs, t0, lane, ls);
    }
    const bool more = c + 1 < nch;
    if constexpr (DECAY) {
      if (more) {
        state_scale<S>(st, __expf(Lc));
        state_update_decay<S>(st, Wacc, es, vf_hi, vf_lo, wave, zrole, lane);
      }
    } else {
      if (more) state_update<S>(st, Wacc, Wz, vf_hi, vf_lo, wave, zrole, lane);
    }
    __syncthreads();
    if (more) publish_state<S>(st, hx_hi, hx_lo, Zs, wave, zrole, lane);
  }
}

// ---- KATA-Mg: g concatenated PSD factors ----------------------------------------------
// The feature is [vec(u_1 u_1^T); ...; vec(u_g u_g^T)] with u_i = P_i x (several PSD
// factors, item "Variantes" of section 2.3 of the gist.science summary; the factors'
// combination is not defined there and is read as concatenation), so a_ts =
// sum_i (u_i,t . w_i,s)^2 and the state is the g one-factor states stacked.

// The projections of the chunk's q and k through one factor (stage_chunk without V).
template <class S, typename TIn>
__device__ __forceinline__ void stage_proj(const ChunkIn<S, TIn>& r, const bf16* Pf, float* Us, float* Ws,
                                           float* Wacc, bf16* Wz, int tw, int lane) {
  const int n = lane & 15, g = lane >> 4;
  ProjP<S> pp;
  read_P<S>(pp, Pf, lane);
#pragma unroll
  for (int m = 0; m < S::MBW; ++m) {
    const int mb = tw + 4 * m;
    if (mb < S::NMB) {
      const f32x4 w = project_tile<S, TIn>(r.k[m], pp);
      *reinterpret_cast<f32x4*>(Wacc + (mb * WAVE + lane) * 4) = w;
      {
        float wv[4] = {w[0], w[1], w[2], w[3]};
        const Op4<true> wz = make4<true>(wv);
        const int idx = ((mb >> 1) * WAVE + lane) * 8 + (mb & 1) * 4;
        *reinterpret_cast<bf16x4*>(Wz + idx) = wz.hi;
        *reinterpret_cast<bf16x4*>(Wz + S::NJ * WAVE * 8 + idx) = wz.lo;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) Ws[(mb * 16 + 4 * g + i) * S::USTR + n] = w[i];
      const f32x4 u = project_tile<S, TIn>(r.q[m], pp);
#pragma unroll
      for (int i = 0; i < 4; ++i) Us[(mb * 16 + 4 * g + i) * S::USTR + n] = u[i];
    }
  }
}

// LDS of the Mg intra kernel: the one-factor layout plus the P fragments of the other
// factors after it.
template <class S, int G>
struct MgLayout {
  static constexpr int SMEM = S::SMEM + (G - 1) * S::PF_BYTES;
  static constexpr int PF_ELEMS = S::PF_BYTES / 2;   // bf16 elements per factor's fragments
};

// grid (n_leaf, B*H), block 256.  ws [B*H*G, n_leaf, E]: row bh*G + i holds factor i's
// exclusive leaf prefix (kata_chunk_state<..., G> then kata_state_scan over B*H*G rows).
// Per chunk: V is staged once; then, factor by factor, the projections through P_i are
// staged, factor i's prefix state is published and read out, its intra tile is added to
// the same output tile and denominator, and its state is advanced; the gate divides
// once at the end.  Two barriers per factor and chunk.
template <class S, typename TIn, typename TOut, int G>
__global__ void __launch_bounds__(256, 2)
kata_chunk_intra_mg(const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
                    const float* __restrict__ P, const float* __restrict__ ws, TOut* __restrict__ y,
                    int64_t T, int H, int leaf_chunks, int64_t n_chunks) {
  using L = MgLayout<S, G>;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* vf_hi = reinterpret_cast<bf16*>(smem + S::OFF_VF);
  bf16* vf_lo = reinterpret_cast<bf16*>(smem + S::OFF_VF + S::VF_BYTES);
  bf16* hx_hi = reinterpret_cast<bf16*>(smem + S::OFF_HX);
  bf16* hx_lo = reinterpret_cast<bf16*>(smem + S::OFF_HX + S::HX_BYTES);
  float* Us = reinterpret_cast<float*>(smem + S::OFF_U);
  float* Ws = reinterpret_cast<float*>(smem + S::OFF_W);
  float* Wacc = reinterpret_cast<float*>(smem + S::OFF_WACC);
  bf16* Wz = reinterpret_cast<bf16*>(smem + S::OFF_WZ);
  bf16* Zs = reinterpret_cast<bf16*>(smem + S::OFF_Z);
  bf16* Pf = reinterpret_cast<bf16*>(smem + S::OFF_PF);      // G factors, PF_ELEMS apart
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bh = blockIdx.y;
  const int h = (int)(bh % H);
  const int64_t leaf = blockIdx.x;
  const int64_t c0 = leaf * leaf_chunks;
  const int nch = (int)min<int64_t>(leaf_chunks, n_chunks - c0);
  const int64_t base_tok = bh * T;

  for (int i = tid; i < S::NB * WAVE; i += 256) {   // readout K-block 4, slots 4..7: zero
    const int idx = ((4 * S::NB) * WAVE + i) * 8 + 4;
    *reinterpret_cast<bf16x4*>(hx_hi + idx) = bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
    if constexpr (S::FSPLIT) *reinterpret_cast<bf16x4*>(hx_lo + idx) = bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
  }
  const int tw = wave;
  const bool zrole = wave == 0;
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < G; ++i) write_P<S>(Pf + i * L::PF_ELEMS, P, h * G + i, lane);
  }
  const bf16x8 sel[2] = {column_selector(0, lane), column_selector(1, lane)};
  StateAcc<S> st[G];
#pragma unroll
  for (int i = 0; i < G; ++i)
    load_state<S>(st[i], ws + ((bh * G + i) * (int64_t)gridDim.x + leaf) * S::E, wave, zrole, lane);

  SeqRsrc rs;
  rs.q = make_rsrc(q + base_tok * S::DIN, T * S::DIN * (int64_t)sizeof(TIn));
  rs.k = make_rsrc(k + base_tok * S::DIN, T * S::DIN * (int64_t)sizeof(TIn));
  rs.v = make_rsrc(v + base_tok * S::DV, T * S::DV * (int64_t)sizeof(TIn));
  rs.y = make_rsrc(y + base_tok * S::DV, T * S::DV * (int64_t)sizeof(TOut));
  const int tc0 = (int)(c0 * S::C);
  ChunkIn<S, TIn> cur;
  load_chunk<S, TIn, true>(cur, rs, tc0, tw, lane);
  __syncthreads();   // P fragments written
  for (int c = 0; c < nch; ++c) {
    const int t0 = tc0 + c * S::C;
    const bool more = c + 1 < nch;
    progress_priority(c, nch);
    f32x4 O[S::MBW][S::NB];
    float den[S::MBW];
#pragma unroll
    for (int m = 0; m < S::MBW; ++m) {
      den[m] = 0.f;
#pragma unroll
      for (int nb = 0; nb < S::NB; ++nb) O[m][nb] = zero4();
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if (i == 0) stage_chunk<S, TIn, true>(cur, Pf, sel, Us, Ws, Wacc, Wz, vf_hi, vf_lo, tw, lane);
      else stage_proj<S, TIn>(cur, Pf + i * L::PF_ELEMS, Us, Ws, Wacc, Wz, tw, lane);
      if (i == G - 1 && more) load_chunk<S, TIn, true>(cur, rs, t0 + S::C, tw, lane);
      publish_state<S>(st[i], hx_hi, hx_lo, Zs, wave, zrole, lane);
      __syncthreads();
#pragma unroll
      for (int m = 0; m < S::MBW; ++m) {
        const int mb = tw + 4 * m;
        if (mb < S::NMB) {
          const int t = mb * 16 + (lane & 15);
          readout_acc<S, false>(t, Us, hx_hi, hx_lo, Zs, lane, O[m], den[m]);
          intra_acc<S, false>(mb, t, Us, Ws, vf_hi, vf_lo, lane, 0.f, nullptr, O[m], den[m]);
        }
      }
      if (more) state_update<S>(st[i], Wacc, Wz, vf_hi, vf_lo, wave, zrole, lane);
      __syncthreads();
    }
#pragma unroll
    for (int m = 0; m < S::MBW; ++m) {
      const int mb = tw + 4 * m;
      if (mb < S::NMB) gate_store<S, TOut>(O[m], den[m], rs, t0, mb * 16 + (lane & 15), lane);
    }
  }
}

// ---- KATA-Sigma-g: g summed PSD factors -------------------------------------------------
// The feature is vec(sum_i u_i u_i^T) (summed PSD factors, item "Variantes" of section 2.3
// of the gist.science summary; read as the sum of the rank-one factors), so the state is
// one p*p x dv state (the sum of the factor states), the readout is sum_i phi(u_i)^T H, the
// denominator's state part sum_i u_i^T Z u_i, and a_ts = sum_i sum_j (u_i,t . w_j,s)^2.

// LDS of the Sigma-g intra kernel: the one-factor layout, then per extra factor its u and
// w rows, key tiles, hi/lo key fragments and P fragments.
template <class S, int G>
struct SgLayout {
  static constexpr int XB = 2 * S::U_BYTES + S::WACC_BYTES + S::WZ_BYTES + S::PF_BYTES;
  static constexpr int SMEM = S::SMEM + (G - 1) * XB;
  static __device__ __forceinline__ int off(int i) { return S::SMEM + (i - 1) * XB; }
};

// grid (n_leaf, B*H), block 256.  ws [B*H, n_leaf, E]: the exclusive leaf prefix of the
// summed state (kata_chunk_state<..., G, true> then kata_state_scan).  Per chunk: V and the
// projections of all factors are staged, the state (published at the end of the previous
// chunk) is read out through every factor's query feature, the g*g score tiles of all
// factor pairs are added, the gate divides, and every factor's keys update the state.
template <class S, typename TIn, typename TOut, int G>
__global__ void __launch_bounds__(256, 2)
kata_chunk_intra_sg(const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
                    const float* __restrict__ P, const float* __restrict__ ws, TOut* __restrict__ y,
                    int64_t T, int H, int leaf_chunks, int64_t n_chunks) {
  using L = SgLayout<S, G>;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* vf_hi = reinterpret_cast<bf16*>(smem + S::OFF_VF);
  bf16* vf_lo = reinterpret_cast<bf16*>(smem + S::OFF_VF + S::VF_BYTES);
  bf16* hx_hi = reinterpret_cast<bf16*>(smem + S::OFF_HX);
  bf16* hx_lo = reinterpret_cast<bf16*>(smem + S::OFF_HX + S::HX_BYTES);
  bf16* Zs = reinterpret_cast<bf16*>(smem + S::OFF_Z);
  float* Us[G];
  float* Ws[G];
  float* Wacc[G];
  bf16* Wz[G];
  bf16* Pf[G];
  Us[0] = reinterpret_cast<float*>(smem + S::OFF_U);
  Ws[0] = reinterpret_cast<float*>(smem + S::OFF_W);
  Wacc[0] = reinterpret_cast<float*>(smem + S::OFF_WACC);
  Wz[0] = reinterpret_cast<bf16*>(smem + S::OFF_WZ);
  Pf[0] = reinterpret_cast<bf16*>(smem + S::OFF_PF);
#pragma unroll
  for (int i = 1; i < G; ++i) {
    unsigned char* xb = smem + L::off(i);
    Us[i] = reinterpret_cast<float*>(xb);
    Ws[i] = reinterpret_cast<float*>(xb + S::U_BYTES);
    Wacc[i] = reinterpret_cast<float*>(xb + 2 * S::U_BYTES);
    Wz[i] = reinterpret_cast<bf16*>(xb + 2 * S::U_BYTES + S::WACC_BYTES);
    Pf[i] = reinterpret_cast<bf16*>(xb + 2 * S::U_BYTES + S::WACC_BYTES + S::WZ_BYTES);
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bh = blockIdx.y;
  const int h = (int)(bh % H);
  const int64_t leaf = blockIdx.x;
  const int64_t c0 = leaf * leaf_chunks;
  const int nch = (int)min<int64_t>(leaf_chunks, n_chunks - c0);
  const int64_t base_tok = bh * T;

  for (int i = tid; i < S::NB * WAVE; i += 256) {   // readout K-block 4, slots 4..7: zero
    const int idx = ((4 * S::NB) * WAVE + i) * 8 + 4;
    *reinterpret_cast<bf16x4*>(hx_hi + idx) = bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
    if constexpr (S::FSPLIT) *reinterpret_cast<bf16x4*>(hx_lo + idx) = bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
  }
  const int tw = wave;
  const bool zrole = wave == 0;
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < G; ++i) write_P<S>(Pf[i], P, h * G + i, lane);
  }
  const bf16x8 sel[2] = {column_selector(0, lane), column_selector(1, lane)};
  StateAcc<S> st;
  load_state<S>(st, ws + (bh * (int64_t)gridDim.x + leaf) * S::E, wave, zrole, lane);
  publish_state<S>(st, hx_hi, hx_lo, Zs, wave, zrole, lane);

  SeqRsrc rs;
  rs.q = make_rsrc(q + base_tok * S::DIN, T * S::DIN * (int64_t)sizeof(TIn));
  rs.k = make_rsrc(k + base_tok * S::DIN, T * S::DIN * (int64_t)sizeof(TIn));
  rs.v = make_rsrc(v + base_tok * S::DV, T * S::DV * (int64_t)sizeof(TIn));
  rs.y = make_rsrc(y + base_tok * S::DV, T * S::DV * (int64_t)sizeof(TOut));
  const int tc0 = (int)(c0 * S::C);
  ChunkIn<S, TIn> cur;
  load_chunk<S, TIn, true>(cur, rs, tc0, tw, lane);
  __syncthreads();   // P fragments written
  for (int c = 0; c < nch; ++c) {
    const int t0 = tc0 + c * S::C;
    const bool more = c + 1 < nch;
    progress_priority(c, nch);
    stage_chunk<S, TIn, true>(cur, Pf[0], sel, Us[0], Ws[0], Wacc[0], Wz[0], vf_hi, vf_lo, tw, lane);
#pragma unroll
    for (int i = 1; i < G; ++i) stage_proj<S, TIn>(cur, Pf[i], Us[i], Ws[i], Wacc[i], Wz[i], tw, lane);
    if (more) load_chunk<S, TIn, true>(cur, rs, t0 + S::C, tw, lane);
    __syncthreads();
#pragma unroll
    for (int m = 0; m < S::MBW; ++m) {
      const int mb = tw + 4 * m;
      if (mb < S::NMB) {
        const int t = mb * 16 + (lane & 15);
        f32x4 O[S::NB];
#pragma unroll
        for (int nb = 0; nb < S::NB; ++nb) O[nb] = zero4();
        float den = 0.f;
#pragma unroll
        for (int i = 0; i < G; ++i) readout_acc<S, false>(t, Us[i], hx_hi, hx_lo, Zs, lane, O, den);
#pragma unroll
        for (int i = 0; i < G; ++i) {
#pragma unroll
          for (int j = 0; j < G; ++j)
            intra_acc<S, false>(mb, t, Us[i], Ws[j], vf_hi, vf_lo, lane, 0.f, nullptr, O, den);
        }
        gate_store<S, TOut>(O, den, rs, t0, t, lane);
      }
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < G; ++i) state_update<S>(st, Wacc[i], Wz[i], vf_hi, vf_lo, wave, zrole, lane);
    }
    __syncthreads();
    if (more) publish_state<S>(st, hx_hi, hx_lo, Zs, wave, zrole, lane);
  }
}

}  // namespace kata
