// kata_flash.h - the flash-style O(T^2) KATA forward (no state): for each query
// block, the masked squared score tiles (U W^T)^2 of all earlier key blocks times
// [V | 1], accumulated on chip and divided at the end.
//
// This is the first of the two operating points of the hardware section of the
// gist.science summary of "Kernelized Linear Attention" (arXiv 2607.17419, section
// 2.3: a flash-attention-like forward that never materialises the state, the fused
// kernel behind the 1.6x-over-FlashAttention-2 figure of the abstract).  The weights
// a_ts = (u_t . w_s)^2 are non-negative and need no running maximum: numerator and
// denominator are plain sums (section 2.1 of the summary: the normaliser is the sum
// of the weights).
//
// Two kernels:
//  * kata_flash_prep  (grid T_pad/64 x B*H): u = P q, w = P k (as hi/lo bf16 pairs) and
//    V, regrouped into MFMA operand order and written once per token to a workspace.
//  * kata_flash_attn  (T_pad/128 * B*H workgroups, XCD-aware order): 4 waves x
//    32 queries; 64-key blocks of w and V fragments copied into an LDS ring.  Per
//    32-key tile: X^T = W U^T (three 32x32x16 MFMAs, K = p, hi/lo operands), squared and
//    masked on the VALU, then O^T += V^T (X^2)^T (32x32x16 MFMAs, K = 16 keys).  Lane l
//    holds output columns of query l%32, so the denominator needs one lane-pair sum.
//
// Precision: the weight (u.w)^2 of a query nearly orthogonal to a key is a small
// difference of large products; with u and w as single bf16 its error would be about
// 2^-8 |u| |w| |u.w|, which decides y_t where the denominator is a small fraction of
// sum_s |u_t|^2 |w_s|^2.  The hi/lo pairs (hi*hi + hi*lo + lo*hi) bring the error of u.w
// to about 2^-16 |u| |w|.
#pragma once

#include "kata_chunk.h"

namespace kata {

constexpr int FL_WAVES = 4;                // waves per workgroup, 32 queries each
constexpr int FL_QB = 32 * FL_WAVES;       // queries per workgroup
constexpr int FL_KB = 64;       // keys per staged block
constexpr int FL_DV = 64;

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma3232(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Layouts (v_mfma_f32_32x32x16_bf16, wave64: A lane l holds row l%32, k = 8*(l/32) + i;
// B lane l holds column l%32, k = 8*(l/32) + i; C lane l holds column l%32 and rows
// 8*(i/4) + 4*(l/32) + i%4, i = 0..15).  Workspace of one (b, h) sequence, T_pad = T
// rounded up to FL_QB, rows past T zero:
//  * U  [2][T_pad][16] bf16: u_t as hi (plane 0) and lo = bf16(u - hi) (plane 1); a query
//    lane reads u_t[8h .. 8h+7] of both (B operands of the score).
//  * Wf [2][T_pad/32][64 lanes][8] bf16: hi and lo planes of the A operand of the score
//    tile of 32 keys, lane l holding w_{32x + l%32}[8h .. 8h+7], h = l/32
//    (lane-contiguous, conflict-free reads).
//  * Vf [T_pad/16][2][64 lanes][8] bf16: the A operand V^T of the value MFMA for the
//    16-key group kappa and the 32-column tile ct: lane l (column 32ct + l%32, h = l/32)
//    holds v at keys 16kappa + 4h + i and 16kappa + 8 + 4h + i (i = 0..3), the order in
//    which the score accumulator hands its squared entries to the value MFMA.
__host__ __device__ constexpr int64_t flash_ws_elems(int64_t tpad) { return tpad * (4 * P_DIM + FL_DV); }

// ---- kata_flash_prep -----------------------------------------------------------
// One 64-token chunk per workgroup, wave w projects tokens 16w..16w+15; V goes
// through LDS to be regrouped into value-MFMA fragments.
template <typename TIn>
__global__ void __launch_bounds__(256)
kata_flash_prep(const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
                const float* __restrict__ P, bf16* __restrict__ ws, int64_t T, int64_t tpad, int H) {
  using S = Shape<64, 64, 64, false>;
  __shared__ __align__(16) bf16 vs[64][FL_DV + 8];   // the chunk's V rows (padded rows)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int64_t bh = blockIdx.y;
  const int h = (int)(bh % H);
  const int t0 = (int)blockIdx.x * 64;       // first token of the chunk
  ProjP<S> pp;
#pragma unroll
  for (int kk = 0; kk < S::KD; ++kk) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = P[((int64_t)h * P_DIM + n) * S::DIN + proj_col<S>(g, kk, i)];
    pp.f[kk] = make8<true>(x);
  }
  SeqRsrc rs;
  rs.q = make_rsrc(q + bh * T * S::DIN, T * S::DIN * (int64_t)sizeof(TIn));
  rs.k = make_rsrc(k + bh * T * S::DIN, T * S::DIN * (int64_t)sizeof(TIn));
  rs.v = make_rsrc(v + bh * T * S::DV, T * S::DV * (int64_t)sizeof(TIn));
  ChunkIn<S, TIn> r;
  load_chunk<S, TIn, true>(r, rs, t0, wave, lane);   // rows past T read zero
  // V rows to LDS: lane (t, g) holds columns 32kk + 8g .. +7 of row 16w + t
#pragma unroll
  for (int kk = 0; kk < S::KV; ++kk)
    *reinterpret_cast<bf16x8*>(&vs[16 * wave + n][32 * kk + 8 * g]) = r.v[0][kk].x;

  bf16* base = ws + bh * flash_ws_elems(tpad);
  bf16* Ub = base;                          // hi plane; the lo plane follows at + tpad * P_DIM
  bf16* Wf = base + 2 * tpad * P_DIM;       // hi plane; the lo plane follows at + tpad * P_DIM
  bf16* Vf = base + 4 * tpad * P_DIM;
  const int tok = t0 + 16 * wave + n;        // this lane's token in the transposed tiles
  // u^T, w^T tiles: P (A operand, lane (a, g)) times q^T / k^T (B operand, lane (t, g)):
  // lane (t, g) receives u_t[4g .. 4g+3]
  f32x4 u = zero4(), w = zero4();
#pragma unroll
  for (int kk = 0; kk < S::KD; ++kk) {
    Op8<false> qa, ka;
    qa.hi = r.q[0][kk].x;
    ka.hi = r.k[0][kk].x;
    u = mma<true, false>(pp.f[kk], qa, u);
    w = mma<true, false>(pp.f[kk], ka, w);
  }
  {
    float uv[4] = {u[0], u[1], u[2], u[3]};
    float wv[4] = {w[0], w[1], w[2], w[3]};
    const Op4<true> us = make4<true>(uv), ws4 = make4<true>(wv);
    const int64_t ui = (int64_t)tok * P_DIM + 4 * g;
    *reinterpret_cast<bf16x4*>(Ub + ui) = us.hi;
    *reinterpret_cast<bf16x4*>(Ub + tpad * P_DIM + ui) = us.lo;
    // features 4g..4g+3 of key tok: lane (tok%32) + 32*(g/2) of its 32-key tile, slots 4*(g%2)..
    const int64_t wi = (((int64_t)(tok >> 5) * WAVE + (tok & 31) + 32 * (g >> 1)) * 8) + 4 * (g & 1);
    *reinterpret_cast<bf16x4*>(Wf + wi) = ws4.hi;
    *reinterpret_cast<bf16x4*>(Wf + tpad * P_DIM + wi) = ws4.lo;
  }
  __syncthreads();
  // value fragments: 4 key groups x 2 column tiles of the chunk, 2 per thread
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int f = wave + 4 * pass;
    const int kap = f >> 1, ct = f & 1;
    const int c = lane & 31, hh = lane >> 5;
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[i] = vs[16 * kap + 4 * hh + i][32 * ct + c];
      o[4 + i] = vs[16 * kap + 8 + 4 * hh + i][32 * ct + c];
    }
    const int64_t gk = t0 / 16 + kap;          // global 16-key group
    *reinterpret_cast<bf16x8*>(Vf + ((gk * 2 + ct) * WAVE + lane) * 8) = o;
  }
}

// ---- kata_flash_attn -----------------------------------------------------------
// Key blocks are copied straight from the workspace into an LDS ring of FL_RING
// buffers by buffer_load ... lds (no registers), FL_RING - 1 blocks ahead of use.  A
// buffer is [Wf hi block: 2 tiles x 64 lanes x 16 B = 2 KB | Wf lo block: 2 KB | Vf
// block: 4 groups x 2 tiles x 64 lanes x 16 B = 8 KB], twelve 1 KB pieces: wave w copies
// pieces w, w + 4 and w + 8, so each wave has exactly FL_DMA_PER_WAVE loads per block in
// flight and waits for a block with an exact vmcnt.
constexpr int FL_W_BYTES = FL_KB * P_DIM * 2;
constexpr int FL_V_BYTES = FL_KB * FL_DV * 2;
constexpr int FL_PIECES = 12;   // 1 KB pieces per buffer
constexpr int FL_BUF_BYTES = FL_PIECES * 1024;
// Two buffers (the copy of block kb + 1 runs during block kb): 24 KB per workgroup, six
// workgroups of four waves per CU (6 waves per SIMD: 78 VGPRs, the register budget).
// Measured against five per CU: three workgroups of eight waves (6 waves per SIMD) 3%
// slower; 16 KB buffers whose last 4 KB were copies read past the workspace (zeros), so
// that eight waves had equal shares, 6% slower; three 12 KB buffers at four workgroups per
// CU, 4% slower (21% against the kernel with the staged output).
constexpr int FL_RING = 2;
constexpr int FL_DMA_PER_WAVE = FL_PIECES / FL_WAVES;
static_assert(FL_PIECES % FL_WAVES == 0 && FL_PIECES * 1024 == 2 * FL_W_BYTES + FL_V_BYTES,
              "every wave copies the same number of pieces, which cover the block");

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
#define KATA_WAIT_VMCNT(N) \
  __builtin_amdgcn_s_waitcnt(((N) & 0xf) | (((N) >> 4) << 14) | (0x7 << 4) | (0xf << 8))

template <typename TOut>
__global__ void __launch_bounds__(64 * FL_WAVES, 6)
kata_flash_attn(const bf16* __restrict__ ws, TOut* __restrict__ y, int64_t T, int64_t tpad, int nbh) {
  __shared__ __align__(16) unsigned char sm[FL_RING * FL_BUF_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31, hh = lane >> 5;
  // XCD-aware order (1-D grid of nqb * nbh workgroups): workgroups are dispatched to
  // the 8 XCDs round-robin, and each XCD has its own L2, so all query blocks of a
  // sequence go to one XCD (when nbh is a multiple of 8) and reuse its key blocks from
  // that L2.  Within a sequence the heaviest query blocks come first.
  const int nqb = (int)(tpad / FL_QB);
  const int L = (int)blockIdx.x;
  int64_t bh;
  int qi;
  if (nbh % 8 == 0) {
    const int slot = L >> 3;
    bh = (int64_t)(slot / nqb) * 8 + (L & 7);
    qi = slot % nqb;
  } else {
    bh = L / nqb;
    qi = L % nqb;
  }
  const int qb = nqb - 1 - qi;
  const bf16* base = ws + bh * flash_ws_elems(tpad);
  const int w_off = (int)(2 * tpad * P_DIM * 2);      // byte offsets inside the workspace:
  const int wlo_off = (int)(3 * tpad * P_DIM * 2);    // W hi and lo planes, then V
  const int v_off = (int)(4 * tpad * P_DIM * 2);
  const __amdgpu_buffer_rsrc_t rws = make_rsrc(base, flash_ws_elems(tpad) * 2);

  const int q0 = qb * FL_QB + 32 * wave;             // this wave's 32 queries
  const int tq = q0 + c32;                           // this lane's query
  const bf16x8 ub = *reinterpret_cast<const bf16x8*>(base + (int64_t)tq * P_DIM + 8 * hh);
  const bf16x8 ubl = *reinterpret_cast<const bf16x8*>(base + (tpad + tq) * P_DIM + 8 * hh);
  f32x16 O[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[ct][i] = 0.f;
  float den = 0.f;

  const int nkb = (qb + 1) * (FL_QB / FL_KB);        // key blocks up to the block's last query
  auto dma = [&](int kb) {
    unsigned char* dst = sm + (kb % FL_RING) * FL_BUF_BYTES;
#pragma unroll
    for (int i = 0; i < FL_DMA_PER_WAVE; ++i) {
      const int c = wave + FL_WAVES * i;               // 1 KB piece of the buffer
      const int src = c < 2 ? w_off + kb * FL_W_BYTES + c * 1024
                    : (c < 4 ? wlo_off + kb * FL_W_BYTES + (c - 2) * 1024
                             : (c < 12 ? v_off + kb * FL_V_BYTES + (c - 4) * 1024 : BUF_OOB));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rws, (lds_void*)(dst + c * 1024), 16,
                                               src >= BUF_OOB ? BUF_OOB : src + lane * 16, 0, 0, 0);
    }
  };
#pragma unroll
  for (int i = 0; i < FL_RING - 1; ++i)
    if (i < nkb) dma(i);
  // the u loads complete here, together with the first ring copies (both in flight at
  // once, one memory latency at the workgroup's start instead of two): consumed by an
  // (empty) asm statement, they get their wait at this point; otherwise their wait
  // sinks to the first use of u in the loop and covers every later copy in flight
  asm volatile("" ::"v"(ub), "v"(ubl));
  for (int kb = 0; kb < nkb; ++kb) {
    // this wave's pieces of block kb have landed once at most the later blocks' are
    // outstanding; the barrier then makes every wave's pieces visible and also ends
    // everyone's use of the buffer the next copy goes to (block kb - 1's)
    const int later = min(nkb - 1 - kb, FL_RING - 2);
    if (later >= 2) KATA_WAIT_VMCNT(2 * FL_DMA_PER_WAVE);
    else if (later == 1) KATA_WAIT_VMCNT(FL_DMA_PER_WAVE);
    else KATA_WAIT_VMCNT(0);
    asm volatile("s_barrier" ::: "memory");
    if (kb + FL_RING - 1 < nkb) dma(kb + FL_RING - 1);
    const bf16* Wl = reinterpret_cast<const bf16*>(sm + (kb % FL_RING) * FL_BUF_BYTES);
    const bf16* Wlo = Wl + FL_KB * P_DIM;
    const bf16* Vl = Wl + 2 * FL_KB * P_DIM;
    const int s_blk = kb * FL_KB;
    if (s_blk > q0 + 31) continue;                   // wave-uniform: every key after every query
    const bool full = s_blk + FL_KB - 1 <= q0;       // no key after any query of the wave
#pragma unroll
    for (int x = 0; x < 2; ++x) {                    // 32-key score tiles
      const int s0 = s_blk + 32 * x;
      if (!full && s0 > q0 + 31) continue;           // wave-uniform
      const bf16x8 wf = *reinterpret_cast<const bf16x8*>(Wl + (x * WAVE + lane) * 8);
      const bf16x8 wfl = *reinterpret_cast<const bf16x8*>(Wlo + (x * WAVE + lane) * 8);
      f32x16 zero16;
#pragma unroll
      for (int i = 0; i < 16; ++i) zero16[i] = 0.f;
      // lane: keys s0 + 8(i/4) + 4hh + i%4 of query tq; hi*hi + hi*lo + lo*hi
      const f32x16 X = mfma3232(wfl, ub, mfma3232(wf, ubl, mfma3232(wf, ub, zero16)));
      float a2[16];
      if (full || s0 + 31 <= q0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) a2[i] = X[i] * X[i];
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) a2[i] = (s0 + 8 * (i >> 2) + 4 * hh + (i & 3) <= tq) ? X[i] * X[i] : 0.f;
      }
#pragma unroll
      for (int a = 0; a < 2; ++a) {                  // 16-key groups: squared entries 8a .. 8a+7
        bf16x8 af;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          den += a2[8 * a + i];
          af[i] = (bf16)a2[8 * a + i];
        }
        // V fragments read at their use, not with the score operands: 78 VGPRs, six
        // workgroups per CU (reading all four up front needs 82 VGPRs, five per CU)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
          O[ct] = mfma3232(*reinterpret_cast<const bf16x8*>(Vl + (((2 * x + a) * 2 + ct) * WAVE + lane) * 8), af, O[ct]);
      }
    }
  }
  // gate and store: den(t) = the sum of the lane pair (hh = 0, 1) of query tq
  den = row_pair_sum<32>(den);
  const float inv = den != 0.f ? __builtin_amdgcn_rcpf(den) : 0.f;
  __amdgpu_buffer_rsrc_t ry = make_rsrc(y + bh * T * FL_DV, T * FL_DV * (int64_t)sizeof(TOut));
  if constexpr (IsBf16<TOut>::value) {
    // The block's 128 x 64 bf16 output tile goes through the LDS ring, idle by now: a
    // lane holds 4-column pieces of its query's row, which stored directly would leave
    // as 16-byte pieces of 128-byte lines.  Read back as 16-byte pieces in row order,
    // every store instruction writes 8 whole rows.
    constexpr int OSTR = FL_DV + 8;                  // bf16 row stride: 144 B, 16-byte aligned
    static_assert(FL_QB * OSTR * 2 <= FL_RING * FL_BUF_BYTES, "the output tile fits the ring");
    bf16* ot = reinterpret_cast<bf16*>(sm);
    __syncthreads();                                 // every wave is done with the last block
    const int ql = 32 * wave + c32;                  // this lane's query within the block
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {                  // columns 32ct + 8j + 4hh .. +3
        bf16x4 b;
#pragma unroll
        for (int r = 0; r < 4; ++r) b[r] = (bf16)(O[ct][4 * j + r] * inv);
        *reinterpret_cast<bf16x4*>(ot + ql * OSTR + 32 * ct + 8 * j + 4 * hh) = b;
      }
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < FL_QB * FL_DV / 8 / (64 * FL_WAVES); ++p) {
      const int piece = p * 64 * FL_WAVES + tid;     // 8-column piece c8 of block row rl
      const int rl = piece >> 3, c8 = piece & 7;
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(ot + rl * OSTR + 8 * c8);
      const int64_t tr = (int64_t)qb * FL_QB + rl;
      const int off = tr < T ? (int)(tr * FL_DV * 2) + 16 * c8 : BUF_OOB;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), ry, off, 0, Y_STORE_POLICY);
    }
  } else {
    const int row = tq < T ? (int)(tq * FL_DV * (int64_t)sizeof(TOut)) : BUF_OOB;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {                  // columns 32ct + 8j + 4hh .. +3
        f32x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = O[ct][4 * j + r] * inv;
        const int col = 32 * ct + 8 * j + 4 * hh;
        Store4<TOut>::st(ry, row >= BUF_OOB ? BUF_OOB : row + col * (int)sizeof(TOut), o);
      }
    }
  }
}

}  // namespace kata
