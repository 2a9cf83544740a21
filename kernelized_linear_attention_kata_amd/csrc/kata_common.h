// kata_common.h - shared device definitions for the KATA gfx950 kernels.
//
// MFMA fragment layouts used throughout (wave64, gfx950):
//   v_mfma_f32_16x16x32_bf16  A[m][k]: lane l holds m = l%16, k = 8*(l/16) + i  (i = 0..7)
//                             B[k][n]: lane l holds n = l%16, k = 8*(l/16) + i
//                             C[m][n]: lane l holds n = l%16, m = 4*(l/16) + i  (i = 0..3)
//   v_mfma_f32_16x16x16_bf16  same with k = 4*(l/16) + i (i = 0..3)
// Throughout, "g" = l/16 (the lane group) and "n" = l%16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kata {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16;

constexpr int WAVE = 64;
constexpr int P_DIM = 16;          // projection dimension p
constexpr int NDELTA = 9;          // circulant diagonals delta = 0..8 of the symmetric u u^T
constexpr int DPACK = NDELTA * P_DIM;   // 144 packed feature slots (136 distinct + 8 zero)
constexpr int READ_KB = 5;         // readout K-blocks of 32 packed features (last one half zero)

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ f32x4 mfma32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// A bf16 MFMA operand that is either one bf16 value per element or a hi/lo pair
// (hi = bf16(x), lo = bf16(x - hi)) carrying ~16 significant bits; products of
// split operands take three MFMAs (hi*hi + hi*lo + lo*hi).
template <bool SPLIT> struct Op8 { bf16x8 hi; };
template <> struct Op8<true> { bf16x8 hi, lo; };
template <bool SPLIT> struct Op4 { bf16x4 hi; };
template <> struct Op4<true> { bf16x4 hi, lo; };

template <bool SPLIT>
__device__ __forceinline__ Op8<SPLIT> make8(const float (&x)[8]) {
  Op8<SPLIT> o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o.hi[i] = (bf16)x[i];
  if constexpr (SPLIT) {
#pragma unroll
    for (int i = 0; i < 8; ++i) o.lo[i] = (bf16)(x[i] - (float)o.hi[i]);
  }
  return o;
}
template <bool SPLIT>
__device__ __forceinline__ Op4<SPLIT> make4(const float (&x)[4]) {
  Op4<SPLIT> o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o.hi[i] = (bf16)x[i];
  if constexpr (SPLIT) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o.lo[i] = (bf16)(x[i] - (float)o.hi[i]);
  }
  return o;
}

// acc += A * B with either operand optionally split.
template <bool SA, bool SB>
__device__ __forceinline__ f32x4 mma(const Op8<SA>& a, const Op8<SB>& b, f32x4 c) {
  c = mfma32(a.hi, b.hi, c);
  if constexpr (SB) c = mfma32(a.hi, b.lo, c);
  if constexpr (SA) c = mfma32(a.lo, b.hi, c);
  return c;
}
template <bool SA, bool SB>
__device__ __forceinline__ f32x4 mma(const Op4<SA>& a, const Op4<SB>& b, f32x4 c) {
  c = mfma16(a.hi, b.hi, c);
  if constexpr (SB) c = mfma16(a.hi, b.lo, c);
  if constexpr (SA) c = mfma16(a.lo, b.hi, c);
  return c;
}

// x + (x of the lane 16 or 32 away, i.e. lane ^ 16 or lane ^ 32) in every lane.
// v_permlane16_swap / v_permlane32_swap exchange rows between their two operands; fed
// the same value twice, the two results hold the two halves of each row pair, and
// their sum is the pair sum whichever half each one holds.
template <int DIST>
__device__ __forceinline__ float row_pair_sum(float x) {
  const unsigned u = __float_as_uint(x);
  if constexpr (DIST == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    static_assert(DIST == 32, "row pair distance");
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}

// ---- buffer (range-checked) memory access ----------------------------------------
// A raw buffer resource covers one sequence; loads past its end return 0 and
// stores past it are dropped, so ragged tails need no branches.  Offsets are
// 32-bit byte offsets (the host limits a sequence to < 2 GiB).
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
constexpr int BUF_OOB = 0x7ffffff0;          // an offset past any sequence: reads 0
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ i32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// ---- element loads / stores in either storage dtype ------------------------------
__device__ __forceinline__ float bf16_bits_to_float(u16 b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, int64_t i, float x) { p[i] = x; }
};
template <> struct Elem<bf16> {
  static __device__ __forceinline__ float load(const bf16* p, int64_t i) { return (float)p[i]; }
  static __device__ __forceinline__ void store(bf16* p, int64_t i, float x) { p[i] = (bf16)x; }
};

// Weight of packed slot (delta, a) on the query side: the unordered pair
// {a, (a+delta) mod 16} appears twice in the full p*p feature unless it is the
// diagonal; for delta = 8 the slots a >= 8 repeat the pairs of a < 8 and are unused.
__device__ __forceinline__ float query_weight(int delta, int a) {
  return delta == 0 ? 1.f : (delta == 8 ? (a < 8 ? 2.f : 0.f) : 2.f);
}
__device__ __forceinline__ float key_weight(int delta, int a) {
  return (delta == 8 && a >= 8) ? 0.f : 1.f;
}

}  // namespace kata
