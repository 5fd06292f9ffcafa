// Matrix-core helpers shared by the MFMA attention kernels (gfx950 only):
// the 32x32x16 bf16/f16 product, the swizzled row-major LDS tile geometry
// and the half-wave reductions.
//
// MFMA 32x32x16 register layout (per lane l, h = l / 32):
//   A: 8 consecutive k of row l % 32;  B: the same 8 k of column l % 32;
//   C: column l % 32, register r holds row 8*(r/4) + 4*h + (r%4).
// A and B use the same k slots, so a contraction needs no assumption about
// which k-slot the hardware gives each half-wave; only the C layout is
// relied on.
//
// ds_read_b64_tr_b16, per group of 16 lanes: if lane r addresses 4 halves
// M[r][0..3], lane i receives M[4e + i/4][i%4] for e = 0..3.
#pragma once

#include <type_traits>

#include "attn_device.h"

namespace attn {

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Mfma;
template <> struct Mfma<__bf16> {
  typedef bf16x8 vec8;
  typedef __bf16 vec4 __attribute__((ext_vector_type(4)));
  typedef __bf16 vec2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ f32x16 mma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // acc + x.x + x.y, summing the rounded weights (v_dot2_f32_bf16).
  static __device__ __forceinline__ float sum2(vec2 x, float acc) {
    const vec2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(x, one, acc, false);
  }
};
template <> struct Mfma<_Float16> {
  typedef f16x8 vec8;
  typedef _Float16 vec4 __attribute__((ext_vector_type(4)));
  typedef _Float16 vec2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ f32x16 mma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float sum2(vec2 x, float acc) {
    const vec2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(x, one, acc, false);
  }
};

// Tile geometry: rows of D halves (2*D bytes) in 16-byte chunks, chunk c of
// row r stored at position c ^ swz(r).  LDS serves 256 bytes per pass: 16
// lanes of a 16-byte read, 32 lanes of an 8-byte read.  The swizzle puts
// the 16 rows of one K-fragment pass (same chunk, consecutive rows) and the
// 4 rows x 2 feature groups of one V transpose-read pass on distinct banks.
template <int D> struct Geo {
  static constexpr int CPR = D / 8;                     // chunks per row
  static constexpr int RPL = CPR >= 16 ? 1 : 16 / CPR;  // rows per 256 bytes
  static constexpr __host__ __device__ int swz(int row) {
    const int u = row / RPL;  // 256-byte line of the row
    return CPR == 16 ? 4 * (u & 3) + ((u >> 2) & 3)
         : CPR == 8  ? 4 * (u & 1) + ((u >> 1) & 3)
         : CPR == 4  ? (u & 3)
                     : (u & 1);
  }
  static __device__ __forceinline__ int off(int row, int chunk) {
    return row * (2 * D) + ((chunk ^ swz(row)) << 4);
  }
  // The K fragment offsets are reused 32 rows down and the V offsets 16 rows
  // down: both steps must leave the swizzle unchanged.
  static constexpr bool steps_keep_swizzle() {
    for (int r = 0; r < 16; ++r)
      if (swz(r + 32) != swz(r) || swz(r + 16) != swz(r) || swz(r + 48) != swz(r)) return false;
    return true;
  }
};

// max / sum of x over lanes l and l ^ 32 (the two half-waves), on the VALU
// (no LDS round trip): v_permlane32_swap leaves {x[l], x[l ^ 32]} in its two
// results.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Calls f(std::integral_constant<int, i>) for i = B .. E-1 in order: a loop
// whose index is a compile-time constant in the body, so register arrays it
// indexes stay in registers whatever the unroller decides.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

}  // namespace attn
