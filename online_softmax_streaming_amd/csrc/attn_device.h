// Device-side helpers shared by the attention kernels (gfx950 only).
//
// The running-state arithmetic follows the answer-key page ("Compare
// reasoning after your own attempt"), rows A1 and A3: a state (m, l) stands
// for sum exp(x) = l * e^m; merging or extending a state re-expresses both
// parts relative to the larger maximum, and the unnormalised output a is
// rescaled by the same factor as l.  Inside the kernels every logit is kept
// in base-2 units (x * log2 e), so each exponential is one v_exp_f32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_inff();

// 2^x with the hardware transcendental (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Reference point for rescaling: the running max, or 0 while nothing has
// been seen.  A row whose max is still -inf would otherwise compute
// (-inf) - (-inf) = NaN ("Kernel Notes & Checklist", gotchas ledger: ghost
// rows must be pinned).
__device__ __forceinline__ float pinned_ref(float m) { return m == kNegInf ? 0.f : m; }

// One A1 merge in base-2 units: returns the weights that carry each side to
// the common maximum, and the new maximum.  Both weights are 0 for an empty
// side, so merging two empty states gives the empty state.
struct MergeWeights {
  float m, w1, w2;
};
__device__ __forceinline__ MergeWeights merge_weights_log2(float m1, float m2) {
  MergeWeights r;
  r.m = fmaxf(m1, m2);
  const float ref = pinned_ref(r.m);
  r.w1 = exp2_hw(m1 - ref);
  r.w2 = exp2_hw(m2 - ref);
  return r;
}

// The full 128-bit product a * m as (lo, hi), from four 32 x 32 -> 64
// products: with a = a1 2^32 + a0 and m = m1 2^32 + m0, t = a1 m0 + hi(a0 m0)
// and u = a0 m1 + lo(t) cannot overflow 64 bits, lo = lo(u) 2^32 + lo(a0 m0)
// and hi = a1 m1 + hi(t) + hi(u).  Each product is one 32-bit multiply-add
// into a 64-bit register pair, where hi and lo taken separately would redo
// the cross products.
__device__ __forceinline__ void mul_wide(uint64_t a, uint64_t m, uint64_t& lo, uint64_t& hi) {
  const uint32_t a0 = (uint32_t)a, a1 = (uint32_t)(a >> 32), m0 = (uint32_t)m, m1 = (uint32_t)(m >> 32);
  const uint64_t p00 = (uint64_t)a0 * m0;
  const uint64_t t = (uint64_t)a1 * m0 + (p00 >> 32);
  const uint64_t u = (uint64_t)a0 * m1 + (uint32_t)t;
  hi = (uint64_t)a1 * m1 + (t >> 32) + (u >> 32);
  lo = (u << 32) | (uint32_t)p00;
}

// a ^ b ^ c with one three-input bitwise operation per 32-bit half (truth
// table 0x96: odd parity of the three bits); the compiler otherwise issues
// two two-input xors.
__device__ __forceinline__ uint64_t xor3(uint64_t a, uint64_t b, uint64_t c) {
  const uint32_t lo = __builtin_amdgcn_bitop3_b32((uint32_t)a, (uint32_t)b, (uint32_t)c, 0x96);
  const uint32_t hi = __builtin_amdgcn_bitop3_b32((uint32_t)(a >> 32), (uint32_t)(b >> 32),
                                                  (uint32_t)(c >> 32), 0x96);
  return (uint64_t)lo | ((uint64_t)hi << 32);
}

// Philox4x64-10, the counter-based generator of Salmon, Moraes, Dror and
// Shaw ("Parallel random numbers: as easy as 1, 2, 3", SC 2011): ten rounds
// on a 4-word counter under a 2-word key.  Each round multiplies counter
// words 0 and 2 by the two multipliers, and the new counter is
// (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); the key
// is bumped by the two Weyl constants between rounds.  The counter is
// replaced by the output.
__device__ __forceinline__ void philox4x64_10(uint64_t (&c)[4], uint64_t k0, uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    uint64_t lo0, hi0, lo1, hi1;
    mul_wide(c[0], M0, lo0, hi0);
    mul_wide(c[2], M1, lo1, hi1);
    const uint64_t n0 = xor3(hi1, c[1], k0), n2 = xor3(hi0, c[3], k1);
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

// Element conversions.  Output casts are round-to-nearest-even.
template <typename T> __device__ __forceinline__ float to_f32(T x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x) { return (T)x; }

}  // namespace attn
