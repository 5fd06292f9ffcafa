// Attention backward on gfx950 matrix cores (bf16 / f16 inputs): dQ, dK and
// dV of O = softmax(scale Q K^T) V, recomputing P tile by tile from each
// row's forward state (m, l) instead of storing it.
//
// Per head, in natural units, with lse = m + ln l (the A1 state of the
// answer-key page, "Compare reasoning after your own attempt", row A1):
//   P  = exp(scale Q K^T - lse) on visible keys, 0 elsewhere
//   dV = P^T dO
//   dP = dO V^T
//   dS = P * (dP - Delta),   Delta = rowsum(dO * O)
//   dQ = scale dS K,          dK = scale dS^T Q
// dS is the row-wise softmax vector-Jacobian product y * (g - <y, g>) of
// the workshops page's I2 ("Intermediate and advanced kernel workshops",
// softmax backward) with y = P and g = dP.  Because O = P V, <P, dP> equals
// rowsum(dO * O): one dot product of length D per row instead of a
// reduction over all keys.
//
// Two kernels, ordered on one stream:
//   1. dq (query-stationary; the forward kernel's structure): a workgroup
//      owns 32*NW query rows, a wave 32 of them, with their Q and dO rows
//      in registers; K and V tiles of 64 keys stream through LDS.  Per tile
//      S^T = K Q^T and dP^T = V dO^T put one query per lane, so lse and
//      Delta are per-lane scalars, and dQ^T += K^T dS^T reads K^T from the
//      row-major K tile with LDS transpose reads.  Before its key loop the
//      wave forms Delta from its O and dO rows and the base-2 lse from
//      (m, l), and writes both for kernel 2.
//   2. dkdv (key-stationary): a workgroup owns 32*NW keys, a wave 32 of
//      them, with their K and V rows in registers; Q and dO tiles of 64
//      query rows, with the rows' (lse, Delta), stream through LDS.  Per
//      tile S = Q K^T and dP = dO V^T put one key per lane; dV^T += dO^T P
//      and dK^T += Q^T dS read dO^T and Q^T by transpose reads.  With
//      grouped K/V heads a workgroup walks the query heads of its group in
//      turn, so dK and dV sum over the group without atomics.
// Every output element is written by one lane, once: no atomics, and the
// result does not depend on scheduling.
//
// Rounding: S, dP and every accumulator are FP32; P and dS are rounded to
// the input type only as matrix-core operands (as the forward rounds P
// before P V); outputs get one round-to-nearest-even cast.
//
// Padding: tiles are staged with buffer loads whose range ends at the last
// real row, so rows past Nq or Nk arrive as zeros.  A ghost query row then
// has Q = dO = 0 and (lse, Delta) = (0, 0): its P is finite and it adds
// exactly zero to dK and dV.  A ghost key in kernel 2 only affects its own,
// unstored, column.  In kernel 1 a ghost key's P = exp2(-lse) could
// overflow, so the ragged key tile is masked there; the causal mask is
// applied in both kernels on tiles that cross the diagonal.
//
// Causal visibility is the forward's: key j is visible to query i iff
// j <= i + (Nk - Nq).

#include <type_traits>

#include "attn_kernels.h"
#include "attn_mfma.h"

namespace attn {
namespace {

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* m;  // forward row state, natural units
  const float* l;
  void* dq;
  void* dk;
  void* dv;
  float* stat;  // [B*H*Nq][2]: base-2 lse, Delta
  int Nq, Nk;
  int group;    // query heads per K/V head
  int ntile;    // query tiles (dq) or key blocks (dkdv) per head
  int nwork;    // workgroups per head: ntile, or ceil(ntile / 2) causal pairs
  int total;    // real workgroups
  int per_xcd;  // gridDim.x / 8
  float c;      // scale * log2(e)
  float scale;
  // dQ with the keys split over workgroups (SPLIT dQ kernels): work item
  // (head, query tile, split s) covers key tiles [s * kpt, (s + 1) * kpt)
  // and writes its FP32 share of dQ to dq_part[s][row][.], rows = B*H*Nq.
  float* dq_part;
  int S, kpt;
  int64_t rows;
};

constexpr int kBT = 64;  // rows of every streamed tile (keys in dq, queries in dkdv)
#ifndef ATTN_BWD_PF
#define ATTN_BWD_PF 6
#endif
#ifndef ATTN_BWD_TPF
#define ATTN_BWD_TPF 4
#endif
constexpr int kPF = ATTN_BWD_PF;    // row-fragment reads in flight ahead of their MFMA
constexpr int kTPF = ATTN_BWD_TPF;  // transpose reads in flight ahead of their MFMA
constexpr float kPosInf = __builtin_inff();
#ifndef ATTN_BWD_STAGE_STRIDE
#define ATTN_BWD_STAGE_STRIDE 2
#endif
constexpr int kStageStride = ATTN_BWD_STAGE_STRIDE;  // MFMAs between two staging loads (dK/dV)

// XCD-aware workgroup order (consecutive ids go round-robin over the 8
// XCDs): each XCD walks a contiguous range of logical workgroups, so the
// tiles one head streams stay in one L2.
__device__ __forceinline__ int logical_workgroup(int per_xcd) {
  const int bid = blockIdx.x;
  return (bid & 7) * per_xcd + (bid >> 3);
}

// Per-lane byte offsets of the transpose-read A operand (X^T for a
// row-major tile X of kBT rows): for feature block n and half `half`, lane
// i of each 16-lane group addresses row 8*half + 4*h32 + i/4 and features
// 4*(i%4) onward of its group's 16, so that after the transpose the lane
// holds feature 32n + l32 of rows 16c + {4*h32 + 0..3} (first read) and
// 16c + 8 + {4*h32 + 0..3} (second), c being the 16-row group: exactly the
// rows that registers 8*(c&1) + 0..7 of C-layout block c/2 hold.
template <int D, int NB>
__device__ __forceinline__ void transpose_offsets(int lane, int (&off)[NB][2]) {
  typedef Geo<D> G;
  const int i = lane & 15;
  const int h32 = lane >> 5;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int row = 8 * half + 4 * h32 + (i >> 2);
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      int col = 16 * ((lane >> 4) & 1) + 32 * n + 4 * (i & 3);
      if (col >= D) col -= D;  // D = 16: rows 16..31 of the result are computed, then discarded
      off[n][half] = G::off(row, col >> 3) + ((col & 7) << 1);
    }
  }
}

// Buffer resources of one staged (query head, tile) pair of the dK/dV
// kernel: Q rows, dO rows and (lse2, Delta) rows, and the tile's first row.
struct StageSource {
  __amdgpu_buffer_rsrc_t q, g, st;
  int q0;
};

template <typename T>
__device__ __forceinline__ typename Mfma<T>::vec8 transpose_read(const unsigned char* tile, int o0,
                                                                 int o1) {
  typedef typename Mfma<T>::vec8 vec8;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, tile + o0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, tile + o1));
  return __builtin_bit_cast(vec8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Stage rows [r0, r0 + kBT) of two row-major [rows, D] arrays into two
// swizzled LDS tiles with buffer loads that write LDS directly: lane l of a
// wave fills the 16 bytes at its wave's 1 KB block base + 16*l.  Rows at or
// past `rows` are outside the buffer range and read as zero.
template <typename T, int D, int NT>
__device__ __forceinline__ void stage_pair(const T* x, const T* y, int rows, int r0,
                                           unsigned char* tx, unsigned char* ty, int tid,
                                           int wave) {
  typedef Geo<D> G;
  constexpr int NSLOT = kBT * D * 2 / 16;
  constexpr int NPT = (NSLOT + NT - 1) / NT;
  static_assert(NSLOT % 64 == 0, "a wave moves whole 1 KB LDS blocks");
  const uint32_t bytes = (uint32_t)rows * (uint32_t)(2 * D);
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(x), 0, (int)bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t yr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(y), 0, (int)bytes, 0x00020000);
#pragma unroll
  for (int u = 0; u < NPT; ++u) {
    const int sl = tid + u * NT;
    const int sl0 = wave * 64 + u * NT;
    if (NSLOT % NT == 0 || sl0 < NSLOT) {
      const int row = sl / G::CPR;
      const int chunk = (sl % G::CPR) ^ G::swz(row);
      const int j = min(r0 + row, rows);
      const uint32_t vo = (uint32_t)j * (uint32_t)(2 * D) + (uint32_t)(chunk << 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, LDS_PTR(void, tx + sl0 * 16), 16, (int)vo, 0,
                                               0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(yr, LDS_PTR(void, ty + sl0 * 16), 16, (int)vo, 0,
                                               0, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// Kernel 1: dQ, plus (lse2, Delta) per row.
// ---------------------------------------------------------------------------
template <typename T, int D, int NW, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dq_kernel(BwdArgs a) {
  typedef typename Mfma<T>::vec8 vec8;
  typedef typename Mfma<T>::vec4 vec4;
  typedef Geo<D> G;
  constexpr int BM = 32 * NW;
  constexpr int BN = kBT;
  constexpr int DP = D < 32 ? 32 : D;
  constexpr int KC = D / 16;
  constexpr int NB = DP / 32;
  constexpr int NT = NW * 64;
  constexpr int TILE = BN * D * 2;
  static_assert(G::steps_keep_swizzle(), "tile steps must keep the LDS swizzle");

  __shared__ __attribute__((aligned(1024))) unsigned char smem0[2][TILE];  // [K, V]
  __shared__ __attribute__((aligned(1024))) unsigned char smem1[2][TILE];
  auto tile_ptr = [&](int buf, int kv) __attribute__((always_inline)) -> unsigned char* {
    return buf == 0 ? &smem0[kv][0] : &smem1[kv][0];
  };

  const int logical = logical_workgroup(a.per_xcd);
  if (logical >= a.total) return;
  const int bh = logical / a.nwork;
  const int rr = logical - bh * a.nwork;
  // Causal: query tile ntile-1-r, then tile r, so workgroups stream equal
  // numbers of key tiles.  Split: one query tile, split sp of its keys.
  const int sp = SPLIT ? rr % a.S : 0;
  const int npass = !SPLIT && CAUSAL && a.ntile - 1 - rr != rr ? 2 : 1;
  for (int pass = 0; pass < npass; ++pass) {
    const int qt = SPLIT ? rr / a.S : CAUSAL ? (pass == 0 ? a.ntile - 1 - rr : rr) : rr;
    const int Nq = a.Nq, Nk = a.Nk, off = Nk - Nq;
    const int64_t qbase = (int64_t)bh * Nq * D;
    const T* __restrict__ Qh = static_cast<const T*>(a.q) + qbase;
    const T* __restrict__ Oh = static_cast<const T*>(a.o) + qbase;
    const T* __restrict__ dOh = static_cast<const T*>(a.dout) + qbase;
    T* __restrict__ dQh = static_cast<T*>(a.dq) + qbase;
    const T* Kh = static_cast<const T*>(a.k) + (int64_t)(bh / a.group) * Nk * D;
    const T* Vh = static_cast<const T*>(a.v) + (int64_t)(bh / a.group) * Nk * D;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h32 = lane >> 5;
    const int l32 = lane & 31;
    const int i0 = qt * BM;
    const int qw0 = i0 + wave * 32;
    const int qrow = qw0 + l32;
    const bool real = qrow < Nq;
    const float c = a.c;

    // Q and dO rows as B operands (8 consecutive features per k-chunk);
    // ghost rows are zero.
    vec8 qf[KC], gf[KC];
    float dlt = 0.f;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int64_t e = (int64_t)qrow * D + kc * 16 + h32 * 8;
      qf[kc] = real ? *reinterpret_cast<const vec8*>(Qh + e) : vec8{};
      gf[kc] = real ? *reinterpret_cast<const vec8*>(dOh + e) : vec8{};
      const vec8 of = real ? *reinterpret_cast<const vec8*>(Oh + e) : vec8{};
#pragma unroll
      for (int i = 0; i < 8; ++i) dlt = __builtin_fmaf(to_f32<T>(gf[kc][i]), to_f32<T>(of[i]), dlt);
    }
    dlt = half_sum(dlt);  // Delta = rowsum(dO * O)
    // Base-2 lse; a row with no visible key (l = 0) gets +inf, so every P
    // of that row is exp2(-inf) = 0.
    float lse2 = 0.f;
    if (real) {
      const int64_t row = (int64_t)bh * Nq + qrow;
      const float ll = a.l[row];
      lse2 = ll > 0.f ? __builtin_fmaf(a.m[row], kLog2e, log2f(ll)) : kPosInf;
      if (h32 == 0 && sp == 0) {
        a.stat[2 * row] = lse2;
        a.stat[2 * row + 1] = dlt;
      }
    }

    int kend = Nk;
    if (CAUSAL) kend = min(Nk, min(i0 + BM, Nq) + off);
    const int nvis = kend > 0 ? (kend + BN - 1) / BN : 0;
    // Key tiles [t_first, ntiles) of this work item.
    const int t_first = SPLIT ? sp * a.kpt : 0;
    const int ntiles = SPLIT ? min(nvis, t_first + a.kpt) : nvis;

    int koff[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) koff[kc] = G::off(l32, 2 * kc + h32);
    int toff[NB][2];
    transpose_offsets<D, NB>(lane, toff);

    f32x16 acc[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[n] = f32x16{};

    auto compute = [&](auto bufc, int j0, bool need_mask) {
      constexpr int buf = decltype(bufc)::value;
      const unsigned char* kt = tile_ptr(buf, 0);
      const unsigned char* vt = tile_ptr(buf, 1);

      // S^T = K Q^T (MFMAs 0..NS-1) and dP^T = V dO^T (NS..2NS-1): operand
      // i is key block (i % NS) / KC, feature chunk i % KC of K or V.
      constexpr int NS = (BN / 32) * KC;
      auto fread = [&](int i) {
        const unsigned char* t = i < NS ? kt : vt;
        const int ii = i < NS ? i : i - NS;
        return *reinterpret_cast<const vec8*>(t + koff[ii % KC] + (ii / KC) * 32 * 2 * D);
      };
      vec8 ff[2 * NS];
#pragma unroll
      for (int i = 0; i < kPF && i < 2 * NS; ++i) ff[i] = fread(i);
      f32x16 s[BN / 32], dp[BN / 32];
#pragma unroll
      for (int mb = 0; mb < BN / 32; ++mb) s[mb] = dp[mb] = f32x16{};
#pragma unroll
      for (int i = 0; i < 2 * NS; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (i + kPF < 2 * NS) ff[i + kPF] = fread(i + kPF);
        if (i < NS)
          s[i / KC] = Mfma<T>::mma(ff[i], qf[i % KC], s[i / KC]);
        else
          dp[(i - NS) / KC] = Mfma<T>::mma(ff[i], gf[(i - NS) % KC], dp[(i - NS) / KC]);
      }
      __builtin_amdgcn_sched_barrier(0);

      // K^T operands of dQ^T += K^T dS^T: feature block i / (BN/16), key
      // group i % (BN/16); the first ones are requested before the softmax.
      constexpr int NV = NB * (BN / 16);
      vec8 kt_f[NV];
      auto tread = [&](int i) {
        const int n = i / (BN / 16), c2 = i % (BN / 16);
        return transpose_read<T>(kt, toff[n][0] + 16 * c2 * 2 * D, toff[n][1] + 16 * c2 * 2 * D);
      };
#pragma unroll
      for (int i = 0; i < kTPF && i < NV; ++i) kt_f[i] = tread(i);
      __builtin_amdgcn_sched_barrier(0);

      if (need_mask) {
#pragma unroll
        for (int mb = 0; mb < BN / 32; ++mb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = j0 + mb * 32 + (r >> 2) * 8 + h32 * 4 + (r & 3);
            const bool vis = j < Nk && (!CAUSAL || j <= qrow + off);
            s[mb][r] = vis ? s[mb][r] : kNegInf;
          }
        }
      }
      // P^T = exp2(S^T c - lse2), dS^T = P^T (dP^T - Delta), rounded to T.
      vec8 dsf[BN / 16];
#pragma unroll
      for (int c2 = 0; c2 < BN / 16; ++c2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int mb = c2 >> 1, r = (c2 & 1) * 8 + e;
          const float p = exp2_hw(__builtin_fmaf(s[mb][r], c, -lse2));
          dsf[c2][e] = from_f32<T>(p * (dp[mb][r] - dlt));
        }
      }

      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (i + kTPF < NV) kt_f[i + kTPF] = tread(i + kTPF);
        acc[i / (BN / 16)] = Mfma<T>::mma(kt_f[i], dsf[i % (BN / 16)], acc[i / (BN / 16)]);
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    const uint32_t kv_rows = (uint32_t)Nk;
    if (ntiles > t_first) {
      stage_pair<T, D, NT>(Kh, Vh, (int)kv_rows, t_first * BN, tile_ptr(0, 0), tile_ptr(0, 1), tid,
                           wave);
      __syncthreads();
      const int q_last = min(qw0 + 32, Nq) - 1;
      auto step = [&](auto bufc, int t) {
        constexpr int buf = decltype(bufc)::value;
        const int j0 = t * BN;
        if (t + 1 < ntiles)
          stage_pair<T, D, NT>(Kh, Vh, (int)kv_rows, j0 + BN, tile_ptr(buf ^ 1, 0),
                               tile_ptr(buf ^ 1, 1), tid, wave);
        const bool active = qw0 < Nq && (!CAUSAL || j0 <= q_last + off);
        if (active) {
          const bool need_mask = (j0 + BN > Nk) || (CAUSAL && j0 + BN - 1 > qw0 + off);
          compute(bufc, j0, need_mask);
        }
        __syncthreads();
      };
      for (int t = t_first; t < ntiles; t += 2) {
        step(std::integral_constant<int, 0>{}, t);
        if (t + 1 < ntiles) step(std::integral_constant<int, 1>{}, t + 1);
      }
    }

    // dQ = scale * (dS K): lane holds features n*32 + 8g + 4*h32 + 0..3 of
    // its query row.  Split: this split's FP32 share.
    if (SPLIT && real) {
      float* row = a.dq_part + ((int64_t)sp * a.rows + (int64_t)bh * Nq + qrow) * D;
#pragma unroll
      for (int n = 0; n < NB; ++n) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = n * 32 + g * 8 + h32 * 4;
          if (d0 < D)
            *reinterpret_cast<f32x4*>(row + d0) =
                f32x4{acc[n][g * 4] * a.scale, acc[n][g * 4 + 1] * a.scale,
                      acc[n][g * 4 + 2] * a.scale, acc[n][g * 4 + 3] * a.scale};
        }
      }
    } else if (real) {
      T* row = dQh + (int64_t)qrow * D;
#pragma unroll
      for (int n = 0; n < NB; ++n) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = n * 32 + g * 8 + h32 * 4;
          if (d0 < D) {
            vec4 o4;
#pragma unroll
            for (int e = 0; e < 4; ++e) o4[e] = from_f32<T>(acc[n][g * 4 + e] * a.scale);
            *reinterpret_cast<vec4*>(row + d0) = o4;
          }
        }
      }
    }
  }  // pass
}

// ---------------------------------------------------------------------------
// Kernel 2: dK and dV.
// ---------------------------------------------------------------------------
#ifndef ATTN_BWD_KV_WAVES_PER_EU
#define ATTN_BWD_KV_WAVES_PER_EU 1
#endif

template <typename T, int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(ATTN_BWD_KV_WAVES_PER_EU)))
void bwd_dkdv_kernel(BwdArgs a) {
  typedef typename Mfma<T>::vec8 vec8;
  typedef typename Mfma<T>::vec4 vec4;
  typedef Geo<D> G;
  constexpr int BK = 32 * NW;  // keys per workgroup
  constexpr int BQ = kBT;      // query rows per tile
  constexpr int DP = D < 32 ? 32 : D;
  constexpr int KC = D / 16;
  constexpr int NB = DP / 32;
  constexpr int NT = NW * 64;
  constexpr int TILE = BQ * D * 2;
  constexpr int STAT = 1024 * NW;  // per wave: (lse2, Delta) of 128 rows, the tile uses 64
  static_assert(G::steps_keep_swizzle(), "tile steps must keep the LDS swizzle");

  __shared__ __attribute__((aligned(1024))) unsigned char smem0[2][TILE];  // [Q, dO]
  __shared__ __attribute__((aligned(1024))) unsigned char smem1[2][TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char stat0[STAT];
  __shared__ __attribute__((aligned(1024))) unsigned char stat1[STAT];
  auto tile_ptr = [&](int buf, int x) __attribute__((always_inline)) -> unsigned char* {
    return buf == 0 ? &smem0[x][0] : &smem1[x][0];
  };
  auto stat_ptr = [&](int buf) __attribute__((always_inline)) -> unsigned char* {
    return buf == 0 ? &stat0[0] : &stat1[0];
  };

  const int logical = logical_workgroup(a.per_xcd);
  if (logical >= a.total) return;
  const int bhkv = logical / a.nwork;
  const int rr = logical - bhkv * a.nwork;
  // Causal: key block ntile-1-r (few visible queries), then block r (many).
  const int npass = CAUSAL && a.ntile - 1 - rr != rr ? 2 : 1;
  for (int pass = 0; pass < npass; ++pass) {
    const int kb = CAUSAL ? (pass == 0 ? a.ntile - 1 - rr : rr) : rr;
    const int Nq = a.Nq, Nk = a.Nk, off = Nk - Nq;
    const int64_t kbase = (int64_t)bhkv * Nk * D;
    const T* __restrict__ Kh = static_cast<const T*>(a.k) + kbase;
    const T* __restrict__ Vh = static_cast<const T*>(a.v) + kbase;
    T* __restrict__ dKh = static_cast<T*>(a.dk) + kbase;
    T* __restrict__ dVh = static_cast<T*>(a.dv) + kbase;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h32 = lane >> 5;
    const int l32 = lane & 31;
    const int k0 = kb * BK;
    const int kw0 = k0 + wave * 32;
    const int krow = kw0 + l32;
    const float c = a.c;

    // K and V rows as B operands; ghost keys are zero.
    vec8 kf[KC], vf[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int64_t e = (int64_t)krow * D + kc * 16 + h32 * 8;
      kf[kc] = krow < Nk ? *reinterpret_cast<const vec8*>(Kh + e) : vec8{};
      vf[kc] = krow < Nk ? *reinterpret_cast<const vec8*>(Vh + e) : vec8{};
    }

    // Query tiles holding a query that sees key k0: from row k0 - off on.
    const int nqt = (Nq + BQ - 1) / BQ;
    const int t0 = CAUSAL ? min(nqt, max(0, k0 - off) / BQ) : 0;
    const int nt = nqt - t0;
    const int nit = a.group * nt;  // (query head of the group, tile) pairs

    int qoff[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) qoff[kc] = G::off(l32, 2 * kc + h32);
    int toff[NB][2];
    transpose_offsets<D, NB>(lane, toff);

    f32x16 adv[NB], adk[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) adv[n] = adk[n] = f32x16{};

    // Staging of (query head, tile) pair `it` into one LDS buffer, one load
    // instruction at a time, so the loads can be spread between the MFMAs of
    // the tile being computed: part u < NPT moves this thread's u-th 16-byte
    // slot of the Q tile, NPT <= u < 2*NPT of the dO tile, and part 2*NPT
    // the tile's (lse2, Delta) rows into the wave's own 1 KB copy, lane l
    // holding rows 2l, 2l+1 (a copy per wave keeps the staging free of
    // branches).  Rows past Nq are out of the buffer range and read as zero.
    constexpr int NSLOT = BQ * D * 2 / 16;
    constexpr int NPT = (NSLOT + NT - 1) / NT;
    constexpr int NPART = 2 * NPT + 1;
    static_assert(NSLOT % 64 == 0, "a wave moves whole 1 KB LDS blocks");
    auto source = [&](int it) __attribute__((always_inline)) -> StageSource {
      const int g = it / nt;
      const int q0 = (t0 + it - g * nt) * BQ;
      const int64_t bh = (int64_t)bhkv * a.group + g;
      const uint32_t bytes = (uint32_t)Nq * (uint32_t)(2 * D);
      StageSource src;
      src.q = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<T*>(static_cast<const T*>(a.q) + bh * Nq * D), 0, (int)bytes, 0x00020000);
      src.g = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<T*>(static_cast<const T*>(a.dout) + bh * Nq * D), 0, (int)bytes, 0x00020000);
      src.st = __builtin_amdgcn_make_buffer_rsrc(a.stat + 2 * bh * Nq, 0,
                                                 (int)((uint32_t)Nq * 8u), 0x00020000);
      src.q0 = q0;
      return src;
    };
    auto stage_part = [&](const StageSource& src, int buf, int u) __attribute__((always_inline)) {
      if (u < 2 * NPT) {
        const int uu = u % NPT;
        const int sl = tid + uu * NT;
        const int sl0 = wave * 64 + uu * NT;
        if (NSLOT % NT == 0 || sl0 < NSLOT) {
          const int row = sl / G::CPR;
          const int chunk = (sl % G::CPR) ^ G::swz(row);
          const int j = min(src.q0 + row, Nq);
          const uint32_t vo = (uint32_t)j * (uint32_t)(2 * D) + (uint32_t)(chunk << 4);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(u < NPT ? src.q : src.g,
                                                   LDS_PTR(void, tile_ptr(buf, u < NPT ? 0 : 1) + sl0 * 16),
                                                   16, (int)vo, 0, 0, 0);
        }
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            src.st, LDS_PTR(void, stat_ptr(buf) + wave * 1024), 16,
            (int)((uint32_t)src.q0 * 8u + (uint32_t)lane * 16u), 0, 0, 0);
      }
    };

    // One tile in four phases over its two 32-query blocks, so the softmax
    // gradient of one block runs on the VALU while the matrix cores work on
    // the other (one wave per SIMD: nothing else would fill the gaps):
    //   1: S, dP of block 0
    //   2: S, dP of block 1     + P, dS of block 0
    //   3: dV, dK of block 0    + P, dS of block 1
    //   4: dV, dK of block 1
    // Every MFMA operand read from LDS is issued kPF MFMAs ahead of its use,
    // across phase boundaries, and the loads of the next tile into the other
    // buffer are spread evenly between the MFMAs.
    auto compute = [&](auto bufc, int q0, bool need_mask, const StageSource& nsrc) {
      constexpr int buf = decltype(bufc)::value;
      const unsigned char* qt = tile_ptr(buf, 0);
      const unsigned char* gt = tile_ptr(buf, 1);
      const float* st = reinterpret_cast<const float*>(stat_ptr(buf) + wave * 1024);
      static_assert(BQ == 64, "two 32-query blocks per tile");
      // Causal mask: key krow is hidden from the query of register r of
      // block mb iff 32mb + 8(r/4) + r%4 < kq (the lane's 4*h32 row offset is
      // folded into kq, so each test compares an immediate); kq is below
      // every row when the tile needs no mask (a select, not a branch).
      const int kq = need_mask ? krow - q0 - off - 4 * h32 : -(1 << 30);
      constexpr int NF = 2 * KC;  // S and dP MFMAs of one block
      constexpr int NG = 4 * NB;  // dV and dK MFMAs of one block
      constexpr int NSTEP = 2 * NF + 2 * NG;
      // Staging loads go out early (one every kStageStride MFMAs from the
      // start) so they have landed by the barrier that ends the tile.
      constexpr int SSTRIDE = NSTEP / NPART < kStageStride ? NSTEP / NPART : kStageStride;
      static_assert(SSTRIDE >= 1, "one staging load per MFMA at most");

      // Operand of MFMA k, in issue order.  S/dP steps: Q (i < KC) or dO
      // fragment, query block mb.  dV/dK steps: dO^T (i < 2NB) or Q^T,
      // feature block n = (i % 2NB) / 2, 16-query group 2mb + i % 2.
      auto read_op = [&](auto kk) __attribute__((always_inline)) -> vec8 {
        constexpr int k = decltype(kk)::value;
        if constexpr (k < 2 * NF) {
          constexpr int mb = k / NF, i = k % NF;
          const unsigned char* t = i < KC ? qt : gt;
          return *reinterpret_cast<const vec8*>(t + qoff[i % KC] + mb * 32 * 2 * D);
        } else {
          constexpr int mb = (k - 2 * NF) / NG, i = (k - 2 * NF) % NG;
          constexpr int ii = i % (2 * NB);
          constexpr int c2 = 2 * mb + (ii & 1), n = ii >> 1;
          const unsigned char* t = i < 2 * NB ? gt : qt;
          return transpose_read<T>(t, toff[n][0] + 16 * c2 * 2 * D, toff[n][1] + 16 * c2 * 2 * D);
        }
      };

      f32x16 s[2], dp[2];
      vec8 pf[2][2], dsf[2][2];  // [block][16-query group]
      vec8 op[NSTEP];
      f32x4 sv[2][4][2];  // (lse2, Delta) of 4 rows: [block][row group][pair of rows]

      auto mma_step = [&](auto kk) __attribute__((always_inline)) {
        constexpr int k = decltype(kk)::value;
        if constexpr (k < 2 * NF) {
          constexpr int mb = k / NF, i = k % NF;
          if constexpr (i < KC) s[mb] = Mfma<T>::mma(op[k], kf[i], s[mb]);
          else dp[mb] = Mfma<T>::mma(op[k], vf[i - KC], dp[mb]);
        } else {
          constexpr int mb = (k - 2 * NF) / NG, i = (k - 2 * NF) % NG;
          constexpr int ii = i % (2 * NB), n = ii >> 1, cc = ii & 1;
          if constexpr (i < 2 * NB) adv[n] = Mfma<T>::mma(op[k], pf[mb][cc], adv[n]);
          else adk[n] = Mfma<T>::mma(op[k], dsf[mb][cc], adk[n]);
        }
      };
      // Rows 32mb + 8g4 + 4*h32 + 0..3: the rows of registers 4g4..4g4+3.
      auto read_stats = [&](int mb, int g4) __attribute__((always_inline)) {
        const int qr = 32 * mb + 8 * g4 + 4 * h32;
        sv[mb][g4][0] = *reinterpret_cast<const f32x4*>(st + 2 * qr);
        sv[mb][g4][1] = *reinterpret_cast<const f32x4*>(st + 2 * qr + 4);
      };
      auto grad = [&](auto mbc, auto rc) __attribute__((always_inline)) {
        constexpr int mb = decltype(mbc)::value, r = decltype(rc)::value;
        // The next row group's statistics are requested one group ahead.
        if constexpr ((r & 3) == 0) {
          if constexpr (r < 12) read_stats(mb, (r >> 2) + 1);
          else if constexpr (mb == 0) read_stats(1, 0);
        }
        const f32x4 pr = sv[mb][r >> 2][(r >> 1) & 1];
        const float l2 = pr[2 * (r & 1)], dl = pr[2 * (r & 1) + 1];
        float x = s[mb][r];
        if (32 * mb + 8 * (r >> 2) + (r & 3) < kq) x = kNegInf;
        const float p = exp2_hw(__builtin_fmaf(x, c, -l2));
        pf[mb][r >> 3][r & 7] = from_f32<T>(p);
        dsf[mb][r >> 3][r & 7] = from_f32<T>(p * (dp[mb][r] - dl));
      };

      s[0] = s[1] = dp[0] = dp[1] = f32x16{};
      static_for<0, (kPF < NSTEP ? kPF : NSTEP)>([&](auto kk) { op[decltype(kk)::value] = read_op(kk); });
      read_stats(0, 0);
      static_for<0, NSTEP>([&](auto kk) {
        constexpr int k = decltype(kk)::value;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (k + kPF < NSTEP)
          op[k + kPF] = read_op(std::integral_constant<int, k + kPF>{});
        mma_step(kk);
        if constexpr (k % SSTRIDE == SSTRIDE - 1 && k / SSTRIDE < NPART)
          stage_part(nsrc, buf ^ 1, k / SSTRIDE);
        // Phase 2 (k in [NF, 2NF)) grads block 0, phase 3 block 1; the 16
        // registers are spread evenly over the phase's MFMAs.
        if constexpr (k >= NF && k < 2 * NF) {
          constexpr int j = k - NF;
          static_for<16 * j / NF, 16 * (j + 1) / NF>(
              [&](auto rc) { grad(std::integral_constant<int, 0>{}, rc); });
        } else if constexpr (k >= 2 * NF && k < 2 * NF + NG) {
          constexpr int j = k - 2 * NF;
          static_for<16 * j / NG, 16 * (j + 1) / NG>(
              [&](auto rc) { grad(std::integral_constant<int, 1>{}, rc); });
        }
      });
      __builtin_amdgcn_sched_barrier(0);
    };

    if (nit > 0) {
      {
        const StageSource s0 = source(0);
#pragma unroll
        for (int u = 0; u < NPART; ++u) stage_part(s0, 0, u);
      }
      __syncthreads();
      auto step = [&](auto bufc, int it) {
        constexpr int buf = decltype(bufc)::value;
        const int g = it / nt;
        const int q0 = (t0 + it - g * nt) * BQ;
        // After the last pair the loads fetch the current tile again into
        // the idle buffer, which nothing reads: staging stays branch-free.
        const StageSource nsrc = source(it + 1 < nit ? it + 1 : it);
        // A causal wave whose keys no query of this tile sees (only on a
        // pass's first tile) still runs the tile with every score masked:
        // P = dS = 0 adds nothing, it would wait at the barrier anyway, and
        // a data-dependent branch here costs the loop ~100 registers.
        if (kw0 < Nk) {
          const bool need_mask = CAUSAL && kw0 + 31 > q0 + off;
          compute(bufc, q0, need_mask, nsrc);
        } else {
#pragma unroll
          for (int u = 0; u < NPART; ++u) stage_part(nsrc, buf ^ 1, u);
        }
        // Buffer buf^1 was last read in step it-1, before that step's
        // barrier; this barrier also waits for the loads into it.
        __syncthreads();
      };
      for (int it = 0; it < nit; it += 2) {
        step(std::integral_constant<int, 0>{}, it);
        if (it + 1 < nit) step(std::integral_constant<int, 1>{}, it + 1);
      }
    }

    // dV = (dO^T P)^T and dK = scale (Q^T dS)^T: lane holds features
    // n*32 + 8g + 4*h32 + 0..3 of its key row.
    if (krow < Nk) {
      T* vrow = dVh + (int64_t)krow * D;
      T* krow_p = dKh + (int64_t)krow * D;
#pragma unroll
      for (int n = 0; n < NB; ++n) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = n * 32 + g * 8 + h32 * 4;
          if (d0 < D) {
            vec4 v4, k4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              v4[e] = from_f32<T>(adv[n][g * 4 + e]);
              k4[e] = from_f32<T>(adk[n][g * 4 + e] * a.scale);
            }
            *reinterpret_cast<vec4*>(vrow + d0) = v4;
            *reinterpret_cast<vec4*>(krow_p + d0) = k4;
          }
        }
      }
    }
  }  // pass
}

#ifndef ATTN_BWD_Q_WAVES
#define ATTN_BWD_Q_WAVES 8
#endif
#ifndef ATTN_BWD_KV_WAVES
#define ATTN_BWD_KV_WAVES 4
#endif
constexpr int kQWaves = ATTN_BWD_Q_WAVES;
constexpr int kKVWaves = ATTN_BWD_KV_WAVES;

// dQ of a split dQ pass: the sum of the S FP32 shares, one cast; four
// features per thread.
template <typename T>
__global__ __launch_bounds__(256) void dq_reduce_kernel(const float* __restrict__ part,
                                                        T* __restrict__ dq, int64_t n4,
                                                        int S) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const f32x4* src = reinterpret_cast<const f32x4*>(part) + i;
  f32x4 acc = src[0];
  for (int s = 1; s < S; ++s) acc += src[(int64_t)s * n4];
  T o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = from_f32<T>(acc[j]);
  u32x2 bits;
  __builtin_memcpy(&bits, o, sizeof(bits));
  reinterpret_cast<u32x2*>(dq)[i] = bits;
}

// Key splits of the dQ pass (1: no split).  Few 256-row query tiles over
// many keys cannot fill the GPU by rows (dQ of a chunk of rows over a long
// context), so their keys are split over about one eight-wave workgroup per
// CU, at least 16 key tiles each, when that puts fewer rows x keys on the
// busiest CU than the unsplit pass (four-wave workgroups of 128 rows, two
// tiles each when causal, up to 128 eight-wave workgroups).
struct DqSplit {
  int S = 1, kpt = 0;
};

DqSplit plan_dq_split(const BwdProblem& p) {
  DqSplit r;
  if (p.dtype == DType::F32 || p.Nq <= 0 || p.Nk <= 0) return r;
  const int64_t nqt = (p.Nq + 255) / 256;
  const int64_t wq = p.B * p.H * nqt;
  const int64_t kt = (p.Nk + kBT - 1) / kBT;
  if (wq > 64 || kt < 32) return r;
  int64_t S = (256 + wq - 1) / wq;
  if (S > kt / 16) S = kt / 16;
  if (S < 2) return r;
  const int64_t kpt = (kt + S - 1) / S;
  S = (kt + kpt - 1) / kpt;
  auto per_cu = [](int64_t w) { return (w + 255) / 256; };
  const int64_t bh = p.B * p.H;
  const int64_t w8 = bh * (p.causal ? (nqt + 1) / 2 : nqt);
  int64_t other;
  if (w8 <= 128) {
    const int64_t nqt4 = (p.Nq + 127) / 128;
    const bool pair = p.causal && nqt4 > 1;
    other = per_cu(bh * (p.causal ? (nqt4 + 1) / 2 : nqt4)) * (pair ? 256 : 128) * p.Nk;
  } else {
    other = per_cu(w8) * (p.causal && nqt > 1 ? 512 : 256) * p.Nk;
  }
  const int64_t mine = per_cu(wq * S) * 256 * kpt * kBT;
  if (mine >= other) return r;
  r.S = (int)S;
  r.kpt = (int)kpt;
  return r;
}

// Scratch: (lse2, Delta) per row, then (split dQ pass) the FP32 shares,
// 16-byte aligned.
int64_t stat_floats(const BwdProblem& p) { return (p.B * p.H * p.Nq * 2 + 3) / 4 * 4; }

void fill_grid(BwdArgs& a, int64_t heads, int ntile, bool causal, int64_t* grid) {
  a.ntile = ntile;
  a.nwork = causal ? (ntile + 1) / 2 : ntile;
  const int64_t total = heads * a.nwork;
  a.total = (int)total;
  *grid = (total + 7) / 8 * 8;
  a.per_xcd = (int)(*grid / 8);
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_typed(const BwdProblem& p, float* stat) {
  BwdArgs a{};
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.o = p.o;
  a.dout = p.dout;
  a.m = p.m;
  a.l = p.l;
  a.dq = p.dq;
  a.dk = p.dk;
  a.dv = p.dv;
  a.stat = stat;
  a.Nq = (int)p.Nq;
  a.Nk = (int)p.Nk;
  a.group = (int)(p.H / p.Hkv);
  a.c = p.scale * kLog2e;
  a.scale = p.scale;
  int64_t grid = 0;
  const DqSplit split = plan_dq_split(p);
  if (p.Nq > 0 && split.S > 1) {
    // Eight-wave workgroups of 256 rows, (head, query tile, split).
    a.dq_part = stat + stat_floats(p);
    a.S = split.S;
    a.kpt = split.kpt;
    a.rows = p.B * p.H * p.Nq;
    fill_grid(a, p.B * p.H, (int)((p.Nq + 255) / 256), false, &grid);
    a.nwork = a.ntile * a.S;
    a.total = (int)(p.B * p.H * a.nwork);
    grid = ((int64_t)a.total + 7) / 8 * 8;
    a.per_xcd = (int)(grid / 8);
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, 8, CAUSAL, true>), dim3((unsigned)grid), dim3(8 * 64),
                       0, p.stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n4 = a.rows * D / 4;
    hipLaunchKernelGGL((dq_reduce_kernel<T>), dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0,
                       p.stream, a.dq_part, static_cast<T*>(p.dq), n4, a.S);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else if (p.Nq > 0) {
    constexpr int BM = 32 * kQWaves;
    fill_grid(a, p.B * p.H, (int)((p.Nq + BM - 1) / BM), CAUSAL, &grid);
    if (a.total <= 128) {
      // A dQ grid that would fill at most half the CUs takes four-wave
      // workgroups (128 rows), twice as many: B1 H8 N4096 D128 causal 267
      // -> 222 us per backward, B1 H4 N8192 causal 478 -> 397 us; with 256
      // or more eight-wave workgroups the two are level.
      fill_grid(a, p.B * p.H, (int)((p.Nq + 127) / 128), CAUSAL, &grid);
      hipLaunchKernelGGL((bwd_dq_kernel<T, D, 4, CAUSAL, false>), dim3((unsigned)grid),
                         dim3(4 * 64), 0, p.stream, a);
    } else {
      hipLaunchKernelGGL((bwd_dq_kernel<T, D, kQWaves, CAUSAL, false>), dim3((unsigned)grid),
                         dim3(kQWaves * 64), 0, p.stream, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.Nk > 0) {
    constexpr int BK = 32 * kKVWaves;
    fill_grid(a, p.B * p.Hkv, (int)((p.Nk + BK - 1) / BK), CAUSAL, &grid);
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, kKVWaves, CAUSAL>), dim3((unsigned)grid),
                       dim3(kKVWaves * 64), 0, p.stream, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <typename T, int D>
hipError_t launch_d(const BwdProblem& p, float* stat) {
  return p.causal ? launch_typed<T, D, true>(p, stat) : launch_typed<T, D, false>(p, stat);
}

template <typename T>
hipError_t launch_t(const BwdProblem& p, float* stat) {
  switch (p.D) {
    case 16: return launch_d<T, 16>(p, stat);
    case 32: return launch_d<T, 32>(p, stat);
    case 64: return launch_d<T, 64>(p, stat);
    case 128: return launch_d<T, 128>(p, stat);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t bwd_scratch_bytes(const BwdProblem& p) {
  const DqSplit split = plan_dq_split(p);
  if (split.S < 2) return (size_t)(p.B * p.H * p.Nq) * 8;
  return (size_t)(stat_floats(p) + (int64_t)split.S * p.B * p.H * p.Nq * p.D) * sizeof(float);
}

hipError_t launch_bwd_mfma(const BwdProblem& p, float* scratch) {
  if (p.dtype == DType::BF16) return launch_t<__bf16>(p, scratch);
  if (p.dtype == DType::F16) return launch_t<_Float16>(p, scratch);
  return hipErrorInvalidValue;
}

}  // namespace attn
