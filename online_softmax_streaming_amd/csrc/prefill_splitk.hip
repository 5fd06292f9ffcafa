// Streaming attention prefill for problems too small to fill the GPU
// (bf16 / f16, plain batched layout): the keys of each 32-row query block
// are split over the waves of one workgroup, and the waves' running states
// are merged in LDS at the end.
//
// Per wave the computation is prefill_mfma.hip's (workshops page, "Scope
// and contracts"; answer-key page, row A3): S = K Q^T and O += P V on the
// matrix cores, the online-softmax update with a lazily refreshed reference
// max, masks only on tiles that cross the diagonal or the ragged end.  Wave
// w of the KS waves streams key tiles w, w + KS, w + 2 KS, ... of the block
// through LDS tiles of its own, the next tile in flight while one is
// computed, so the waves never wait on each other until the end.  There the
// states (m, l, O) are combined with the merge of the answer-key page's row
// A1: each is rescaled by 2^(m_w - M) to the common reference M = max_w m_w,
// then summed.
//
// Up to D = 64 a wave double-buffers its K and V tiles in LDS (direct-to-LDS
// loads).  At D = 128 two such pairs per wave would leave room for only two
// waves, so a wave keeps one pair in LDS and the next tile in registers,
// written into the pair after the tile in it has been computed: four waves
// per workgroup instead of two.
//
// With B*H*Nq/32 workgroups of KS waves, a problem of a few heads keeps
// KS times more waves busy than one wave per row block would, and each
// wave's chain of dependent tile steps is KS times shorter.

#include <type_traits>

#include "attn_kernels.h"
#include "attn_mfma.h"

namespace attn {
namespace {

struct SplitArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* m_out;
  float* l_out;
  int Nq, Nk;
  int group;  // query heads per K/V head
  int nrb;    // 32-row query blocks per (b, h)
  int total;    // B * H * nrb workgroups of work
  int per_xcd;  // gridDim.x / 8 when workgroups are regrouped by XCD, else 0
  float c;    // scale * log2(e)
};

constexpr int kBN = 64;              // keys per tile
constexpr int kKPF = 4;              // K fragments read ahead of their MFMA
constexpr int kVPF = 4;              // V^T operands read ahead of their MFMA
constexpr float kRefreshGap = 8.0f;  // base-2 units, as in prefill_mfma.hip

// Waves per workgroup, each with its own K and V tiles (64 * D * 2 bytes
// each) in LDS: two pairs per wave up to D = 64, one pair and the next tile
// in registers at D = 128.
constexpr int kSplits = 4;
template <int D>
constexpr bool kRegStage = D > 64;

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kSplits * 64) void prefill_splitk_kernel(SplitArgs a) {
  typedef typename Mfma<T>::vec8 vec8;
  typedef typename Mfma<T>::vec4 vec4;
  typedef typename Mfma<T>::vec2 vec2;
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  typedef Geo<D> G;
  constexpr int KS = kSplits;
  constexpr bool STAGE = kRegStage<D>;
  constexpr int BN = kBN;
  constexpr int DP = D < 32 ? 32 : D;  // O^T rows, padded to one MFMA block
  constexpr int KC = D / 16;           // k-chunks of Q.K^T
  constexpr int NB = DP / 32;          // 32-row blocks of O^T
  constexpr int TILE = BN * D * 2;     // bytes of one K or V tile
  constexpr int NSLOT = TILE / 16;     // 16-byte slots per tile
  constexpr int NU = NSLOT / 64;       // 1 KB LDS blocks per tile
  constexpr int NREG = 16 * NB;        // O^T registers per lane
  static_assert(G::steps_keep_swizzle(), "tile steps must keep the LDS swizzle");
  static_assert(NSLOT % 64 == 0, "a wave moves whole 1 KB LDS blocks");

  // Buffer parity 0 and 1 as separate objects, so the compiler can tell a
  // tile being loaded from the one being read; [wave][K or V] tiles.  The
  // states of waves 1..KS-1 for the merge, [wave - 1][register][lane], have
  // their own array, or (register staging, one pair per wave) take buf0's
  // place once every tile has been read.
  constexpr int kPairs = KS * 2 * TILE;
  constexpr int kMergeFloats = (KS - 1) * (NREG + 3) * 64;
  constexpr int kBuf0 = STAGE && kMergeFloats * 4 > kPairs ? kMergeFloats * 4 : kPairs;
  __shared__ __attribute__((aligned(1024))) unsigned char buf0[kBuf0];
  __shared__ __attribute__((aligned(1024))) unsigned char buf1[STAGE ? 16 : kPairs];
  __shared__ float mrg_own[STAGE ? 1 : kMergeFloats];
  float* const mrg = STAGE ? reinterpret_cast<float*>(buf0) : mrg_own;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  auto tile_ptr = [&](int buf, int kv) __attribute__((always_inline)) -> unsigned char* {
    return buf == 0 ? &buf0[(wave * 2 + kv) * TILE] : &buf1[(wave * 2 + kv) * TILE];
  };

  // Consecutive workgroup ids land on different XCDs (round-robin over 8).
  // When the problem's K/V outgrow one XCD's L2 (4 MB), the ids are
  // regrouped so each XCD takes a contiguous range of heads: the row blocks
  // of a head then read its K/V tiles through one L2, about together,
  // instead of every XCD fetching every head's K/V (B1 H32 Nq256 Nk16384
  // D128 causal: 322 -> 124 us; B4 H8 Nq256 Nk4096: 81 -> 37 us).
  const int bid = blockIdx.x;
  const int logical = a.per_xcd ? (bid & 7) * a.per_xcd + (bid >> 3) : bid;
  if (logical >= a.total) return;
  const int bh = logical / a.nrb;
  const int rb = logical - bh * a.nrb;
  const int Nq = a.Nq, Nk = a.Nk;
  const int off = Nk - Nq;
  const int64_t qbase = (int64_t)bh * Nq * D;
  const int64_t kbase = (int64_t)(bh / a.group) * Nk * D;
  const T* __restrict__ Qh = static_cast<const T*>(a.q) + qbase;
  const T* Kh = static_cast<const T*>(a.k) + kbase;
  const T* Vh = static_cast<const T*>(a.v) + kbase;
  T* __restrict__ Oh = static_cast<T*>(a.o) + qbase;

  const int h32 = lane >> 5;
  const int l32 = lane & 31;
  const int qw0 = rb * 32;
  const int qrow = qw0 + l32;
  const float c = a.c;

  vec8 qf[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    qf[kc] = qrow < Nq ? *reinterpret_cast<const vec8*>(Qh + (int64_t)qrow * D + kc * 16 + h32 * 8)
                       : vec8{};
  }

  // Key tiles holding a key that some row of the block may see.
  int kend = Nk;
  if (CAUSAL) kend = min(Nk, min(qw0 + 32, Nq) + off);
  const int ntiles = kend > 0 ? (kend + BN - 1) / BN : 0;

  const uint32_t kpitch = (uint32_t)(2 * D);
  const uint32_t kv_bytes = (uint32_t)Nk * (uint32_t)(2 * D);
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(Kh), 0, (int)kv_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(Vh), 0, (int)kv_bytes, 0x00020000);

  int koff[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) koff[kc] = G::off(l32, 2 * kc + h32);
  int voff[NB][2];
  {
    const int i = lane & 15;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int row = 8 * half + 4 * h32 + (i >> 2);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        int col = 16 * ((lane >> 4) & 1) + 32 * nb + 4 * (i & 3);
        if (col >= D) col -= D;
        voff[nb][half] = G::off(row, col >> 3) + ((col & 7) << 1);
      }
    }
  }

  float m_run = kNegInf;   // reference max, base-2 units
  float m_true = kNegInf;  // exact running max, base-2 units
  float l_run = 0.f;       // this half-wave's share of the running sum
  f32x16 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x16{};

  // Slot s of a tile (lane l of 1 KB block u holds slot l + 64u) is chunk
  // (s % CPR) ^ swz(row) of row s / CPR; rows past Nk are out of the buffer
  // range and arrive as zeros.
  auto slot_off = [&](int t, int u) __attribute__((always_inline)) {
    const int sl = lane + u * 64;
    const int row = sl / G::CPR;
    const int chunk = (sl % G::CPR) ^ G::swz(row);
    const int j = min(t * BN + row, Nk);
    return (int)((uint32_t)j * kpitch + (uint32_t)(chunk << 4));
  };
  // Tile t straight into buffer buf.
  auto load_tile = [&](int t, auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int vo = slot_off(t, u);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, LDS_PTR(void, tile_ptr(buf, 0) + u * 1024), 16,
                                               vo, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, LDS_PTR(void, tile_ptr(buf, 1) + u * 1024), 16,
                                               vo, 0, 0, 0);
    }
  };
  // Register staging: tile t into registers, and from there into buffer 0
  // in the same layout.
  u32x4 kst[STAGE ? NU : 1], vst[STAGE ? NU : 1];
  auto stage_tile = [&](int t) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int vo = slot_off(t, u);
      kst[u] = __builtin_amdgcn_raw_buffer_load_b128(krs, vo, 0, 0);
      vst[u] = __builtin_amdgcn_raw_buffer_load_b128(vrs, vo, 0, 0);
    }
  };
  auto unstage_tile = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      *reinterpret_cast<u32x4*>(tile_ptr(0, 0) + u * 1024 + lane * 16) = kst[u];
      *reinterpret_cast<u32x4*>(tile_ptr(0, 1) + u * 1024 + lane * 16) = vst[u];
    }
  };

  auto compute = [&](auto bufc, int j0) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    const unsigned char* kt = tile_ptr(buf, 0);
    const unsigned char* vt = tile_ptr(buf, 1);
    constexpr int NS = (BN / 32) * KC;
    vec8 kf[NS];
    auto kread = [&](int i) {
      return *reinterpret_cast<const vec8*>(kt + koff[i % KC] + (i / KC) * 32 * 2 * D);
    };
#pragma unroll
    for (int i = 0; i < kKPF && i < NS; ++i) kf[i] = kread(i);
    f32x16 s[BN / 32];
#pragma unroll
    for (int mb = 0; mb < BN / 32; ++mb) s[mb] = f32x16{};
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if (i + kKPF < NS) kf[i + kKPF] = kread(i + kKPF);
      s[i / KC] = Mfma<T>::mma(kf[i], qf[i % KC], s[i / KC]);
    }
    __builtin_amdgcn_sched_barrier(0);

    constexpr int NV = NB * (BN / 16);
    vec8 vf[NV];
    auto vread = [&](int i) {
      const int nb = i / (BN / 16), c2 = i % (BN / 16);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          LDS_PTR(s16x4, vt + voff[nb][0] + 16 * c2 * 2 * D));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          LDS_PTR(s16x4, vt + voff[nb][1] + 16 * c2 * 2 * D));
      return __builtin_bit_cast(vec8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
#pragma unroll
    for (int i = 0; i < kVPF && i < NV; ++i) vf[i] = vread(i);
    __builtin_amdgcn_sched_barrier(0);

    if ((j0 + BN > Nk) || (CAUSAL && j0 + BN - 1 > qw0 + off)) {
      // Register r of block mb holds key j0 + 4*h32 + kr, kr = 32mb + 8(r/4) + r%4.
      const int lim = min(Nk - j0, CAUSAL ? qrow + off - j0 + 1 : Nk - j0) - 4 * h32;
#pragma unroll
      for (int mb = 0; mb < BN / 32; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kr = mb * 32 + (r >> 2) * 8 + (r & 3);
          s[mb][r] = kr < lim ? s[mb][r] : kNegInf;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int mb = 0; mb < BN / 32; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
    mx = half_max(mx);
    const float m_tile = mx * c;
    m_true = fmaxf(m_true, m_tile);
    const bool refresh = m_tile > m_run + kRefreshGap;
    if (__builtin_amdgcn_ballot_w64(refresh)) {
      const float m_new = refresh ? m_tile : m_run;
      const float alpha = exp2_hw(m_run - pinned_ref(m_new));
      l_run *= alpha;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] *= alpha;
      m_run = m_new;
    }
    const float ref = pinned_ref(m_run);
#pragma unroll
    for (int mb = 0; mb < BN / 32; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[mb][r] = exp2_hw(__builtin_fmaf(s[mb][r], c, -ref));
    vec8 pf[BN / 16];
    float rs = 0.f;
#pragma unroll
    for (int c2 = 0; c2 < BN / 16; ++c2) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[c2][e] = from_f32<T>(s[c2 >> 1][(c2 & 1) * 8 + e]);
#pragma unroll
      for (int e = 0; e < 4; ++e) rs = Mfma<T>::sum2(vec2{pf[c2][2 * e], pf[c2][2 * e + 1]}, rs);
    }
    l_run += rs;

    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if (i + kVPF < NV) vf[i + kVPF] = vread(i + kVPF);
      acc[i / (BN / 16)] = Mfma<T>::mma(vf[i], pf[i % (BN / 16)], acc[i / (BN / 16)]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // This wave's tiles: wave, wave + KS, ...; the next one is in flight while
  // the current one is computed.
  constexpr int kWaitLoads = 0x0F70;  // s_waitcnt vmcnt(0) (expcnt, lgkmcnt untouched)
  if (qw0 < Nq && wave < ntiles) {
    load_tile(wave, std::integral_constant<int, 0>{});
    if constexpr (STAGE) {
      // The pair is rewritten from the registers only after the tile in it
      // has been computed (a wave's LDS accesses complete in order), and the
      // registers are reloaded only after that write.
      if (wave + KS < ntiles) stage_tile(wave + KS);
      __builtin_amdgcn_s_waitcnt(kWaitLoads);
      for (int t = wave;;) {
        compute(std::integral_constant<int, 0>{}, t * BN);
        t += KS;
        if (t >= ntiles) break;
        unstage_tile();
        if (t + KS < ntiles) stage_tile(t + KS);
      }
    } else {
      // Reads of a buffer finish (their values feed the products) before the
      // same wave reloads it two tiles later.  Each step ends by waiting for
      // its own loads, so a step's reads never wait on the tile it just put
      // in flight.
      __builtin_amdgcn_s_waitcnt(kWaitLoads);
      for (int t = wave; t < ntiles; t += 2 * KS) {
        if (t + KS < ntiles) load_tile(t + KS, std::integral_constant<int, 1>{});
        compute(std::integral_constant<int, 0>{}, t * BN);
        __builtin_amdgcn_s_waitcnt(kWaitLoads);
        if (t + KS < ntiles) {
          if (t + 2 * KS < ntiles) load_tile(t + 2 * KS, std::integral_constant<int, 0>{});
          compute(std::integral_constant<int, 1>{}, (t + KS) * BN);
          __builtin_amdgcn_s_waitcnt(kWaitLoads);
        }
      }
    }
  }

  // Merge (answer-key row A1): waves 1..KS-1 leave their states in LDS,
  // wave 0 rescales every state to the common reference and sums.
  const float l_tot = half_sum(l_run);
  if constexpr (STAGE) __syncthreads();  // the states go where the tiles were
  if (wave > 0) {
    float* dst = mrg + (wave - 1) * (NREG + 3) * 64;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[(nb * 16 + r) * 64 + lane] = acc[nb][r];
    dst[NREG * 64 + lane] = m_run;
    dst[(NREG + 1) * 64 + lane] = l_tot;
    dst[(NREG + 2) * 64 + lane] = m_true;
  }
  __syncthreads();
  if (wave != 0) return;

  float M = m_run;
#pragma unroll
  for (int w = 1; w < KS; ++w) M = fmaxf(M, mrg[((w - 1) * (NREG + 3) + NREG) * 64 + lane]);
  const float ref = pinned_ref(M);
  const float w0 = exp2_hw(m_run - ref);  // 0 for an empty state
  float L = l_tot * w0;
  float mt = m_true;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] *= w0;
#pragma unroll
  for (int w = 1; w < KS; ++w) {
    const float* src = mrg + (w - 1) * (NREG + 3) * 64;
    const float ws = exp2_hw(src[NREG * 64 + lane] - ref);
    L = __builtin_fmaf(src[(NREG + 1) * 64 + lane], ws, L);
    mt = fmaxf(mt, src[(NREG + 2) * 64 + lane]);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nb][r] = __builtin_fmaf(src[(nb * 16 + r) * 64 + lane], ws, acc[nb][r]);
  }

  // Epilogue: normalise, one cast, store; row state relative to the exact max.
  if (qrow < Nq) {
    const float inv = L > 0.f ? 1.f / L : 0.f;
    T* orow = Oh + (int64_t)qrow * D;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = nb * 32 + g * 8 + h32 * 4;
        if (d0 < D) {
          vec4 o4;
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = from_f32<T>(acc[nb][g * 4 + e] * inv);
          *reinterpret_cast<vec4*>(orow + d0) = o4;
        }
      }
    }
    if (h32 == 0) {
      const int64_t row = (int64_t)bh * Nq + qrow;
      const float to_true = mt == kNegInf ? 0.f : exp2_hw(ref - mt);
      if (a.m_out) a.m_out[row] = mt * kLn2;
      if (a.l_out) a.l_out[row] = L * to_true;
    }
  }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_typed(const Problem& p) {
  SplitArgs a;
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.o = p.o;
  a.m_out = p.m_out;
  a.l_out = p.l_out;
  a.Nq = (int)p.Nq;
  a.Nk = (int)p.Nk;
  a.group = (int)(p.H / p.Hkv);
  a.nrb = (int)((p.Nq + 31) / 32);
  a.c = p.scale * kLog2e;
  const int64_t total = p.B * p.H * a.nrb;
  const bool regroup = p.B * p.Hkv * p.Nk * p.D * 4 > ((int64_t)4 << 20);  // K and V bytes
  const int64_t grid = regroup ? (total + 7) / 8 * 8 : total;
  a.total = (int)total;
  a.per_xcd = regroup ? (int)(grid / 8) : 0;
  hipLaunchKernelGGL((prefill_splitk_kernel<T, D, CAUSAL>), dim3((unsigned)grid),
                     dim3(kSplits * 64), 0, p.stream, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const Problem& p) {
  switch (p.D) {
    case 16: return p.causal ? launch_typed<T, 16, true>(p) : launch_typed<T, 16, false>(p);
    case 32: return p.causal ? launch_typed<T, 32, true>(p) : launch_typed<T, 32, false>(p);
    case 64: return p.causal ? launch_typed<T, 64, true>(p) : launch_typed<T, 64, false>(p);
    case 128: return p.causal ? launch_typed<T, 128, true>(p) : launch_typed<T, 128, false>(p);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefill_splitk(const Problem& p) {
  if (p.dtype == DType::BF16) return launch_t<__bf16>(p);
  if (p.dtype == DType::F16) return launch_t<_Float16>(p);
  return hipErrorInvalidValue;
}

}  // namespace attn
