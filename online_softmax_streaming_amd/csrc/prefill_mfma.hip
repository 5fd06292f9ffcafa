// Streaming attention prefill on gfx950 matrix cores (bf16 / f16 inputs).
//
// What is computed is the streaming_attention contract of the workshops page
// ("Intermediate and advanced kernel workshops", section "Scope and
// contracts"), batched over (B, H): each query row carries a running max m,
// running sum l and unnormalised output a across key tiles, rescaling l and
// a together when m rises (answer-key page, row A3), and one score tile is
// alive at a time.  Masked or padded scores are -inf before the max and add
// 0 to the sums, and rows with nothing visible are pinned at reference 0
// ("Kernel Notes & Checklist", gotchas ledger).
//
// Work decomposition (one workgroup = NW waves = 32*NW query rows):
//   * Each wave owns 32 query rows.  Its Q rows stay in registers for the
//     whole kernel as the B operand of v_mfma_f32_32x32x16_{bf16,f16}.
//   * Key tiles of BN = 64 rows are staged in LDS, double-buffered: K
//     row-major, V transposed (V^T[d][key]) so the P.V product can read its
//     key-contiguous operand with one 16-byte LDS read.
//   * S^T = K Q^T is formed per 32-key block, so each lane owns one query
//     column: the row max/sum over keys is in-lane plus one exchange between
//     the two half-waves.  P^T stays in registers as the B operand of
//     O^T += V^T P^T, again with one query per lane, so the rescale by
//     alpha is a per-lane scalar.
//   * Causal: a query tile visits only key tiles that hold a visible key
//     (the pages' answer visits every tile); inside a tile a wave whose rows
//     see none of its keys skips the math, and masks are applied only on
//     tiles that cross the diagonal or the ragged end.
//
// MFMA 32x32x16 register layout used here (per lane l, h = l / 32):
//   A: 8 consecutive k of row l % 32;  B: the same 8 k of column l % 32;
//   C: column l % 32, register r holds row 8*(r/4) + 4*h + (r%4).
// A and B use the same k slots, so the contraction needs no assumption
// about which k-slot the hardware gives each half-wave; only the C layout
// is relied on, and any other C layout fails the parity tests.

#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {
namespace {

template <typename T> struct Mfma;
template <> struct Mfma<__bf16> {
  typedef bf16x8 vec8;
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
  typedef _Float16 vec2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ f32x16 mma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float sum2(vec2 x, float acc) {
    const vec2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(x, one, acc, false);
  }
};

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* m_out;
  float* l_out;
  int Nq, Nk;
  int nqt;      // query tiles per (b, h)
  int total;    // (B*H) * nqt real workgroups
  int per_xcd;  // gridDim.x / 8
  float c;      // scale * log2(e)
};

constexpr int kBN = 64;  // keys per tile

template <typename T, int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void prefill_mfma_kernel(PrefillArgs a) {
  typedef typename Mfma<T>::vec8 vec8;
  constexpr int NT = NW * 64;
  constexpr int BM = 32 * NW;
  constexpr int BN = kBN;
  constexpr int DP = D < 32 ? 32 : D;   // O^T rows, padded to one MFMA block
  constexpr int KC = D / 16;            // k-chunks of Q.K^T
  constexpr int NB = DP / 32;           // 32-row blocks of O^T
  constexpr int KSTR = D + 8;           // LDS row stride of K (elements)
  constexpr int VSTR = BN + 8;          // LDS row stride of V^T (elements)
  constexpr int DV = D / 8;             // 16-byte chunks per row
  constexpr int KCHUNKS = BN * DV;      // 16-byte chunks per K tile
  constexpr int KPT = (KCHUNKS + NT - 1) / NT;
  constexpr int VBLK = (BN / 4) * DV;   // 4-key x 8-column blocks per V tile
  constexpr int VPT = (VBLK + NT - 1) / NT;

  __shared__ __attribute__((aligned(16))) T Ks[2][BN * KSTR];
  __shared__ __attribute__((aligned(16))) T Vt[2][DP * VSTR];

  // Workgroup -> (head, query tile).  Consecutive workgroup ids land on
  // different XCDs (round-robin over 8); regroup them so each XCD walks a
  // contiguous range of heads and their K/V stays in that XCD's L2.  Within
  // a head, causal tiles go longest-first.
  const int bid = blockIdx.x;
  const int logical = (bid & 7) * a.per_xcd + (bid >> 3);
  if (logical >= a.total) return;
  const int bh = logical / a.nqt;
  const int rr = logical - bh * a.nqt;
  const int qt = CAUSAL ? (a.nqt - 1 - rr) : rr;

  const int Nq = a.Nq, Nk = a.Nk, off = Nk - Nq;
  const T* __restrict__ Qh = static_cast<const T*>(a.q) + (int64_t)bh * Nq * D;
  const T* __restrict__ Kh = static_cast<const T*>(a.k) + (int64_t)bh * Nk * D;
  const T* __restrict__ Vh = static_cast<const T*>(a.v) + (int64_t)bh * Nk * D;
  T* __restrict__ Oh = static_cast<T*>(a.o) + (int64_t)bh * Nq * D;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h32 = lane >> 5;
  const int l32 = lane & 31;
  const int i0 = qt * BM;
  const int qw0 = i0 + wave * 32;  // first query row of this wave
  const int qrow = qw0 + l32;      // this lane's query row
  const float c = a.c;

  // Q fragment: B operand, 8 consecutive features per k-chunk.  Rows past
  // Nq (ghost rows) are zero so their scores stay finite; never stored.
  vec8 qf[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    if (qrow < Nq) {
      qf[kc] = *reinterpret_cast<const vec8*>(Qh + (int64_t)qrow * D + kc * 16 + h32 * 8);
    } else {
      qf[kc] = vec8{};
    }
  }

  // Key range that holds a visible key for some real row of this tile.
  int kend = Nk;
  if (CAUSAL) kend = min(Nk, min(i0 + BM, Nq) + off);
  const int ntiles = kend > 0 ? (kend + BN - 1) / BN : 0;

  float m_run = kNegInf;  // running max, base-2 units
  float l_run = 0.f;      // this half-wave's share of the running sum
  f32x16 acc[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) acc[n] = f32x16{};

  if (D < 32) {
    // O^T rows D..31 are computed from these V^T rows and then discarded;
    // zero them once so they hold no stale LDS contents.
    for (int e = tid; e < 2 * (DP - D) * VSTR; e += NT) {
      const int b = e / ((DP - D) * VSTR);
      const int r = e - b * (DP - D) * VSTR;
      Vt[b][D * VSTR + r] = T(0.f);
    }
  }

  vec8 kreg[KPT];
  vec8 vreg[VPT][4];

  auto load_tile = [&](int j0) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int ch = tid + u * NT;
      if (KCHUNKS % NT == 0 || ch < KCHUNKS) {
        const int row = ch / DV, col = ch - row * DV;
        const int j = j0 + row;
        kreg[u] = j < Nk ? *reinterpret_cast<const vec8*>(Kh + (int64_t)j * D + col * 8) : vec8{};
      }
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int b = tid + u * NT;
      if (VBLK % NT == 0 || b < VBLK) {
        const int kq = b / DV, dc = b - kq * DV;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = j0 + kq * 4 + i;
          vreg[u][i] = j < Nk ? *reinterpret_cast<const vec8*>(Vh + (int64_t)j * D + dc * 8) : vec8{};
        }
      }
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int ch = tid + u * NT;
      if (KCHUNKS % NT == 0 || ch < KCHUNKS) {
        const int row = ch / DV, col = ch - row * DV;
        *reinterpret_cast<vec8*>(&Ks[buf][row * KSTR + col * 8]) = kreg[u];
      }
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int b = tid + u * NT;
      if (VBLK % NT == 0 || b < VBLK) {
        const int kq = b / DV, dc = b - kq * DV;
        // Keys 4kq..4kq+3 go to 4 adjacent V^T columns.  Within each group
        // of 16 keys, key 8a + 4b + c sits at column 8b + 4a + c: then the
        // 8 keys one lane feeds to one P.V MFMA (see compute) are adjacent.
        const int pos = (kq >> 2) * 16 + (kq & 1) * 8 + ((kq >> 1) & 1) * 4;
        const u32x4 r0 = __builtin_bit_cast(u32x4, vreg[u][0]);
        const u32x4 r1 = __builtin_bit_cast(u32x4, vreg[u][1]);
        const u32x4 r2 = __builtin_bit_cast(u32x4, vreg[u][2]);
        const u32x4 r3 = __builtin_bit_cast(u32x4, vreg[u][3]);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // Feature 2w: low halves; feature 2w+1: high halves.
          u32x2 lo, hi;
          lo.x = __builtin_amdgcn_perm(r1[w], r0[w], 0x05040100u);
          lo.y = __builtin_amdgcn_perm(r3[w], r2[w], 0x05040100u);
          hi.x = __builtin_amdgcn_perm(r1[w], r0[w], 0x07060302u);
          hi.y = __builtin_amdgcn_perm(r3[w], r2[w], 0x07060302u);
          *reinterpret_cast<u32x2*>(&Vt[buf][(dc * 8 + 2 * w) * VSTR + pos]) = lo;
          *reinterpret_cast<u32x2*>(&Vt[buf][(dc * 8 + 2 * w + 1) * VSTR + pos]) = hi;
        }
      }
    }
  };

  auto compute = [&](int buf, int j0, bool need_mask) {
    const T* ks = Ks[buf];
    const T* vt = Vt[buf];
    // S^T = K Q^T for two 32-key blocks.
    f32x16 s[BN / 32];
#pragma unroll
    for (int mb = 0; mb < BN / 32; ++mb) {
      s[mb] = f32x16{};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const vec8 ka = *reinterpret_cast<const vec8*>(ks + (mb * 32 + l32) * KSTR + kc * 16 + h32 * 8);
        s[mb] = Mfma<T>::mma(ka, qf[kc], s[mb]);
      }
    }
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
    // Row max over this tile: in-lane, then across the two half-waves.
    float mx = s[0][0];
#pragma unroll
    for (int mb = 0; mb < BN / 32; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * c);
    const float ref = pinned_ref(m_new);
    const float alpha = exp2_hw(m_run - ref);
#pragma unroll
    for (int mb = 0; mb < BN / 32; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[mb][r] = exp2_hw(__builtin_fmaf(s[mb][r], c, -ref));

    // P^T rounded to the input type: the B operand of O^T += V^T P^T.  The
    // row sum adds the same rounded weights, so the normalisation matches
    // the numerator exactly (one visible key gives weight 1 and out = V).
    typedef typename Mfma<T>::vec2 vec2;
    vec8 pf[BN / 16];
    float rs = 0.f;
#pragma unroll
    for (int c2 = 0; c2 < BN / 16; ++c2) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[c2][e] = from_f32<T>(s[c2 >> 1][(c2 & 1) * 8 + e]);
#pragma unroll
      for (int e = 0; e < 4; ++e) rs = Mfma<T>::sum2(vec2{pf[c2][2 * e], pf[c2][2 * e + 1]}, rs);
    }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[n] *= alpha;
    m_run = m_new;
#pragma unroll
    for (int n = 0; n < NB; ++n) {
#pragma unroll
      for (int c2 = 0; c2 < BN / 16; ++c2) {
        const vec8 va = *reinterpret_cast<const vec8*>(vt + (n * 32 + l32) * VSTR + c2 * 16 + h32 * 8);
        acc[n] = Mfma<T>::mma(va, pf[c2], acc[n]);
      }
    }
  };

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
    __syncthreads();
    const int q_last = min(qw0 + 32, Nq) - 1;  // last real row of this wave
    for (int t = 0; t < ntiles; ++t) {
      const int j0 = t * BN;
      const bool more = t + 1 < ntiles;
      if (more) load_tile(j0 + BN);
      const bool active = qw0 < Nq && (!CAUSAL || j0 <= q_last + off);
      if (active) {
        const bool need_mask = (j0 + BN > Nk) || (CAUSAL && j0 + BN - 1 > qw0 + off);
        compute(t & 1, j0, need_mask);
      }
      if (more) store_tile((t + 1) & 1);
      __syncthreads();
    }
  }

  // Epilogue: join the two half-wave sums, normalise, one cast, store.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qrow < Nq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    T* orow = Oh + (int64_t)qrow * D;
#pragma unroll
    for (int n = 0; n < NB; ++n) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = n * 32 + g * 8 + h32 * 4;
        if (d0 < D) {
          typedef T t4 __attribute__((ext_vector_type(4)));
          t4 o4;
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = from_f32<T>(acc[n][g * 4 + e] * inv);
          *reinterpret_cast<t4*>(orow + d0) = o4;
        }
      }
    }
    if (h32 == 0) {
      const int64_t row = (int64_t)bh * Nq + qrow;
      if (a.m_out) a.m_out[row] = m_run * kLn2;
      if (a.l_out) a.l_out[row] = l_tot;
    }
  }
}

template <typename T, int D, int NW, bool CAUSAL>
hipError_t launch_typed(const Problem& p) {
  constexpr int BM = 32 * NW;
  PrefillArgs a;
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.o = p.o;
  a.m_out = p.m_out;
  a.l_out = p.l_out;
  a.Nq = (int)p.Nq;
  a.Nk = (int)p.Nk;
  a.nqt = (int)((p.Nq + BM - 1) / BM);
  const int64_t total = p.B * p.H * a.nqt;
  a.total = (int)total;
  const int64_t grid = (total + 7) / 8 * 8;
  a.per_xcd = (int)(grid / 8);
  a.c = p.scale * kLog2e;
  hipLaunchKernelGGL((prefill_mfma_kernel<T, D, NW, CAUSAL>), dim3((unsigned)grid), dim3(NW * 64),
                     0, p.stream, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const Problem& p) {
  return p.causal ? launch_typed<T, D, 4, true>(p) : launch_typed<T, D, 4, false>(p);
}

template <typename T>
hipError_t launch_t(const Problem& p) {
  switch (p.D) {
    case 16: return launch_d<T, 16>(p);
    case 32: return launch_d<T, 32>(p);
    case 64: return launch_d<T, 64>(p);
    case 128: return launch_d<T, 128>(p);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefill_mfma(const Problem& p) {
  if (p.dtype == DType::BF16) return launch_t<__bf16>(p);
  if (p.dtype == DType::F16) return launch_t<_Float16>(p);
  return hipErrorInvalidValue;
}

}  // namespace attn
