// Streaming attention prefill for FP32 inputs, on the vector ALUs.
//
// Same contract and running-state algorithm as the matrix-core kernel
// (workshops page, "Scope and contracts"; answer-key page, row A3), kept in
// FP32 end to end: P is not rounded before P.V because the input type is
// already FP32.  This path exists for FP32 accuracy (max abs error 1e-5
// against the FP64 oracle), not for throughput: gfx950 has no FP32 matrix
// instruction faster than its vector FMA path by enough to matter here.
//
// One workgroup = 128 threads = 128/TPQ query rows; a row's features are
// split over TPQ threads (by default TPQ = 2 for D = 128, so a thread keeps
// at most 64 features of q and 64 of the running output in registers; see
// kTpqWide and kThreadsWide for small problems).  Key tiles of 32 rows (16
// in the wide split up to D = 64) are staged in LDS and read by broadcast.

#include <climits>

#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {
namespace {

struct F32Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* m_out;
  float* l_out;
  int Nq, Nk;
  int nqt;
  int group;  // query heads per K/V head
  float c;  // scale * log2(e)
  // Packed variable-length sequences (VARLEN only), as in the matrix-core
  // kernel: Q/out [total_q, H, D], K/V [total_k, Hkv, D], states [H, total_q].
  const int* cu_q;
  const int* cu_k;
  int H, Hkv;
  int total_q, total_k;
  // Masked mode: optional bit-packed mask and sliding window, as in the
  // matrix-core kernel.
  const uint32_t* mask;
  int64_t mask_sb, mask_sh;
  int mask_words;
  int window;
  // Dropout mode, as in the matrix-core kernel.
  uint64_t seed, offset;
  uint32_t drop_t;
  float keep_gain;
  // Split-key mode (batched layout): workgroup (head, query tile, split s)
  // covers key tiles [s * kpt, (s + 1) * kpt) and writes each row's state,
  // base 2, l and a relative to the exact maximum m: a[D] to
  // part[row][s][.], (m, l) to part_ml[row][s][.].
  float* part;
  float* part_ml;
  int S, kpt;
};

enum : int { kModeBatched = 0, kModeVarlen = 1, kModeMasked = 2, kModeDropout = 3, kModeSplitKv = 4 };

constexpr int kThreads = 128;
constexpr int kBNF = 32;

// Threads per query row: the default keeps at most 64 features of q and of
// the running output per thread; the wide split (4 features per thread)
// serves problems too small to fill the GPU, trading a few lane exchanges
// per key for an eighth to a thirty-second of the serial work per thread.
// Its thread groups are one wave up to D = 64 (so the few rows of a small
// problem spread over more CUs, each SIMD running one wave) and two at
// D = 128.  Measured against 8 features per thread and 128-thread groups:
// B1 H1 N128 D64 9.4 -> 6.9 us, B1 H2 N512 D128 causal 51 -> 44 us.
template <int D>
constexpr int kTpqDefault = D > 64 ? 2 : 1;
template <int D>
constexpr int kTpqWide = D / 4;
template <int D>
constexpr int kThreadsWide = D > 64 ? 128 : 64;
// Key-split groups of the wide split and their key tiles: eight groups of
// 16-key tiles up to D = 64 (against four of 32 keys: B1 H1 N128 D64 causal
// 7.1 -> 6.2 us, B1 H1 N1024 causal 41 -> 27 us), two of 32 keys at D = 128,
// whose four-group workgroup would need more than 256 registers per thread
// in dropout mode.
template <int D>
constexpr int kKsfWide = D > 64 ? 2 : 8;
template <int D>
constexpr int kBnWide = D > 64 ? 32 : 16;

// KSF groups of NT threads split the key tiles of the workgroup's rows
// (group g takes tiles t_first + g, t_first + g + KSF, ...) and merge their
// states at the end (answer-key row A1); KSF = 1 streams every tile in one
// group.
template <int D, int TPQ, bool CAUSAL, int MODE, int KSF, int NT, int BN>
__global__ __launch_bounds__(NT * KSF) void prefill_f32_kernel(F32Args a) {
  constexpr bool VARLEN = MODE == kModeVarlen;
  constexpr bool MASKED = MODE == kModeMasked;
  constexpr bool DROPOUT = MODE == kModeDropout;
  constexpr bool SPLITKV = MODE == kModeSplitKv;
  constexpr int DT = D / TPQ;
  constexpr int QPB = NT / TPQ;

  __shared__ __attribute__((aligned(16))) float Ksm[KSF][BN * D];
  __shared__ __attribute__((aligned(16))) float Vsm[KSF][BN * D];

  const int nwork = SPLITKV ? a.nqt * a.S : a.nqt;
  const int bh = blockIdx.x / nwork;
  const int rr = blockIdx.x - bh * nwork;
  const int qt = SPLITKV ? rr / a.S : rr;
  const int sp = SPLITKV ? rr - qt * a.S : 0;
  int Nq = a.Nq, Nk = a.Nk;
  int64_t qbase, kbase, stat0, sq = D, sk = D;
  if (VARLEN) {
    // Sequence bounds clamped into the packed tensors (see prefill_mfma).
    const int b = bh / a.H, h = bh - b * a.H;
    const int q0 = min(max(a.cu_q[b], 0), a.total_q);
    const int q1 = min(max(a.cu_q[b + 1], q0), a.total_q);
    const int k0 = min(max(a.cu_k[b], 0), a.total_k);
    const int k1 = min(max(a.cu_k[b + 1], k0), a.total_k);
    Nq = q1 - q0;
    Nk = k1 - k0;
    if (qt * QPB >= Nq) return;
    sq = (int64_t)a.H * D;
    sk = (int64_t)a.Hkv * D;
    qbase = (int64_t)q0 * sq + (int64_t)h * D;
    kbase = (int64_t)k0 * sk + (int64_t)(h / a.group) * D;
    stat0 = (int64_t)h * a.total_q + q0;
  } else {
    qbase = (int64_t)bh * Nq * D;
    kbase = (int64_t)(bh / a.group) * Nk * D;  // K/V head bh / group
    stat0 = (int64_t)bh * Nq;
  }
  const int off = Nk - Nq;
  const float* __restrict__ Qh = a.q + qbase;
  const float* __restrict__ Kh = a.k + kbase;
  const float* __restrict__ Vh = a.v + kbase;
  float* __restrict__ Oh = a.o + qbase;

  const int tid = threadIdx.x % NT;
  const int grp = threadIdx.x / NT;
  float* __restrict__ Ks = Ksm[grp];
  float* __restrict__ Vs = Vsm[grp];
  const int part = tid % TPQ;
  const int i0 = qt * QPB;
  const int qrow = i0 + tid / TPQ;
  const float c = a.c;

  float q[DT], acc[DT];
#pragma unroll
  for (int d = 0; d < DT; ++d) {
    q[d] = qrow < Nq ? Qh[(int64_t)qrow * sq + part * DT + d] : 0.f;
    acc[d] = 0.f;
  }
  float m_run = kNegInf, l_run = 0.f;

  int kend = Nk;
  if (CAUSAL) kend = min(Nk, min(i0 + QPB, Nq) + off);
  const int nvis = kend > 0 ? (kend + BN - 1) / BN : 0;
  const int win = MASKED ? a.window : 0;
  const int t_first = SPLITKV ? sp * a.kpt : win > 0 ? max(0, i0 + off - win + 1) / BN : 0;
  const int ntiles = SPLITKV ? min(nvis, t_first + a.kpt) : nvis;
  const uint32_t* mrow = nullptr;
  if (MASKED && a.mask && qrow < Nq) {
    const int b = bh / a.H, h = bh - b * a.H;
    mrow = a.mask + (int64_t)b * a.mask_sb + (int64_t)h * a.mask_sh + (int64_t)qrow * a.mask_words;
  }

  for (int t0 = t_first; t0 < ntiles; t0 += KSF) {
    const int t = t0 + grp;
    const bool live = KSF == 1 || t < ntiles;  // this group has a tile in this round
    const int j0 = t * BN;
    // Stage the tile: 16-byte loads, rows past Nk zero.
#pragma unroll 4
    for (int e = tid; live && e < BN * D / 4; e += NT) {
      const int row = e / (D / 4), col = e - row * (D / 4);
      const int j = j0 + row;
      f32x4 kv = f32x4{}, vv = f32x4{};
      if (j < Nk) {
        kv = *reinterpret_cast<const f32x4*>(Kh + (int64_t)j * sk + col * 4);
        vv = *reinterpret_cast<const f32x4*>(Vh + (int64_t)j * sk + col * 4);
      }
      *reinterpret_cast<f32x4*>(&Ks[row * D + col * 4]) = kv;
      *reinterpret_cast<f32x4*>(&Vs[row * D + col * 4]) = vv;
    }
    __syncthreads();
    if (!live) {
      __syncthreads();
      continue;
    }

    // The row's mask bits for keys j0 .. j0+BN-1 from bit 0 on (all set
    // without a mask; a 16-key tile starts at bit 0 or 16 of its word) and
    // the window's lower limit (visible iff j > wlo), one compare per key.
    const int wlo = win > 0 ? qrow + off - win : INT_MIN;
    uint32_t mw = ~0u;
    if (MASKED && a.mask) mw = mrow && j0 / 32 < a.mask_words ? mrow[j0 / 32] >> (j0 & 31) : 0u;
    float s[BN];
    float mx = kNegInf;
#pragma unroll
    for (int jj = 0; jj < BN; ++jj) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < DT; ++d) dot = __builtin_fmaf(q[d], Ks[jj * D + part * DT + d], dot);
#pragma unroll
      for (int o = 1; o < TPQ; o <<= 1) dot += __shfl_xor(dot, o);  // the row's TPQ lanes
      const int j = j0 + jj;
      bool vis = j < Nk && (!CAUSAL || j <= qrow + off);
      if (MASKED) vis = vis && j > wlo && ((mw >> jj) & 1u);
      // Rounded product kept apart from the later subtraction, so the
      // largest score gives exactly 2^0 = 1.
      s[jj] = vis ? dot * c : kNegInf;
      mx = fmaxf(mx, s[jj]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float ref = pinned_ref(m_new);
    const float alpha = exp2_hw(m_run - ref);
    float rs = 0.f;
#pragma unroll
    for (int jj = 0; jj < BN; ++jj) {
      s[jj] = exp2_hw(s[jj] - ref);
      rs += s[jj];
    }
    l_run = l_run * alpha + rs;
    if (DROPOUT) {
      // Keys j0 .. j0+BN-1 are fields of Philox blocks j0/16, ... of this
      // row (counter (j / 16, i, bh, offset), key (seed, 0)).
#pragma unroll
      for (int blk = 0; blk < BN / 16; ++blk) {
        uint64_t w[4] = {(uint64_t)((j0 >> 4) + blk), (uint64_t)qrow, (uint64_t)bh, a.offset};
        philox4x64_10(w, a.seed, 0);
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const uint32_t field = (uint32_t)(w[t >> 2] >> (16 * (t & 3))) & 0xFFFFu;
          if (field < a.drop_t) s[16 * blk + t] = 0.f;
        }
      }
    }
#pragma unroll
    for (int d = 0; d < DT; ++d) {
      float x = acc[d] * alpha;
#pragma unroll
      for (int jj = 0; jj < BN; ++jj) x = __builtin_fmaf(s[jj], Vs[jj * D + part * DT + d], x);
      acc[d] = x;
    }
    m_run = m_new;
    __syncthreads();
  }

  if constexpr (KSF > 1) {
    // Merge (answer-key row A1): groups 1..KSF-1 leave (m, l, acc) in LDS;
    // group 0 rescales each state to the common reference and sums.
    __shared__ float mst[KSF - 1][DT + 2][NT];
    if (grp > 0) {
      mst[grp - 1][0][tid] = m_run;
      mst[grp - 1][1][tid] = l_run;
  #pragma unroll
      for (int d = 0; d < DT; ++d) mst[grp - 1][2 + d][tid] = acc[d];
    }
    __syncthreads();
    if (grp > 0) return;
    float M = m_run;
  #pragma unroll
    for (int g = 1; g < KSF; ++g) M = fmaxf(M, mst[g - 1][0][tid]);
    const float ref = pinned_ref(M);
    const float w0 = exp2_hw(m_run - ref);
    l_run *= w0;
  #pragma unroll
    for (int d = 0; d < DT; ++d) acc[d] *= w0;
  #pragma unroll
    for (int g = 1; g < KSF; ++g) {
      const float wg = exp2_hw(mst[g - 1][0][tid] - ref);
      l_run = __builtin_fmaf(mst[g - 1][1][tid], wg, l_run);
  #pragma unroll
      for (int d = 0; d < DT; ++d) acc[d] = __builtin_fmaf(mst[g - 1][2 + d][tid], wg, acc[d]);
    }
    m_run = M;
  }

  if (SPLITKV) {
    // The split's state (a = 0, l = 0, m = -inf for a row that sees no key
    // of the split).
    if (qrow < Nq) {
      const int64_t st = (stat0 + qrow) * a.S + sp;
#pragma unroll
      for (int d = 0; d < DT; ++d) a.part[st * D + part * DT + d] = acc[d];
      if (part == 0) {
        a.part_ml[2 * st] = m_run;
        a.part_ml[2 * st + 1] = l_run;
      }
    }
    return;
  }
  if (qrow < Nq) {
    float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    if (DROPOUT) inv *= a.keep_gain;
#pragma unroll
    for (int d = 0; d < DT; ++d) Oh[(int64_t)qrow * sq + part * DT + d] = acc[d] * inv;
    if (part == 0) {
      const int64_t row = stat0 + qrow;
      if (a.m_out) a.m_out[row] = m_run * kLn2;
      if (a.l_out) a.l_out[row] = l_run;
    }
  }
}

template <int D, int TPQ, bool CAUSAL, int MODE, int KSF, int NT, int BN>
hipError_t launch_typed(const Problem& p) {
  constexpr int QPB = NT / TPQ;
  F32Args a;
  a.q = static_cast<const float*>(p.q);
  a.k = static_cast<const float*>(p.k);
  a.v = static_cast<const float*>(p.v);
  a.o = static_cast<float*>(p.o);
  a.m_out = p.m_out;
  a.l_out = p.l_out;
  a.Nq = (int)p.Nq;
  a.Nk = (int)p.Nk;
  a.nqt = (int)((p.Nq + QPB - 1) / QPB);
  a.group = (int)(p.H / p.Hkv);
  a.c = p.scale * kLog2e;
  a.cu_q = p.cu_q;
  a.cu_k = p.cu_k;
  a.H = (int)p.H;
  a.Hkv = (int)p.Hkv;
  a.total_q = (int)p.total_q;
  a.total_k = (int)p.total_k;
  a.mask = p.mask;
  a.mask_sb = p.mask_sb;
  a.mask_sh = p.mask_sh;
  a.mask_words = (int)((p.Nk + 31) / 32);
  a.window = (int)p.window;
  a.seed = p.seed;
  a.offset = p.offset;
  a.drop_t = p.drop_t;
  a.keep_gain = (float)(65536.0 / (65536.0 - (double)p.drop_t));
  a.part = p.part;
  a.part_ml = p.part ? p.part + p.B * p.H * p.Nq * p.splits * D : nullptr;
  a.S = (int)p.splits;
  a.kpt = (int)p.split_tiles;
  const int64_t grid = p.B * p.H * a.nqt * (MODE == kModeSplitKv ? p.splits : 1);
  hipLaunchKernelGGL((prefill_f32_kernel<D, TPQ, CAUSAL, MODE, KSF, NT, BN>), dim3((unsigned)grid), dim3(NT * KSF), 0,
                     p.stream, a);
  return hipGetLastError();
}

template <int D, int TPQ, int KSF, int NT, int BN>
hipError_t launch_mode(const Problem& p) {
  if (p.cu_q)
    return p.causal ? launch_typed<D, TPQ, true, kModeVarlen, KSF, NT, BN>(p)
                    : launch_typed<D, TPQ, false, kModeVarlen, KSF, NT, BN>(p);
  if (p.mask || p.window > 0)
    return p.causal ? launch_typed<D, TPQ, true, kModeMasked, KSF, NT, BN>(p)
                    : launch_typed<D, TPQ, false, kModeMasked, KSF, NT, BN>(p);
  if (p.dropout)
    return p.causal ? launch_typed<D, TPQ, true, kModeDropout, KSF, NT, BN>(p)
                    : launch_typed<D, TPQ, false, kModeDropout, KSF, NT, BN>(p);
  return p.causal ? launch_typed<D, TPQ, true, kModeBatched, KSF, NT, BN>(p)
                  : launch_typed<D, TPQ, false, kModeBatched, KSF, NT, BN>(p);
}

template <int D>
hipError_t launch_d(const Problem& p) {
  // Fewer than 512 default workgroups (of two waves each, at most one wave
  // per SIMD): the wide split, with the key tiles shared out over kKsfWide
  // thread groups (against the default: B1 H8 N2048 D64 noncausal, 128
  // workgroups, 1118 -> 594 us; B1 H8 N4096 D64 causal, 256, 2179 -> 1254
  // us; B2 H4 N4096 D32 noncausal 1169 -> 897 us; at 512 and more the
  // default kernel wins).  The rule depends only on (B, H, Nq), so every
  // mode of one problem shape splits its rows the same way and computes
  // each row identically.
  constexpr int64_t qpb = kThreads / kTpqDefault<D>;
  if (p.B * p.H * ((p.Nq + qpb - 1) / qpb) < 512)
    return launch_mode<D, kTpqWide<D>, kKsfWide<D>, kThreadsWide<D>, kBnWide<D>>(p);
  return launch_mode<D, kTpqDefault<D>, 1, kThreads, kBNF>(p);
}

}  // namespace

#ifndef F32_SPLITKV
#define F32_SPLITKV 1
#endif

bool plan_prefill_f32_splitkv(const Problem& p, SplitKvPlan* plan) {
  // Batched FP32 problems of fewer than 512 default workgroups (the ones
  // that would take the wide split) over at least 32 key tiles of 32 keys:
  // the default kernel with each query tile's keys split over about four
  // two-wave workgroups per CU, 16 key tiles a split at least (against the
  // wide split: B1 H32 Nq512 Nk8192 D128 causal 7203 -> 1949 us, B1 H1
  // Nq512 Nk65536 D64 causal 1896 -> 313 us, B1 H8 N2048 D64 592 -> 303
  // us, B1 H2 N4096 D128 causal 970 -> 499 us).
  if (!F32_SPLITKV || p.cu_q) return false;
  const int64_t qpb = kThreads / (p.D > 64 ? 2 : 1);
  const int64_t wq = p.B * p.H * ((p.Nq + qpb - 1) / qpb);
  const int64_t kt = (p.Nk + kBNF - 1) / kBNF;
  if (wq >= 512 || kt < 32) return false;
  int64_t S = (1024 + wq - 1) / wq;
  if (S > kt / 16) S = kt / 16;
  // At least two workgroups per CU, else the wide split keeps more lanes
  // busy (B1 H4 N1024 D64 causal: 2 splits x 32 workgroups 273 us, wide
  // split 61 us).
  if (S < 2 || wq * S < 512) return false;
  const int64_t kpt = (kt + S - 1) / S;
  S = (kt + kpt - 1) / kpt;
  plan->splits = S;
  plan->split_tiles = kpt;
  plan->scratch_bytes =
      (size_t)(p.B * p.H * p.Nq) * (size_t)S * (size_t)(p.D + 2) * sizeof(float);
  return true;
}

hipError_t launch_prefill_f32_partials(const Problem& p) {
  switch (p.D) {
    case 16:
      return p.causal ? launch_typed<16, kTpqDefault<16>, true, kModeSplitKv, 1, kThreads, kBNF>(p)
                      : launch_typed<16, kTpqDefault<16>, false, kModeSplitKv, 1, kThreads, kBNF>(p);
    case 32:
      return p.causal ? launch_typed<32, kTpqDefault<32>, true, kModeSplitKv, 1, kThreads, kBNF>(p)
                      : launch_typed<32, kTpqDefault<32>, false, kModeSplitKv, 1, kThreads, kBNF>(p);
    case 64:
      return p.causal ? launch_typed<64, kTpqDefault<64>, true, kModeSplitKv, 1, kThreads, kBNF>(p)
                      : launch_typed<64, kTpqDefault<64>, false, kModeSplitKv, 1, kThreads, kBNF>(p);
    case 128:
      return p.causal
                 ? launch_typed<128, kTpqDefault<128>, true, kModeSplitKv, 1, kThreads, kBNF>(p)
                 : launch_typed<128, kTpqDefault<128>, false, kModeSplitKv, 1, kThreads, kBNF>(p);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill_f32(const Problem& p) {
  switch (p.D) {
    case 16: return launch_d<16>(p);
    case 32: return launch_d<32>(p);
    case 64: return launch_d<64>(p);
    case 128: return launch_d<128>(p);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
