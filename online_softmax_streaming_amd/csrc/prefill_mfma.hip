// Streaming attention prefill on gfx950 matrix cores (bf16 / f16 inputs).
//
// What is computed is the streaming_attention contract of the workshops page
// ("Intermediate and advanced kernel workshops", section "Scope and
// contracts"), batched over (B, H): each query row carries a running max m,
// running sum l and unnormalised output a across key tiles, rescaling l and
// a together when m moves (answer-key page, row A3), and one score tile is
// alive at a time.  Masked or padded scores are -inf before the max and add
// 0 to the sums, and rows with nothing visible are pinned at reference 0
// ("Kernel Notes & Checklist", gotchas ledger).
//
// Work decomposition (one workgroup = NW waves = 32*NW query rows):
//   * Each wave owns 32 query rows.  Its Q rows stay in registers for the
//     whole kernel as the B operand of v_mfma_f32_32x32x16_{bf16,f16}.
//   * Key tiles of BN = 64 rows of K and V are staged in LDS, double-buffered:
//     buffer loads with the LDS modifier move tile t+1 from HBM straight
//     into LDS (no register round trip, no LDS store instructions) while
//     tile t is computed, and rows past Nk fall outside the buffer's range
//     and arrive as zeros, so the ragged tail needs no branch.  Both tiles are stored row-major with
//     an XOR swizzle of 16-byte chunks that makes every LDS read below
//     bank-conflict free.
//   * S^T = K Q^T is formed per 32-key block, so each lane owns one query
//     column: the row max over keys is in-lane plus one exchange between the
//     two half-waves.  P^T stays in registers as the B operand of
//     O^T += V^T P^T, again one query per lane, so the rescale is a per-lane
//     scalar.  The V^T operand (8 keys of one feature per lane) is read from
//     the row-major V tile with the LDS transpose read ds_read_b64_tr_b16.
//   * The reference max is refreshed only when a row's max rises by more
//     than 8 in base-2 units; until then exponentials may reach 2^8, which
//     FP32 accumulators and bf16/f16 weights carry without loss.  Skipping
//     the refresh removes the O rescale from most tiles.  The exact row max
//     is tracked separately for the returned row state.
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
//
// ds_read_b64_tr_b16, per group of 16 lanes: if lane r addresses 4 halves
// M[r][0..3], lane i receives M[4e + i/4][i%4] for e = 0..3.

#include <type_traits>

#include "attn_kernels.h"
#include "attn_mfma.h"

namespace attn {
namespace {

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* m_out;
  float* l_out;
  int Nq, Nk;
  int group;    // query heads per K/V head
  int nqt;      // query tiles per (b, h)
  int nwork;    // workgroups per (b, h): nqt, or ceil(nqt / 2) paired causal tiles
  int total;    // (B*H) * nwork real workgroups
  int per_xcd;  // gridDim.x / 8
  float c;      // scale * log2(e)
  // Packed variable-length sequences (VARLEN kernels only): Q/out are
  // [total_q, H, D], K/V [total_k, Hkv, D], sequence b owns rows
  // cu_q[b] .. cu_q[b+1]-1 and keys cu_k[b] .. cu_k[b+1]-1; row states are
  // [H, total_q].  nqt is then the tile count of the longest sequence.
  const int* cu_q;
  const int* cu_k;
  int B, H, Hkv;
  int total_q, total_k;
  // Masked mode (MASKED kernels only, batched layout): an optional
  // bit-packed mask, bit j % 32 of word j / 32 of row (b, h, i) at
  // mask + b*mask_sb + h*mask_sh + i*mask_words, and an optional sliding
  // window (0 = none).
  const uint32_t* mask;
  int64_t mask_sb, mask_sh;
  int mask_words;
  int window;
  // Dropout mode: key j of row i of head bh is kept iff 16-bit field j % 16
  // of Philox4x64-10 on counter (j / 16, i, bh, offset) under key (seed, 0)
  // is >= drop_t; kept weights are scaled by keep_gain = 65536/(65536 - T).
  uint64_t seed, offset;
  uint32_t drop_t;
  float keep_gain;
  // Split-key mode (SPLITKV kernels only, batched or packed layout): work
  // item (head, query tile, split s) covers key tiles [s * kpt, (s + 1) *
  // kpt) and writes each row's state, FP32, base 2, l and a relative to the
  // exact maximum m: a[D] to part[row][s][.], (m, l) to part_ml[row][s][.],
  // rows in row-state order.
  float* part;
  float* part_ml;
  int S;    // splits per row
  int kpt;  // key tiles per split
};

// Kernel modes: batched [B, H, N, D]; packed variable-length sequences;
// batched with an arbitrary mask and/or a sliding window; batched with
// dropout on the probabilities; batched or packed with the keys split over
// workgroups (partial states to scratch).
enum : int {
  kModeBatched = 0,
  kModeVarlen = 1,
  kModeMasked = 2,
  kModeDropout = 3,
  kModeSplitKv = 4,
  kModeVarlenSplitKv = 5
};

constexpr int kBN = 64;              // keys per tile
// LDS operand reads in flight ahead of the MFMA that uses them.
#ifndef ATTN_KPF
#define ATTN_KPF 6
#endif
#ifndef ATTN_VPF
#define ATTN_VPF 4
#endif
constexpr int kKPF = ATTN_KPF;
// At D = 64 (8 V operands per tile) two ahead measured 8 % faster noncausal
// (770 against 711 TFLOP/s, B3 H8 N4099 bf16) and level elsewhere.
template <int D> constexpr int kVPF = D == 64 ? 2 : ATTN_VPF;
constexpr float kRefreshGap = 8.0f;  // base-2 units; see the file comment

// Sixteen-wave workgroups (four waves per SIMD) need at most 128 VGPRs.
template <int NW> constexpr int kWavesPerEu = NW >= 16 ? 4 : 2;

template <typename T, int D, int NW, bool CAUSAL, int MODE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(kWavesPerEu<NW>)))
void prefill_mfma_kernel(PrefillArgs a) {
  constexpr bool VARLEN = MODE == kModeVarlen || MODE == kModeVarlenSplitKv;
  constexpr bool MASKED = MODE == kModeMasked;
  constexpr bool DROPOUT = MODE == kModeDropout;
  constexpr bool SPLITKV = MODE == kModeSplitKv || MODE == kModeVarlenSplitKv;
  typedef typename Mfma<T>::vec8 vec8;
  typedef typename Mfma<T>::vec4 vec4;
  typedef typename Mfma<T>::vec2 vec2;
  typedef Geo<D> G;
  constexpr int BM = 32 * NW;
  constexpr int BN = kBN;
  constexpr int DP = D < 32 ? 32 : D;  // O^T rows, padded to one MFMA block
  constexpr int KC = D / 16;           // k-chunks of Q.K^T
  constexpr int NB = DP / 32;          // 32-row blocks of O^T
  constexpr int NT = NW * 64;          // threads per workgroup
  constexpr int TILE = BN * D * 2;     // bytes of one K or V tile
  static_assert(G::steps_keep_swizzle(), "tile steps must keep the LDS swizzle");

  // Two LDS buffers as separate objects, so the compiler can tell the
  // direct-to-LDS loads into one from the operand reads of the other.
  __shared__ __attribute__((aligned(1024))) unsigned char smem0[2][TILE];  // [K, V]
  __shared__ __attribute__((aligned(1024))) unsigned char smem1[2][TILE];
  // Under a mask: which key tiles hold a key visible to some row of the
  // workgroup's query tile (bit b covers tiles t_first + b*g .. + g-1).
  constexpr int kTileBitWords = MASKED ? 256 : 1;
  __shared__ uint32_t tile_bits[kTileBitWords];
  // Packed sequences: key counts of up to kSortMaxB sequences, and the
  // sequence a workgroup takes (see below).  The ranking costs each
  // workgroup about B*B/(64*NW) LDS reads, so it stops at 64 sequences; with
  // many sequences the hardware's dispatch already interleaves their lengths.
  constexpr int kSortMaxB = VARLEN ? 64 : 1;
  __shared__ int seq_keys[kSortMaxB];
  __shared__ int seq_pick;
  auto tile_ptr = [&](int buf, int kv) __attribute__((always_inline)) -> unsigned char* {
    return buf == 0 ? &smem0[kv][0] : &smem1[kv][0];
  };

  // Workgroup -> (head, query tiles).  Consecutive workgroup ids land on
  // different XCDs (round-robin over 8); regroup them so each XCD walks a
  // contiguous range of heads and their K/V stays in that XCD's L2.
  // Causal: a workgroup takes query tile nqt-1-r and then tile r of its
  // head, so every workgroup streams the same number of key tiles and the
  // grid fills the CUs evenly (with one tile per workgroup, the short
  // diagonal tiles at the end of each XCD's range leave CUs idle).  The
  // second pass walks its key tiles from the diagonal down: the head's
  // workgroups then read key tile x at step x of their first passes and
  // together at one later step of their second passes, so a tile stays in
  // L2 between its reads far more often (HBM reads of the B4 H16 N4096
  // causal workload fall from 1.60 to 1.30 times the algorithmic bytes).
  const int bid = blockIdx.x;
  const int logical = (bid & 7) * a.per_xcd + (bid >> 3);
  if (logical >= a.total) return;
  const int bh = logical / a.nwork;
  const int rr = logical - bh * a.nwork;

  // This head's rows: element offsets of Q/out and K/V row 0, row strides,
  // and the row-state index of query row 0 (stride 1).
  int Nq = a.Nq, Nk = a.Nk, nqt = a.nqt;
  int64_t qbase, kbase, stat0;
  int64_t sq = D, sk = D;
  if (VARLEN) {
    // Sequence bounds are clamped into the packed tensors, so no value of
    // cu_q / cu_k can address memory outside them.
    // Head-major order: each XCD's contiguous range of workgroups then holds
    // a few heads of every sequence, so ragged sequence lengths do not pile
    // the long sequences onto some XCDs (batch-major order would give each
    // XCD a few whole sequences).  Within a head the sequences go in
    // decreasing key count (ties by index), so the longest workgroups start
    // first and the short ones fill in behind them (up to kSortMaxB = 64
    // sequences; beyond that, input order).
    const int h = bh / a.B;
    int b = bh - h * a.B;
    if (a.B > 1 && a.B <= kSortMaxB) {
      const int kq = b;
      for (int s = threadIdx.x; s < a.B; s += NW * 64) {
        const int s0 = min(max(a.cu_k[s], 0), a.total_k);
        seq_keys[s] = min(max(a.cu_k[s + 1], s0), a.total_k) - s0;
      }
      __syncthreads();
      for (int s = threadIdx.x; s < a.B; s += NW * 64) {
        const int ks = seq_keys[s];
        int rank = 0;
        for (int s2 = 0; s2 < a.B; ++s2) {
          const int k2 = seq_keys[s2];
          rank += k2 > ks || (k2 == ks && s2 < s);
        }
        if (rank == kq) seq_pick = s;
      }
      __syncthreads();
      b = seq_pick;
    }
    const int q0 = min(max(a.cu_q[b], 0), a.total_q);
    const int q1 = min(max(a.cu_q[b + 1], q0), a.total_q);
    const int k0 = min(max(a.cu_k[b], 0), a.total_k);
    const int k1 = min(max(a.cu_k[b + 1], k0), a.total_k);
    Nq = q1 - q0;
    Nk = k1 - k0;
    nqt = (Nq + BM - 1) / BM;
    // Shorter than the longest sequence.
    if (rr >= (SPLITKV ? nqt * a.S : CAUSAL ? (nqt + 1) / 2 : nqt)) return;
    sq = (int64_t)a.H * D;
    sk = (int64_t)a.Hkv * D;
    qbase = (int64_t)q0 * sq + (int64_t)h * D;
    kbase = (int64_t)k0 * sk + (int64_t)(h / a.group) * D;
    stat0 = (int64_t)h * a.total_q + q0;
  } else {
    qbase = (int64_t)bh * Nq * D;
    // Query head (b, h) reads K/V head (b, h / group): bh / group.
    kbase = (int64_t)(bh / a.group) * Nk * D;
    stat0 = (int64_t)bh * Nq;
  }
  // Split-key mode: one query tile per work item (no causal pairing) and
  // split sp of its keys.
  const int sp = SPLITKV ? rr % a.S : 0;
  const int npass = !SPLITKV && CAUSAL && nqt - 1 - rr != rr ? 2 : 1;
  for (int pass = 0; pass < npass; ++pass) {
    const int qt = SPLITKV ? rr / a.S : CAUSAL ? (pass == 0 ? nqt - 1 - rr : rr) : rr;

    const int off = Nk - Nq;
    const T* __restrict__ Qh = static_cast<const T*>(a.q) + qbase;
    const T* Kh = static_cast<const T*>(a.k) + kbase;
    const T* Vh = static_cast<const T*>(a.v) + kbase;
    T* __restrict__ Oh = static_cast<T*>(a.o) + qbase;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h32 = lane >> 5;
    const int l32 = lane & 31;
    // Causal: query tiles are aligned to the last row, so when Nq is not a
    // multiple of BM the partial tile is tile 0, whose rows see the fewest
    // keys (one key tile at the ragged workload's 3-row tail instead of all
    // of them); rows i0 .. -1 of that tile are ghosts.
    const int i0 = qt * BM - (CAUSAL ? (BM - Nq % BM) % BM : 0);
    const int qw0 = i0 + wave * 32;  // first query row of this wave
    const int qrow = qw0 + l32;      // this lane's query row
    const float c = a.c;

    // Q fragment: B operand, 8 consecutive features per k-chunk.  Rows
    // outside [0, Nq) (ghost rows) are zero so their scores stay finite;
    // never stored.
    vec8 qf[KC];
  #pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      qf[kc] = qrow >= 0 && qrow < Nq
                   ? *reinterpret_cast<const vec8*>(Qh + (int64_t)qrow * sq + kc * 16 + h32 * 8)
                   : vec8{};
    }

    // Key range that holds a visible key for some real row of this tile
    // (a window hides every key below row i0's lower bound from all rows).
    int kend = Nk;
    if (CAUSAL) kend = min(Nk, min(i0 + BM, Nq) + off);
    const int win = MASKED ? a.window : 0;
    const int t_first = SPLITKV ? sp * a.kpt : win > 0 ? max(0, i0 + off - win + 1) / BN : 0;
    const int ntiles = SPLITKV ? min(kend > 0 ? (kend + BN - 1) / BN : 0, (sp + 1) * a.kpt)
                               : kend > 0 ? (kend + BN - 1) / BN : 0;

    // Buffer resources over this head's K and V: offsets at or past Nk rows
    // are out of range and read as zero (rows are 2*sk bytes apart; the
    // range ends at the last byte of row Nk-1).
    const uint32_t kpitch = (uint32_t)(2 * sk);
    const uint32_t kv_bytes =
        VARLEN ? (Nk > 0 ? (uint32_t)(Nk - 1) * kpitch + (uint32_t)(2 * D) : 0u)
               : (uint32_t)Nk * (uint32_t)(2 * D);
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(Kh), 0, (int)kv_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(Vh), 0, (int)kv_bytes, 0x00020000);

    // Per-lane LDS byte offsets, loop invariant.
    int koff[KC];  // K fragment of k-chunk kc for key l32 (+32 rows for block 1)
  #pragma unroll
    for (int kc = 0; kc < KC; ++kc) koff[kc] = G::off(l32, 2 * kc + h32);
    // Transpose-read addresses: key 8*half + 4*h32 + i/4 (+16 per key group),
    // features 4*(i%4).. of feature block n, with i = lane % 16.
    int voff[NB][2];
    {
      const int i = lane & 15;
  #pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int row = 8 * half + 4 * h32 + (i >> 2);
  #pragma unroll
        for (int n = 0; n < NB; ++n) {
          int col = 16 * ((lane >> 4) & 1) + 32 * n + 4 * (i & 3);
          if (col >= D) col -= D;  // D = 16: O^T rows 16..31 are computed, then discarded
          voff[n][half] = G::off(row, col >> 3) + ((col & 7) << 1);
        }
      }
    }

    float m_run = kNegInf;   // reference max for the exponentials, base-2 units
    float m_true = kNegInf;  // exact running max, base-2 units
    float l_run = 0.f;       // this half-wave's share of the running sum
    f32x16 acc[NB];
  #pragma unroll
    for (int n = 0; n < NB; ++n) acc[n] = f32x16{};

    // Tile staging: each thread moves NPT 16-byte slots of K and of V per
    // tile.  LDS slot s holds chunk (s % CPR) ^ swz(row) of row s / CPR, so
    // consecutive lanes fill consecutive 16 bytes of LDS and read a
    // permutation of one row's chunks (one coalesced row per 16 lanes for
    // D = 128).
    constexpr int NSLOT = TILE / 16;
    constexpr int NPT = (NSLOT + NT - 1) / NT;
    static_assert(NSLOT % 64 == 0, "a wave moves whole 1 KB LDS blocks");
    // Tile staging straight from HBM into LDS (buffer loads with the LDS
    // modifier): lane l of a wave writes the 16 bytes at the wave's block
    // base + 16*l, i.e. LDS slot s = tid + u*NT, which holds chunk
    // (s % CPR) ^ swz(row) of row s / CPR.  Rows past Nk are out of the
    // buffer range and arrive as zeros.  The barrier after the step waits
    // for these loads (its fence covers writes into LDS by the loads).
    auto load_tile = [&](int j0, int buf) __attribute__((always_inline)) {
  #pragma unroll
      for (int u = 0; u < NPT; ++u) {
        const int sl = tid + u * NT;
        const int sl0 = wave * 64 + u * NT;  // first slot of this wave's block
        if (NSLOT % NT == 0 || sl0 < NSLOT) {
          const int row = sl / G::CPR;
          const int chunk = (sl % G::CPR) ^ G::swz(row);
          const int j = min(j0 + row, Nk);  // rows past Nk: out of range, read as 0
          const uint32_t vo = (uint32_t)j * kpitch + (uint32_t)(chunk << 4);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, LDS_PTR(void, tile_ptr(buf, 0) + sl0 * 16),
                                                   16, (int)vo, 0, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, LDS_PTR(void, tile_ptr(buf, 1) + sl0 * 16),
                                                   16, (int)vo, 0, 0, 0);
        }
      }
    };

    // Mask words of this lane's row for keys j0 .. j0+63 (MASKED only).
    const uint32_t* mrow = nullptr;
    if (MASKED && a.mask && qrow >= 0 && qrow < Nq) {
      const int b = bh / a.H, h = bh - b * a.H;
      mrow = a.mask + (int64_t)b * a.mask_sb + (int64_t)h * a.mask_sh + (int64_t)qrow * a.mask_words;
    }
    auto mask_word = [&](int w) -> uint32_t {
      if (!MASKED || !a.mask) return ~0u;
      return mrow && w < a.mask_words ? mrow[w] : 0u;
    };

    auto compute = [&](auto bufc, int j0, bool need_mask, uint32_t mw0, uint32_t mw1) {
      constexpr int buf = decltype(bufc)::value;
      const unsigned char* kt = tile_ptr(buf, 0);
      const unsigned char* vt = tile_ptr(buf, 1);

      // S^T = K Q^T.  MFMA i uses K fragment i (key block i / KC, feature
      // chunk i % KC); each fragment is read KPF MFMAs ahead so LDS latency
      // hides behind the matrix work, and scheduling barriers keep that order.
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

      // The first V^T operands of O^T += V^T P^T do not depend on the softmax:
      // request them now so they arrive while it runs.  Slot e (0..3) of the
      // first transpose read is key 16*c2 + 4*h32 + e, of the second key
      // 16*c2 + 8 + 4*h32 + e: the keys that registers 8*(c2&1) + 0..7 of S^T
      // block c2/2 hold.  Operand i is feature block i / (BN/16), key group
      // i % (BN/16).
      constexpr int NV = NB * (BN / 16);
      vec8 vf[NV];
      auto vread = [&](int i) {
        const int n = i / (BN / 16), c2 = i % (BN / 16);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            LDS_PTR(s16x4, vt + voff[n][0] + 16 * c2 * 2 * D));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            LDS_PTR(s16x4, vt + voff[n][1] + 16 * c2 * 2 * D));
        return __builtin_bit_cast(vec8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
  #pragma unroll
      for (int i = 0; i < kVPF<D> && i < NV; ++i) vf[i] = vread(i);
      __builtin_amdgcn_sched_barrier(0);

      if (need_mask) {
        // Register r of block mb holds key j0 + 4*h32 + kr with the
        // immediate kr = 32mb + 8(r/4) + r%4; the ragged end and the causal
        // rule become one per-lane limit (visible iff kr < lim), so each test
        // compares an immediate.  The mask word bit of the key is bit
        // 8(r/4) + r%4 of the lane's word for block mb shifted by 4*h32.
        const int lim = min(Nk - j0, CAUSAL ? qrow + off - j0 + 1 : Nk - j0) - 4 * h32;
        const int wlo = win > 0 ? qrow + off - win - j0 - 4 * h32 : -(1 << 30);  // visible iff kr > wlo
        const uint32_t mws[2] = {mw0 >> (4 * h32), mw1 >> (4 * h32)};
  #pragma unroll
        for (int mb = 0; mb < BN / 32; ++mb) {
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kr = mb * 32 + (r >> 2) * 8 + (r & 3);
            bool vis = kr < lim;
            if (MASKED) {
              vis = vis && kr > wlo;
              vis = vis && ((mws[mb] >> ((r >> 2) * 8 + (r & 3))) & 1u);
            }
            s[mb][r] = vis ? s[mb][r] : kNegInf;
          }
        }
      }
      // Tile max of this row: in-lane, then across the two half-waves.
      float mx = s[0][0];
  #pragma unroll
      for (int mb = 0; mb < BN / 32; ++mb)
  #pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
      mx = half_max(mx);
      const float m_tile = mx * c;  // -inf when nothing in the tile is visible
      m_true = fmaxf(m_true, m_tile);
      const bool refresh = m_tile > m_run + kRefreshGap;
      if (__builtin_amdgcn_ballot_w64(refresh)) {
        const float m_new = refresh ? m_tile : m_run;
        const float alpha = exp2_hw(m_run - pinned_ref(m_new));
        l_run *= alpha;
  #pragma unroll
        for (int n = 0; n < NB; ++n) acc[n] *= alpha;
        m_run = m_new;
      }
      const float ref = pinned_ref(m_run);
  #pragma unroll
      for (int mb = 0; mb < BN / 32; ++mb)
  #pragma unroll
        for (int r = 0; r < 16; ++r) s[mb][r] = exp2_hw(__builtin_fmaf(s[mb][r], c, -ref));

      // P^T rounded to the input type: the B operand of O^T += V^T P^T.  The
      // row sum adds the same rounded weights, so the normalisation matches
      // the numerator exactly (one visible key gives weight 1 and out = V).
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

      if (DROPOUT) {
        // Group c2 of pf holds keys j0 + 16c2 + t with t = 4*h32 + e%4 +
        // 8*(e/4): fields t of Philox block ((j0 / 16) + c2, qrow, bh,
        // offset), i.e. words h32 and h32 + 2 of it.  The lanes of half h32
        // run blocks 2*h32 + cc (cc = 0, 1) of their row in full.  A
        // permlane32 swap of (word 2x, word 2x + 1) trades the upper half's
        // first register for the lower half's second, which leaves in every
        // lane word h32 + 2x of block cc in the first register and of block
        // 2 + cc in the second: the words this lane's groups need, with no
        // per-lane choice.
        uint64_t own[2][4];
  #pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          own[cc][0] = (uint64_t)((j0 >> 4) + 2 * h32 + cc);
          own[cc][1] = (uint64_t)qrow;
          own[cc][2] = (uint64_t)bh;
          own[cc][3] = a.offset;
          philox4x64_10(own[cc], a.seed, 0);
        }
        // fw[c2][k]: the two 16-bit fields of 32-bit register k of pf[c2].
        uint32_t fw[BN / 16][4];
  #pragma unroll
        for (int cc = 0; cc < 2; ++cc)
  #pragma unroll
          for (int x = 0; x < 2; ++x)
  #pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
              const auto r = __builtin_amdgcn_permlane32_swap(
                  (uint32_t)(own[cc][2 * x] >> (32 * hf)),
                  (uint32_t)(own[cc][2 * x + 1] >> (32 * hf)), false, false);
              fw[cc][2 * x + hf] = r[0];
              fw[2 + cc][2 * x + hf] = r[1];
            }
        // Keep a weight iff its field is >= T, two weights per 32-bit
        // register: d = max(T - field, 0) and g = max(1 - d, 0) per 16-bit
        // half (saturating packed subtracts), so g = 1 exactly for a kept
        // weight and 0 otherwise, and the packed 16-bit product of the
        // weight's bits with g keeps or clears them.  Written out because
        // the compiler turns the same arithmetic in C into two compares and
        // two selects per register.
        const uint32_t t2 = a.drop_t * 0x10001u, one2 = 0x10001u;
  #pragma unroll
        for (int c2 = 0; c2 < BN / 16; ++c2) {
          uint32_t pw[4];
          __builtin_memcpy(pw, &pf[c2], sizeof(pw));
  #pragma unroll
          for (int k = 0; k < 4; ++k) {
            uint32_t g;
            asm("v_pk_sub_u16 %1, %2, %3 clamp\n\t"
                "v_pk_sub_u16 %1, %4, %1 clamp\n\t"
                "v_pk_mul_lo_u16 %0, %5, %1"
                : "=v"(pw[k]), "=&v"(g)
                : "v"(t2), "v"(fw[c2][k]), "v"(one2), "v"(pw[k]));
          }
          __builtin_memcpy(&pf[c2], pw, sizeof(pw));
        }
      }

      // O^T += V^T P^T, each V^T operand read kVPF MFMAs ahead.
      __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
      for (int i = 0; i < NV; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (i + kVPF<D> < NV) vf[i + kVPF<D>] = vread(i + kVPF<D>);
        acc[i / (BN / 16)] = Mfma<T>::mma(vf[i], pf[i % (BN / 16)], acc[i / (BN / 16)]);
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    if (ntiles > t_first) {
      const int q_last = min(qw0 + 32, Nq) - 1;  // last real row of this wave
      // Whether the causal rule and the window leave tile u any key this
      // wave's rows may see.
      auto wave_active = [&](int u) __attribute__((always_inline)) {
        const int ju = u * BN;
        bool act = qw0 < Nq && qw0 + 31 >= 0 && (!CAUSAL || ju <= q_last + off);
        if (MASKED && win > 0) act = act && ju + BN - 1 > qw0 + off - win;
        return act;
      };
      // Under a mask, key tiles no row of the workgroup may see are neither
      // staged nor computed, and cost no step: before the key loop the
      // workgroup maps which tiles of [t_first, ntiles) hold a visible key
      // for some row (its rows' mask words, clipped to each row's causal and
      // window range), and the loop walks only those.  Bit b covers g tiles
      // (g = 1 unless more than 8192 tiles are in range).
      const bool skip_tiles = MASKED && a.mask != nullptr;
      constexpr int kTileBits = 32 * kTileBitWords;
      const int span = ntiles - t_first;
      const int g = skip_tiles ? (span + kTileBits - 1) / kTileBits : 1;
      if (skip_tiles) {
        for (int w = tid; w < kTileBitWords; w += NT) tile_bits[w] = 0u;
        __syncthreads();
        // Two threads per row, alternate mask words; loads go out in
        // batches so their latencies overlap.
        const int r = tid >> 1, par = tid & 1;
        const int i = i0 + r;
        if (r < BM && i >= 0 && i < Nq) {
          const int b = bh / a.H, h = bh - b * a.H;
          const uint32_t* row = a.mask + (int64_t)b * a.mask_sb + (int64_t)h * a.mask_sh +
                                (int64_t)i * a.mask_words;
          // Keys this row may see at all: [klo, khi).
          int khi = Nk;
          if (CAUSAL) khi = min(khi, i + off + 1);
          khi = min(khi, ntiles * BN);
          int klo = t_first * BN;
          if (win > 0) klo = max(klo, i + off - win + 1);
          if (khi > klo) {
            const int wlo = klo >> 5, whi = (khi + 31) >> 5;
            // Sets the bit of each tile whose (clipped) words in x[] are not
            // all zero; x[e] is word w0 + e * wstep.
            auto mark = [&](const uint32_t* x, int n, int w0, int wstep) __attribute__((always_inline)) {
              uint32_t bits = 0u;
              int bw = -1;  // bitmap word `bits` belongs to
              for (int e = 0; e < n; ++e) {
                const int w = w0 + e * wstep;
                uint32_t xv = w >= wlo && w < whi ? x[e] : 0u;
                if (w == (klo >> 5)) xv &= ~0u << (klo & 31);
                if (w == ((khi - 1) >> 5) && (khi & 31)) xv &= ~0u >> (32 - (khi & 31));
                if (xv != 0u) {
                  const int bb = ((w >> 1) - t_first) / g;
                  if ((bb >> 5) != bw) {
                    if (bits) atomicOr(&tile_bits[bw], bits);
                    bw = bb >> 5;
                    bits = 0u;
                  }
                  bits |= 1u << (bb & 31);
                }
              }
              if (bits) atomicOr(&tile_bits[bw], bits);
            };
            if ((a.mask_words & 3) == 0 && (reinterpret_cast<uintptr_t>(row) & 15) == 0) {
              // 16-byte loads (rows of whole 4-word chunks, so no chunk runs
              // past its row): the pair's threads take alternate chunks, 8
              // in flight per thread.
              constexpr int kBatch = 8;
              for (int c0 = (wlo >> 2) + par; 4 * c0 < whi; c0 += 2 * kBatch) {
                uint32_t x[4 * kBatch];
  #pragma unroll
                for (int e = 0; e < kBatch; ++e) {
                  const int c = c0 + 2 * e;
                  const u32x4 v = 4 * c < whi ? *reinterpret_cast<const u32x4*>(row + 4 * c) : u32x4{};
  #pragma unroll
                  for (int f = 0; f < 4; ++f) x[4 * e + f] = v[f];
                }
  #pragma unroll
                for (int e = 0; e < kBatch; ++e) mark(x + 4 * e, 4, 4 * (c0 + 2 * e), 1);
              }
            } else {
              // Word loads: alternate words, 16 in flight per thread.
              constexpr int kBatch = 16;
              for (int w0 = wlo + par; w0 < whi; w0 += 2 * kBatch) {
                uint32_t x[kBatch];
  #pragma unroll
                for (int e = 0; e < kBatch; ++e) {
                  const int w = w0 + 2 * e;
                  x[e] = w < whi ? row[w] : 0u;
                }
                mark(x, kBatch, w0, 2);
              }
            }
          }
        }
        __syncthreads();
      }
      // The next key tile after t the workgroup needs (ntiles if none).
      auto next_tile = [&](int t) __attribute__((always_inline)) -> int {
        if (!skip_tiles) return t + 1;
        int u = t + 1;
        if (u >= ntiles) return ntiles;
        int b = (u - t_first) / g;
        if ((u - t_first) % g != 0) return u;  // inside the super tile being walked
        const int nbits = (span + g - 1) / g;
        while (b < nbits) {
          const uint32_t word =
              __builtin_amdgcn_readfirstlane(tile_bits[b >> 5]) & (~0u << (b & 31));
          if (word != 0u) return min(ntiles, t_first + (32 * (b >> 5) + __builtin_ctz(word)) * g);
          b = 32 * ((b >> 5) + 1);
        }
        return ntiles;
      };
      // Key tile of step t: the second causal pass runs from the diagonal
      // down (plain, packed and dropout layouts alike, so they agree bit for
      // bit); the masked layout and every first pass run in increasing order.
      const bool down = !MASKED && CAUSAL && pass == 1;
      auto tile_of = [&](int t) __attribute__((always_inline)) { return down ? ntiles - 1 - t : t; };
      const int t_start = skip_tiles ? next_tile(t_first - 1) : t_first;
      // Mask words of this lane's row for the tile being computed (mw) and
      // the next one (nw), fetched one step ahead.
      uint32_t nw0 = 0u, nw1 = 0u;
      if (MASKED && t_start < ntiles) {
        nw0 = mask_word(2 * t_start);
        nw1 = mask_word(2 * t_start + 1);
      }
      if (t_start < ntiles) load_tile(tile_of(t_start) * BN, 0);
      __syncthreads();
      auto step = [&](auto bufc, int t, int tn) {
        constexpr int buf = decltype(bufc)::value;
        const int j0 = tile_of(t) * BN;
        if (tn < ntiles) load_tile(tile_of(tn) * BN, buf ^ 1);  // in flight while this tile is computed
        const uint32_t mw0 = nw0, mw1 = nw1;
        if (MASKED && tn < ntiles) {
          nw0 = mask_word(2 * tn);
          nw1 = mask_word(2 * tn + 1);
        }
        bool active = wave_active(tile_of(t));
        // A tile none of this wave's rows may see under the mask is skipped.
        if (MASKED && a.mask) active = active && __builtin_amdgcn_ballot_w64((mw0 | mw1) != 0u) != 0;
        if (active) {
          bool need_mask = (j0 + BN > Nk) || (CAUSAL && j0 + BN - 1 > qw0 + off);
          // Mask bits are applied only where some row of the wave hides a
          // key of the tile (a tile wholly inside every row's mask costs no
          // mask work).
          if (MASKED)
            need_mask = need_mask || (win > 0 && j0 <= q_last + off - win) ||
                        (a.mask && __builtin_amdgcn_ballot_w64((mw0 & mw1) != ~0u) != 0);
          compute(bufc, j0, need_mask, mw0, mw1);
        }
        // Buffer buf^1 was last read in the previous step, before its barrier.
        __syncthreads();
      };
      for (int t = t_start; t < ntiles;) {
        int tn = next_tile(t);
        step(std::integral_constant<int, 0>{}, t, tn);
        t = tn;
        if (t >= ntiles) break;
        tn = next_tile(t);
        step(std::integral_constant<int, 1>{}, t, tn);
        t = tn;
      }
    }

    // Epilogue: join the two half-wave sums, normalise, one cast, store.
    const float l_tot = half_sum(l_run);
    if (SPLITKV) {
      // The split's state, relative to the exact maximum (a = 0, l = 0,
      // m = -inf for a row that sees no key of the split).
      if (qrow >= 0 && qrow < Nq) {
        const float to_true = m_true == kNegInf ? 0.f : exp2_hw(m_run - m_true);
        const int64_t st = (stat0 + qrow) * a.S + sp;
        float* pa = a.part + st * D;
  #pragma unroll
        for (int n = 0; n < NB; ++n) {
  #pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int d0 = n * 32 + g * 8 + h32 * 4;
            if (d0 < D)
              *reinterpret_cast<f32x4*>(pa + d0) =
                  f32x4{acc[n][g * 4] * to_true, acc[n][g * 4 + 1] * to_true,
                        acc[n][g * 4 + 2] * to_true, acc[n][g * 4 + 3] * to_true};
          }
        }
        if (h32 == 0)
          *reinterpret_cast<f32x2*>(a.part_ml + 2 * st) = f32x2{m_true, l_tot * to_true};
      }
    } else if (qrow >= 0 && qrow < Nq) {
      float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      if (DROPOUT) inv *= a.keep_gain;
      T* orow = Oh + (int64_t)qrow * sq;
  #pragma unroll
      for (int n = 0; n < NB; ++n) {
  #pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = n * 32 + g * 8 + h32 * 4;
          if (d0 < D) {
            vec4 o4;
  #pragma unroll
            for (int e = 0; e < 4; ++e) o4[e] = from_f32<T>(acc[n][g * 4 + e] * inv);
            *reinterpret_cast<vec4*>(orow + d0) = o4;
          }
        }
      }
      if (h32 == 0) {
        // Row state relative to the exact max: sum exp = l * e^m.
        const int64_t row = stat0 + qrow;
        const float to_true = m_true == kNegInf ? 0.f : exp2_hw(m_run - m_true);
        if (a.m_out) a.m_out[row] = m_true * kLn2;
        if (a.l_out) a.l_out[row] = l_tot * to_true;
      }
    }
  }  // pass
}

template <typename T, int D, int NW, bool CAUSAL, int MODE>
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
  a.group = (int)(p.H / p.Hkv);
  a.nqt = (int)((p.Nq + BM - 1) / BM);  // varlen: p.Nq is the longest sequence
  a.cu_q = p.cu_q;
  a.cu_k = p.cu_k;
  a.B = (int)p.B;
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
  const int64_t state_rows = p.cu_q ? p.H * p.total_q : p.B * p.H * p.Nq;
  a.part_ml = p.part ? p.part + state_rows * p.splits * D : nullptr;
  a.S = (int)p.splits;
  a.kpt = (int)p.split_tiles;
  a.nwork = MODE == kModeSplitKv || MODE == kModeVarlenSplitKv ? a.nqt * a.S
            : CAUSAL                                         ? (a.nqt + 1) / 2
                                                             : a.nqt;
  const int64_t total = p.B * p.H * a.nwork;
  a.total = (int)total;
  const int64_t grid = (total + 7) / 8 * 8;
  a.per_xcd = (int)(grid / 8);
  a.c = p.scale * kLog2e;
  hipLaunchKernelGGL((prefill_mfma_kernel<T, D, NW, CAUSAL, MODE>), dim3((unsigned)grid),
                     dim3(NW * 64), 0, p.stream, a);
  return hipGetLastError();
}

// Waves per workgroup (32 query rows each); a build-time tuning knob.
#ifndef ATTN_PREFILL_WAVES
#define ATTN_PREFILL_WAVES 8
#endif
constexpr int kWaves = ATTN_PREFILL_WAVES;
// Up to this many eight-wave workgroups the key-split kernel wins; beyond,
// per-workgroup chains are long enough that the tiled kernel (with four-wave
// workgroups up to half the CUs) does.  D = 128: below 64 (B1 H2 N4096
// causal, 16 workgroups: 36 us split, 75 tiled; at 64 the two trade places
// by shape).  D <= 64: up to 64 (B2 H8 N2048 D32 causal, 64 workgroups: 21.0
// us split, 25.5 tiled; B1 H4 N4096 D64 causal, 32: 36 against 52; at 128
// the four-wave kernel is level or ahead, B4 H8 N2048 D16 causal 21.9
// against 27.0 us).
template <int D>
constexpr int64_t kSmallGridWgs = D > 64 ? 63 : 64;
#ifndef SPLITKV_MAX_WQ
#define SPLITKV_MAX_WQ 64
#endif
#ifndef SPLITKV_MIN_KEY_TILES
#define SPLITKV_MIN_KEY_TILES 32
#endif
#ifndef SPLITKV_MIN_TILES
#define SPLITKV_MIN_TILES 16
#endif
#ifndef SPLITKV_TARGET_WGS
#define SPLITKV_TARGET_WGS 256
#endif
constexpr int64_t kNumCUs = 256;

// Every layout of one workgroup size.
template <typename T, int D, int NW>
hipError_t launch_nw(const Problem& p) {
  if (p.cu_q)
    return p.causal ? launch_typed<T, D, NW, true, kModeVarlen>(p)
                    : launch_typed<T, D, NW, false, kModeVarlen>(p);
  if (p.mask || p.window > 0)
    return p.causal ? launch_typed<T, D, NW, true, kModeMasked>(p)
                    : launch_typed<T, D, NW, false, kModeMasked>(p);
  if (p.dropout)
    return p.causal ? launch_typed<T, D, NW, true, kModeDropout>(p)
                    : launch_typed<T, D, NW, false, kModeDropout>(p);
  return p.causal ? launch_typed<T, D, NW, true, kModeBatched>(p)
                  : launch_typed<T, D, NW, false, kModeBatched>(p);
}

template <typename T, int D>
hipError_t launch_d(const Problem& p) {
  // Workgroups of kWaves waves the problem would take (varlen: with every
  // sequence as long as the longest).  The choices below depend only on
  // (B, H, Nq, D, causal), so the layouts of one problem (plain, varlen,
  // masked, dropout) split their rows alike and agree bit for bit where
  // their arithmetic does.
  const int64_t nqt = (p.Nq + 32 * kWaves - 1) / (32 * kWaves);
  const int64_t wgs = p.B * p.H * (p.causal ? (nqt + 1) / 2 : nqt);
  const bool plain = !p.cu_q && !p.mask && p.window <= 0 && !p.dropout;
  // A small problem (few workgroups, kSmallGridWgs) splits the keys of each
  // 32-row block over the waves of a workgroup (prefill_splitk.hip): more
  // waves busy, each with a shorter chain.
  if (plain && wgs <= kSmallGridWgs<D>) return launch_prefill_splitk(p);
  // A grid that would fill at most half the CUs takes four-wave workgroups
  // (128 rows): twice as many, one per CU, each SIMD running one wave.  B1
  // H8 N8192 D64 causal 137 -> 97 us, B1 H4 N16384 D128 causal 363 -> 280
  // us, B1 H8 N4096 D128 noncausal 93 -> 73 us; with 256 eight-wave
  // workgroups they lose (B2 H8 N4096 D128 noncausal 122 -> 129 us).
  if (wgs <= kNumCUs / 2) return launch_nw<T, D, 4>(p);
  if constexpr (D == 64) {
    // Noncausal D = 64 whose eight-wave grid would put a second workgroup
    // on some CUs while sixteen-wave workgroups (512 rows) fit one per CU:
    // the larger workgroups fill the CUs once, each with four waves per SIMD
    // (B3 H8 N4099 f16: 780 against 730 TFLOP/s; shapes that fill the GPU
    // several times over are level, small ones lose and keep eight waves).
    const int64_t wgs16 = p.B * p.H * ((p.Nq + 511) / 512);
    if (plain && !p.causal && wgs > kNumCUs && wgs16 <= kNumCUs)
      return launch_typed<T, D, 16, false, kModeBatched>(p);
  }
  return launch_nw<T, D, kWaves>(p);
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

// Folds the S split states of each row into out and (m, l), merge A1 over
// groups of G splits: a group's states are loaded at once (one round
// of memory latency per group), then weighted by 2^(m_s - M) against the
// exact maximum M so far, the running sums rescaled when M grows.  D / 4
// lanes per row, four features per lane, 16-byte loads.
constexpr int kCombineThreads = 256;

template <typename T, int D, int G>
__global__ __launch_bounds__(kCombineThreads) void splitkv_combine_kernel(
    const float* __restrict__ part, const float* __restrict__ part_ml, T* __restrict__ out,
    float* __restrict__ m_out, float* __restrict__ l_out, int rows, int S, const int* cu_q, int H,
    int total_q, int row_span, int causal) {
  constexpr int LPR = D / 4;
  constexpr int RPB = kCombineThreads / LPR;
  const int lr = threadIdx.x % LPR;
  int row;       // row-state index
  int64_t orow;  // output row
  if (cu_q) {
    // Packed sequences: workgroup (sequence b, head h, chunk c) takes rows
    // c * RPB .. of the sequence, as far as the split kernel wrote states:
    // its row_span / BM query tiles of BM rows, which under causal masking
    // end at the sequence's last row, so the first tile starts pad rows
    // before row 0 (sequence bounds clamped as there).
    const int nchunk = row_span / RPB;
    const int bh = blockIdx.x / nchunk;
    const int b = bh / H, h = bh - b * H;
    const int i = (blockIdx.x - bh * nchunk) * RPB + threadIdx.x / LPR;
    const int q0 = min(max(cu_q[b], 0), total_q);
    const int q1 = min(max(cu_q[b + 1], q0), total_q);
    constexpr int BM = 32 * kWaves;
    const int pad = causal ? (BM - (q1 - q0) % BM) % BM : 0;
    if (i >= q1 - q0 || i >= row_span - pad) return;
    row = h * total_q + q0 + i;
    orow = (int64_t)(q0 + i) * H + h;
  } else {
    row = blockIdx.x * RPB + threadIdx.x / LPR;
    if (row >= rows) return;
    orow = row;
  }
  const f32x2* ml = reinterpret_cast<const f32x2*>(part_ml) + (int64_t)row * S;
  const f32x4* pa = reinterpret_cast<const f32x4*>(part + (int64_t)row * S * D) + lr;
  float M = kNegInf, L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += G) {
    f32x2 st[G];
    f32x4 x[G];
    // Past the last split the loads repeat it (no branches between the
    // loads) and its maximum is masked out, so its weight is 0.
  #pragma unroll
    for (int j = 0; j < G; ++j) {
      const int sj = min(s0 + j, S - 1);
      st[j] = ml[sj];
      if (s0 + j >= S) st[j][0] = kNegInf;
      x[j] = pa[sj * LPR];
    }
    float mg = M;
  #pragma unroll
    for (int j = 0; j < G; ++j) mg = fmaxf(mg, st[j][0]);
    if (mg == kNegInf) continue;  // no visible key in any split so far
    const float r = exp2_hw(M - mg);  // 0 while M = -inf (L and acc are 0)
    L *= r;
    acc *= r;
  #pragma unroll
    for (int j = 0; j < G; ++j) {
      const float w = exp2_hw(st[j][0] - mg);  // 0 for a split with no visible key
      L += w * st[j][1];
      acc += w * x[j];
    }
    M = mg;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<f32x4*>(out + orow * D + 4 * lr) = acc * inv;
  } else {
    T o[4];
  #pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = from_f32<T>(acc[j] * inv);
    u32x2 bits;
    __builtin_memcpy(&bits, o, sizeof(bits));
    *reinterpret_cast<u32x2*>(out + orow * D + 4 * lr) = bits;
  }
  if (lr == 0) {
    if (m_out) m_out[row] = M * kLn2;
    if (l_out) l_out[row] = L;
  }
}

template <typename T, int D>
hipError_t launch_splitkv_d(const Problem& p) {
  hipError_t e;
  if constexpr (sizeof(T) == 4)
    e = launch_prefill_f32_partials(p);  // prefill_f32.hip
  else if (p.cu_q)
    e = p.causal ? launch_typed<T, D, kWaves, true, kModeVarlenSplitKv>(p)
                 : launch_typed<T, D, kWaves, false, kModeVarlenSplitKv>(p);
  else
    e = p.causal ? launch_typed<T, D, kWaves, true, kModeSplitKv>(p)
                 : launch_typed<T, D, kWaves, false, kModeSplitKv>(p);
  if (e != hipSuccess) return e;
  const int64_t rows = p.cu_q ? p.H * p.total_q : p.B * p.H * p.Nq;
  // Packed: rows of each (sequence, head) up to the split kernel's tiles.
  const int span = (int)((p.Nq + 32 * kWaves - 1) / (32 * kWaves) * (32 * kWaves));
  constexpr int RPB = kCombineThreads / (D / 4);
  const dim3 grid((unsigned)(p.cu_q ? p.B * p.H * (span / RPB) : (rows + RPB - 1) / RPB));
  const float* ml = p.part + rows * p.splits * D;
  T* o = static_cast<T*>(p.o);
  // Groups no larger than the splits (a group past the last split repeats
  // its loads): 4, 8 or 16.
  auto launch = [&](auto group) {
    constexpr int G = decltype(group)::value;
    hipLaunchKernelGGL((splitkv_combine_kernel<T, D, G>), grid, dim3(kCombineThreads), 0, p.stream,
                       p.part, ml, o, p.m_out, p.l_out, (int)rows, (int)p.splits, p.cu_q,
                       (int)p.H, (int)p.total_q, span, p.causal ? 1 : 0);
  };
  if (p.splits <= 4)
    launch(std::integral_constant<int, 4>{});
  else if (p.splits <= 8)
    launch(std::integral_constant<int, 8>{});
  else
    launch(std::integral_constant<int, 16>{});
  return hipGetLastError();
}

template <typename T>
hipError_t launch_splitkv_t(const Problem& p) {
  switch (p.D) {
    case 16: return launch_splitkv_d<T, 16>(p);
    case 32: return launch_splitkv_d<T, 32>(p);
    case 64: return launch_splitkv_d<T, 64>(p);
    case 128: return launch_splitkv_d<T, 128>(p);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool plan_prefill_splitkv(const Problem& p, SplitKvPlan* plan) {
  if (p.dtype == DType::F32) return plan_prefill_f32_splitkv(p, plan);  // prefill_f32.hip
  // Query tiles of the eight-wave kernel (no causal pairing here) and key
  // tiles: few query tiles over many keys cannot fill the GPU by rows, so
  // their keys are split over workgroups, for about one workgroup per CU.
  // Packed sequences: the host does not read the sequence lengths, so the
  // plan takes every sequence as long as the longest query sequence over
  // total_k keys (exact for one sequence); splits past a shorter sequence's
  // keys write empty states.
  const bool packed = p.cu_q != nullptr;
  const int64_t nk = packed ? p.total_k : p.Nk;
  const int64_t nqt = (p.Nq + 32 * kWaves - 1) / (32 * kWaves);
  const int64_t wq = p.B * p.H * nqt;
  const int64_t kt = (nk + kBN - 1) / kBN;
  if (wq > SPLITKV_MAX_WQ || kt < SPLITKV_MIN_KEY_TILES) return false;
  int64_t S = (SPLITKV_TARGET_WGS + wq - 1) / wq;
  // Splits of at least 16 key tiles; half that when the 16-tile splits
  // would fill fewer than half the CUs (B1 H4 Nq256 Nk8192 D64 causal 24.3
  // -> 19.0 us, B2 H1 Nq300 Nk12000 D128 37.1 -> 28.0 us; with shorter
  // splits on every shape, B2 H4 N2048 D16 went 10.3 -> 14.2 us).
  int64_t cap = kt / SPLITKV_MIN_TILES;
  if (wq * (S < cap ? S : cap) < kNumCUs / 2) cap = kt / (SPLITKV_MIN_TILES / 2);
  if (S > cap) S = cap;
  if (S < 2) return false;
  const int64_t kpt = (kt + S - 1) / S;
  S = (kt + kpt - 1) / kpt;
  // Rows x keys streamed by the busiest CU, here (padding rows of the
  // 256-row tiles included) and on the route launch_prefill_mfma takes
  // otherwise: the key-split kernel (batched layout), one four-wave
  // workgroup per 32-row block over all keys, or four-wave tiled workgroups
  // of 128 rows (two tiles each when causal): packed sequences, and D = 128
  // with 64 eight-wave workgroups.
  // Split keys when that load is lower or equal: the tiled kernel runs two
  // waves per SIMD where the key-split kernel runs one, which pays for the
  // partial states and their combine (equal loads: B1 H32 Nq512 Nk8192 D128
  // causal 126 -> 73 us, B1 H32 Nq256 Nk16384 D64 causal 63 -> 49 us, B1 H4
  // N4096 D64 causal 36.6 -> 30.6 us, B1 H8 Nq1024 Nk8192 D64 34.1 -> 33.6
  // us; lower loads: B1 H8 Nq512 Nk16384 D128 causal 117 -> 52 us, B1 H1
  // Nq512 Nk65536 D64 causal 227 -> 31 us).  Higher loads lose (B4 H8 Nq256
  // Nk4096 D128 causal 37 -> 44 us, B2 H8 Nq512 Nk4096 D64 causal 20 -> 34
  // us, the latter before the combine and the scratch were made faster).
  auto per_cu = [](int64_t wgs) { return (wgs + kNumCUs - 1) / kNumCUs; };
  const int64_t bh = p.B * p.H;
  const int64_t w8 = bh * (p.causal ? (nqt + 1) / 2 : nqt);
  const int64_t small = p.D > 64 ? kSmallGridWgs<128> : kSmallGridWgs<64>;
  int64_t other;
  if (!packed && w8 <= small) {
    other = per_cu(bh * ((p.Nq + 31) / 32)) * 32 * nk;
  } else {
    const int64_t nqt4 = (p.Nq + 127) / 128;
    const bool pair = p.causal && nqt4 > 1;
    other = per_cu(bh * (p.causal ? (nqt4 + 1) / 2 : nqt4)) * (pair ? 256 : 128) * nk;
  }
  const int64_t mine = per_cu(wq * S) * 32 * kWaves * kpt * kBN;
  if (mine > other) return false;
  plan->splits = S;
  plan->split_tiles = kpt;
  const int64_t rows = packed ? p.H * p.total_q : p.B * p.H * p.Nq;
  plan->scratch_bytes = (size_t)rows * (size_t)S * (size_t)(p.D + 2) * sizeof(float);
  return true;
}

hipError_t launch_prefill_splitkv(const Problem& p) {
  if (p.dtype == DType::BF16) return launch_splitkv_t<__bf16>(p);
  if (p.dtype == DType::F16) return launch_splitkv_t<_Float16>(p);
  return launch_splitkv_t<float>(p);
}

hipError_t launch_prefill_mfma(const Problem& p) {
  if (p.dtype == DType::BF16) return launch_t<__bf16>(p);
  if (p.dtype == DType::F16) return launch_t<_Float16>(p);
  return hipErrorInvalidValue;
}

}  // namespace attn
