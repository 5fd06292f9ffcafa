// Split-key decode with grouped K/V heads on the matrix cores (bf16 / f16):
// the partial-state kernel of the decode path for G = H / Hkv > 1, over
// contiguous K/V or a paged cache, with an optional sliding window.
//
// With grouped heads the G query heads of a K/V head read the same keys.
// Streaming them row by row (the vector-ALU partial kernel in
// decode_splitk.hip) reads every K/V byte G * Nq times.  Here the G * Nq
// query rows that share a K/V head are packed, 32 at a time, into the 32
// columns of one matrix tile (packed row r = g * Nq + i is query head
// h0 + g, query i; chunk z of a group holds rows 32z .. 32z + 31, lane l32
// row 32z + l32), so each K/V tile is read once per chunk, ceil(G * Nq / 32)
// times in all, and feeds S = K Q^T and O += P V on the matrix cores.
// Work item (b, K/V head, split s) with row chunk z covers
// keys [kbeg + s * kps, kbeg + (s + 1) * kps) (kbeg = 0 unless a sliding
// window hides the first keys from every row); its KS waves take the 64-key tiles of that
// range in turn through their own double-buffered LDS tiles, keep the
// running state of the streaming method per row (answer-key page, row A3),
// merge their states in LDS (row A1) and write the split's (m, l, a) per
// query row to the scratch array the decode path's combine kernel folds
// (same layout: [row][S][D + 2], m in base-2 units relative to the exact
// maximum of the split).
//
// Paged cache [num_pages, Hkv, page_size, D]: each 16-byte load instruction
// of a tile moves 512 / D consecutive rows, and with page_size >= 512 / D
// (both powers of two) those rows sit in one page.  Each instruction then
// gets a buffer descriptor of its own over that page's rows of this K/V
// head, so all per-lane offsets stay 32-bit however large the cache is;
// rows past the sequence's length are outside the descriptor's range and
// arrive as zeros, and a table entry outside [0, num_pages) gives an empty
// range and marks its keys absent (masked like keys past the end).  The
// table is read only for keys below the sequence's length.
//
// Sliding window (causal): row i sees keys j with i + off - window < j <=
// i + off.  The splits cover keys from the lowest such bound over the
// group's rows, rounded down to a tile boundary.

#include <cstdint>
#include <type_traits>

#include "attn_kernels.h"
#include "attn_mfma.h"

namespace attn {
namespace {

struct GqaArgs {
  const void* q;
  const void* k;
  const void* v;
  float* part;  // [rows][S][D + 2]
  int H, Hkv, G, Nq, Nk;
  int S;        // splits per row
  int kps;      // keys per split (a multiple of 64)
  int chunks;   // ceil(G * Nq / 32) row chunks per K/V head
  int nwork;    // B * Hkv * S work items
  float c;      // scale * log2(e)
  int window;   // 0: none
  // Paged cache (PAGED kernels only): sequence b's key j is row j % page_size
  // of page table[b * max_pages + j / page_size]; lens[b] keys.
  const int* table;
  const int* lens;
  int max_pages;
  int page_shift;  // log2(page_size)
  int num_pages;
};

constexpr int kBN = 64;
constexpr int kKPF = 4;
constexpr int kVPF = 4;
constexpr float kRefreshGap = 8.0f;  // base-2 units, as in prefill_mfma.hip

template <int D>
constexpr int kWaves = D > 64 ? 2 : 4;  // per-wave double-buffered tiles fit in LDS

// Rows of one all-zero 16-byte chunk: the source of the per-row paged loads
// for keys past the sequence's length or in absent pages.
__device__ uint4 g_zero_chunk = {0u, 0u, 0u, 0u};  // never written

template <typename T, int D, bool CAUSAL, bool PAGED, bool ROWPAGE>
__global__ __launch_bounds__(kWaves<D> * 64) void decode_gqa_kernel(GqaArgs a) {
  typedef typename Mfma<T>::vec8 vec8;
  typedef typename Mfma<T>::vec2 vec2;
  typedef Geo<D> G_;
  constexpr int KS = kWaves<D>;
  constexpr int BN = kBN;
  constexpr int DP = D < 32 ? 32 : D;
  constexpr int KC = D / 16;
  constexpr int NB = DP / 32;
  constexpr int TILE = BN * D * 2;
  constexpr int NSLOT = TILE / 16;
  constexpr int NREG = 16 * NB;
  static_assert(G_::steps_keep_swizzle(), "tile steps must keep the LDS swizzle");
  static_assert(NSLOT % 64 == 0, "a wave moves whole 1 KB LDS blocks");
  constexpr int RPU = 64 / G_::CPR;  // rows moved by one load instruction

  __shared__ __attribute__((aligned(1024))) unsigned char buf0[KS][2][TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char buf1[KS][2][TILE];
  __shared__ float mrg[KS - 1][NREG + 3][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  auto tile_ptr = [&](int buf, int kv) __attribute__((always_inline)) -> unsigned char* {
    return buf == 0 ? &buf0[wave][kv][0] : &buf1[wave][kv][0];
  };

  // Block -> work item w = (b * Hkv + K/V head) * S + split and row chunk
  // z.  Blocks are dealt to the 8 XCDs round-robin; the chunks of one work
  // item are 8 blocks apart, so they run on one XCD close together in time
  // and the later ones find the K/V tiles in that XCD's L2.
  const int blk = blockIdx.x;
  const int xcd = blk & 7;
  const int r8 = blk >> 3;
  const int chunk = r8 % a.chunks;  // 32 packed rows of the group
  const int w = (r8 / a.chunks) * 8 + xcd;
  if (w >= a.nwork) return;
  const int split = w % a.S;
  const int bk = w / a.S;  // b * Hkv + K/V head
  const int b = bk / a.Hkv, hk = bk - b * a.Hkv;
  const int Nq = a.Nq;
  int Nk = a.Nk;
  const int* trow = nullptr;
  if (PAGED) {
    trow = a.table + (int64_t)b * a.max_pages;
    Nk = min(max(a.lens[b], 0), a.max_pages << a.page_shift);
  }
  const int off = Nk - Nq;
  const int h32 = lane >> 5;
  const int l32 = lane & 31;
  // Packed row of this lane: query head hk*G + g, query row i.
  const int R = a.G * Nq;
  const int pr = chunk * 32 + l32;
  const bool real = pr < R;
  const int g = real ? pr / Nq : 0;
  const int qi = real ? pr - g * Nq : 0;
  const int64_t qrow = ((int64_t)b * a.H + (int64_t)hk * a.G + g) * Nq + qi;  // row of [B, H, Nq]
  const T* Kh = static_cast<const T*>(a.k) + (PAGED ? 0 : (int64_t)bk * Nk * D);
  const T* Vh = static_cast<const T*>(a.v) + (PAGED ? 0 : (int64_t)bk * Nk * D);
  const float c = a.c;

  vec8 qf[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    qf[kc] = real ? *reinterpret_cast<const vec8*>(static_cast<const T*>(a.q) + qrow * D + kc * 16 + h32 * 8)
                  : vec8{};
  }

  // Keys below every row's window are skipped: the splits start at the
  // lowest visible key of the group (row 0's bound), on a tile boundary.
  const int win = a.window;
  const int kbeg = win > 0 ? max(0, off - win + 1) & ~(BN - 1) : 0;
  const int k0 = kbeg + split * a.kps;
  const int k1 = min(Nk, k0 + a.kps);
  const int t0 = k0 / BN;
  const int t1 = k1 > k0 ? (k1 + BN - 1) / BN : t0;  // tiles [t0, t1) of this split

  const uint32_t kpitch = (uint32_t)(2 * D);
  // Contiguous K/V: one descriptor over the head (fewer than 2^31 elements,
  // so its byte size fits 32 bits); rows past Nk read as zeros.
  const uint32_t kv_bytes = PAGED ? 0u : (uint32_t)Nk * (uint32_t)(2 * D);
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(Kh), 0, (int)kv_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(Vh), 0, (int)kv_bytes, 0x00020000);

  int koff[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) koff[kc] = G_::off(l32, 2 * kc + h32);
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
        voff[nb][half] = G_::off(row, col >> 3) + ((col & 7) << 1);
      }
    }
  }

  float m_run = kNegInf, m_true = kNegInf, l_run = 0.f;
  f32x16 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x16{};

  // Paged: lane u holds the physical page of the rows that load instruction
  // u of a tile moves (-1 past the sequence's length), fetched a step before
  // the tile's loads need it.
  constexpr int NU = NSLOT / 64;  // load instructions per tile and K or V
  const int pshift = a.page_shift;
  // Pages smaller than RPU rows (ROWPAGE): lane i holds the page of row i
  // of the tile instead.
  auto fetch_pages = [&](int t) __attribute__((always_inline)) -> int {
    if (!PAGED || t >= t1) return -1;
    const int j = ROWPAGE ? t * BN + lane : t * BN + lane * RPU;
    return (ROWPAGE || lane < NU) && j < Nk ? trow[j >> pshift] : -1;
  };
  // Per tile buffer, the rows whose page is absent (bit r = row r of the
  // tile); rows past the sequence's length are handled by the length.
  uint64_t absent0 = 0, absent1 = 0;
  auto load_tile = [&](int t, auto bufc, int pv) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    if (PAGED && ROWPAGE) {
      // Every lane addresses its own row (any page size): 64-bit addresses,
      // global loads straight into LDS; rows past the length or in absent
      // pages read the zero chunk.  Bit i of the absent set is row i.
      const int ji = t * BN + lane;
      const bool present_i = pv >= 0 && pv < a.num_pages;
      const uint64_t absent = __builtin_amdgcn_ballot_w64(ji < Nk && !present_i);
      const unsigned char* kb = reinterpret_cast<const unsigned char*>(Kh);
      const unsigned char* vb = reinterpret_cast<const unsigned char*>(Vh);
      const unsigned char* zero = reinterpret_cast<const unsigned char*>(&g_zero_chunk);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int sl = lane + u * 64;
        const int row = sl / G_::CPR;
        const int chunk = (sl % G_::CPR) ^ G_::swz(row);
        const int pg = __shfl(pv, row);
        const int j = t * BN + row;
        const bool ok = j < Nk && pg >= 0 && pg < a.num_pages;
        const uint64_t off =
            ok ? (uint64_t)((((int64_t)pg * a.Hkv + hk) << pshift) + (j & ((1 << pshift) - 1))) *
                         (uint64_t)(2 * D) +
                     (uint64_t)(chunk << 4)
               : 0u;
        __builtin_amdgcn_global_load_lds(
            (__attribute__((address_space(1))) void*)(ok ? kb + off : zero),
            LDS_PTR(void, tile_ptr(buf, 0) + u * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(
            (__attribute__((address_space(1))) void*)(ok ? vb + off : zero),
            LDS_PTR(void, tile_ptr(buf, 1) + u * 1024), 16, 0, 0);
      }
      if (buf == 0) absent0 = absent; else absent1 = absent;
      return;
    }
    if (PAGED) {
      // Lane u works out instruction u's rows (one page: page_size >= RPU),
      // its byte offset in the cache and how many of its rows exist; each
      // instruction then reads them back as scalars for its descriptor.
      const int ju = t * BN + lane * RPU;
      const bool inside = lane < NU && ju < Nk;
      const bool ok = inside && pv >= 0 && pv < a.num_pages;
      const uint32_t bytes_u = ok ? (uint32_t)min(Nk - ju, RPU) * kpitch : 0u;
      const uint64_t off_u =
          ok ? (uint64_t)(((((int64_t)pv * a.Hkv + hk) << pshift) + (ju & ((1 << pshift) - 1))) * D) * 2u
             : 0u;
      const uint64_t absent_u = __builtin_amdgcn_ballot_w64(inside && !ok);
      uint64_t absent = 0;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)off_u, u);
        const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(off_u >> 32), u);
        const uint32_t bytes = __builtin_amdgcn_readlane(bytes_u, u);
        const uint64_t off = ((uint64_t)hi << 32) | lo;
        if ((absent_u >> u) & 1ull) absent |= ((1ull << RPU) - 1) << (u * RPU);
        const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<unsigned char*>(reinterpret_cast<const unsigned char*>(Kh) + off), 0, (int)bytes,
            0x00020000);
        const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<unsigned char*>(reinterpret_cast<const unsigned char*>(Vh) + off), 0, (int)bytes,
            0x00020000);
        const int sl = lane + u * 64;
        const int row = sl / G_::CPR;
        const int chunk = (sl % G_::CPR) ^ G_::swz(row);
        const int vo = (int)((uint32_t)(row - u * RPU) * kpitch + (uint32_t)(chunk << 4));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, LDS_PTR(void, tile_ptr(buf, 0) + u * 1024), 16,
                                                 vo, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, LDS_PTR(void, tile_ptr(buf, 1) + u * 1024), 16,
                                                 vo, 0, 0, 0);
      }
      if (buf == 0) absent0 = absent; else absent1 = absent;
      return;
    }
#pragma unroll
    for (int u = 0; u < NSLOT / 64; ++u) {
      const int sl = lane + u * 64;
      const int row = sl / G_::CPR;
      const int chunk = (sl % G_::CPR) ^ G_::swz(row);
      const int j = min(t * BN + row, Nk);
      const int vo = (int)((uint32_t)j * kpitch + (uint32_t)(chunk << 4));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, LDS_PTR(void, tile_ptr(buf, 0) + u * 1024), 16,
                                               vo, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, LDS_PTR(void, tile_ptr(buf, 1) + u * 1024), 16,
                                               vo, 0, 0, 0);
    }
  };

  // One 64-key tile: the split's keys past k1 (and Nk), when causal keys
  // past the row's diagonal, keys below the row's window and keys of absent
  // pages are masked.
  auto compute = [&](auto bufc, int j0) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    const uint64_t absent = PAGED ? (buf == 0 ? absent0 : absent1) : 0;
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

    if ((j0 + BN > k1) || (CAUSAL && j0 + BN - 1 > off) || (win > 0 && j0 <= Nq - 1 + off - win) ||
        (PAGED && absent != 0)) {
      // Register r of block mb holds key j0 + 4*h32 + kr, kr = 32mb + 8(r/4) + r%4:
      // visible iff wlo < kr < lim and its page is present.
      const int lim = min(k1 - j0, CAUSAL ? qi + off - j0 + 1 : k1 - j0) - 4 * h32;
      const int wlo = win > 0 ? qi + off - win - j0 - 4 * h32 : -(1 << 30);
      const uint64_t present = ~(absent >> (4 * h32));
#pragma unroll
      for (int mb = 0; mb < BN / 32; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kr = mb * 32 + (r >> 2) * 8 + (r & 3);
          bool vis = kr < lim && kr > wlo;
          if (PAGED) vis = vis && ((present >> kr) & 1ull);
          s[mb][r] = vis ? s[mb][r] : kNegInf;
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

  // This wave's tiles: t0 + wave, t0 + wave + KS, ...  Each step ends by
  // waiting for its own loads, so the next step's reads never wait on the
  // tile it puts in flight.
  constexpr int kWaitLoads = 0x0F70;  // s_waitcnt vmcnt(0)
  // Paged: the page entries of the next tile to load are fetched one step
  // ahead and arrive with that step's wait.
  if (t0 + wave < t1) {
    int pv = fetch_pages(t0 + wave);
    load_tile(t0 + wave, std::integral_constant<int, 0>{}, pv);
    pv = fetch_pages(t0 + wave + KS);
    __builtin_amdgcn_s_waitcnt(kWaitLoads);
    for (int t = t0 + wave; t < t1; t += 2 * KS) {
      if (t + KS < t1) load_tile(t + KS, std::integral_constant<int, 1>{}, pv);
      pv = fetch_pages(t + 2 * KS);
      compute(std::integral_constant<int, 0>{}, t * BN);
      __builtin_amdgcn_s_waitcnt(kWaitLoads);
      if (t + KS < t1) {
        if (t + 2 * KS < t1) load_tile(t + 2 * KS, std::integral_constant<int, 0>{}, pv);
        pv = fetch_pages(t + 3 * KS);
        compute(std::integral_constant<int, 1>{}, (t + KS) * BN);
        __builtin_amdgcn_s_waitcnt(kWaitLoads);
      }
    }
  }

  // Merge the waves' states (answer-key row A1), then write the split's
  // state per real row relative to its exact maximum.
  const float l_tot = half_sum(l_run);
  if (wave > 0) {
    float* dst = &mrg[wave - 1][0][0];
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
  for (int w = 1; w < KS; ++w) M = fmaxf(M, mrg[w - 1][NREG][lane]);
  const float ref = pinned_ref(M);
  const float w0 = exp2_hw(m_run - ref);
  float L = l_tot * w0;
  float mt = m_true;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] *= w0;
#pragma unroll
  for (int w = 1; w < KS; ++w) {
    const float* src = &mrg[w - 1][0][0];
    const float ws = exp2_hw(src[NREG * 64 + lane] - ref);
    L = __builtin_fmaf(src[(NREG + 1) * 64 + lane], ws, L);
    mt = fmaxf(mt, src[(NREG + 2) * 64 + lane]);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nb][r] = __builtin_fmaf(src[(nb * 16 + r) * 64 + lane], ws, acc[nb][r]);
  }
  if (real) {
    // Relative to the exact maximum mt (the lagging reference is at most
    // kRefreshGap below it); an empty split is (-inf, 0, 0).
    const float f = mt == kNegInf ? 0.f : exp2_hw(ref - mt);
    float* dst = a.part + (qrow * a.S + split) * (D + 2);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int d0 = nb * 32 + gg * 8 + h32 * 4;
        if (d0 < D) {
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[2 + d0 + e] = acc[nb][gg * 4 + e] * f;
        }
      }
    if (h32 == 0) {
      dst[0] = mt;
      dst[1] = L * f;
    }
  }
}

template <typename T, int D, bool CAUSAL, bool PAGED, bool ROWPAGE>
hipError_t launch_typed(const Problem& p, const DecodePlan& plan, float* scratch) {
  GqaArgs a;
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.part = scratch;
  a.H = (int)p.H;
  a.Hkv = (int)p.Hkv;
  a.G = (int)(p.H / p.Hkv);
  a.Nq = (int)p.Nq;
  a.Nk = (int)p.Nk;
  a.S = plan.splits;
  a.kps = plan.keys_per_split;
  a.c = p.scale * kLog2e;
  a.window = (int)p.window;
  a.table = p.table;
  a.lens = p.lens;
  a.max_pages = (int)p.max_pages;
  a.page_shift = 0;
  while ((int64_t(1) << a.page_shift) < p.page_size) ++a.page_shift;
  // Entries at or past 2^31 pages cannot be stored in the int32 table.
  a.num_pages = (int)(p.num_pages < INT32_MAX ? p.num_pages : INT32_MAX);
  a.chunks = (int)((a.G * p.Nq + 31) / 32);
  a.nwork = (int)(p.B * p.Hkv * plan.splits);
  const int64_t blocks = (int64_t)(a.nwork + 7) / 8 * 8 * a.chunks;
  hipLaunchKernelGGL((decode_gqa_kernel<T, D, CAUSAL, PAGED, ROWPAGE>), dim3((unsigned)blocks),
                     dim3(kWaves<D> * 64), 0, p.stream, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const Problem& p, const DecodePlan& plan, float* scratch) {
  // Pages of at least the RPU = 512 / D rows one load instruction moves get
  // one descriptor per instruction; smaller pages, per-row addresses.
  if (p.table && p.page_size < 512 / D)
    return p.causal ? launch_typed<T, D, true, true, true>(p, plan, scratch)
                    : launch_typed<T, D, false, true, true>(p, plan, scratch);
  if (p.table)
    return p.causal ? launch_typed<T, D, true, true, false>(p, plan, scratch)
                    : launch_typed<T, D, false, true, false>(p, plan, scratch);
  return p.causal ? launch_typed<T, D, true, false, false>(p, plan, scratch)
                  : launch_typed<T, D, false, false, false>(p, plan, scratch);
}

template <typename T>
hipError_t launch_t(const Problem& p, const DecodePlan& plan, float* scratch) {
  switch (p.D) {
    case 16: return launch_d<T, 16>(p, plan, scratch);
    case 32: return launch_d<T, 32>(p, plan, scratch);
    case 64: return launch_d<T, 64>(p, plan, scratch);
    case 128: return launch_d<T, 128>(p, plan, scratch);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_gqa_partial(const Problem& p, const DecodePlan& plan, float* scratch) {
  if (p.dtype == DType::BF16) return launch_t<__bf16>(p, plan, scratch);
  if (p.dtype == DType::F16) return launch_t<_Float16>(p, plan, scratch);
  return hipErrorInvalidValue;
}

}  // namespace attn
