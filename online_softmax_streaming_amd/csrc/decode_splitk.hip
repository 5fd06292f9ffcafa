// Split-key decode path: few query rows per head, many keys.
//
// With Nq <= 8 a query tile of the prefill kernels would be mostly ghost
// rows, and one workgroup per (b, h) cannot fill 256 CUs.  Instead each
// query row's keys are cut into S splits.  This follows the wide-row split
// softmax of the workshops page (split_softmax row of "Scope and
// contracts") and its answer-key row A2: partial statistics per chunk, then
// a rescaled merge, ordered by launching both kernels on one stream, with a
// per-call scratch array.
//
//   kernel 1 (partial): workgroup (row, split) streams its keys, carrying
//     (m, l, a) per lane group exactly as the prefill kernels do (answer-key
//     row A3), folds the groups with the A1 merge, and writes the split's
//     state (m, l, a[0..D)) to scratch.  Base-2 units.
//   kernel 2 (combine): workgroup `row` folds the S partial states with the
//     A1 merge (answer-key row A1), normalises and casts once.
//
// The path is bound by HBM bandwidth (each K/V byte is read once and used
// for one multiply-add), so it runs on the vector ALUs: lanes read 16-byte
// chunks, D/VEC lanes cover one key row, and each loop step keeps U rows
// per lane group in flight.
//
// Two key layouts share the kernels: contiguous [B, Hkv, Nk, D], and a paged
// cache [num_pages, Hkv, page_size, D] where an int32 table maps page p of
// sequence b to a physical page and an int32 length gives each sequence's
// key count (a KV-cache slice; the pages plan one for a later week).  A
// sliding window (causal only) keeps the `window` keys ending at the row's
// diagonal; the splits cover only the visible key range of each row.  Table
// entries outside [0, num_pages) are read as absent keys and lengths are
// clamped to [0, max_pages * page_size]: table values are never used to
// address memory outside the cache.

#include <cstdint>

#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {
namespace {

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* m_out;
  float* l_out;
  float* part;  // [rows][S][D + 2]: m, l, a[D]
  int H, Nq, Nk;
  int group;  // query heads per K/V head
  int S;
  int kps;     // keys per split
  int window;  // 0: none; else the visible keys end at the diagonal, at most this many
  float c;     // scale * log2(e)
  // Paged layout (PAGED kernels only).
  const int* table;   // [B, max_pages]
  const int* lens;    // [B]
  int Hkv;
  int max_pages;
  int page_shift;     // log2(page_size)
  int64_t num_pages;
};

constexpr int kThreads = 256;

template <typename T> struct Vec16;
template <> struct Vec16<__bf16> { typedef bf16x8 type; static constexpr int n = 8; };
template <> struct Vec16<_Float16> { typedef f16x8 type; static constexpr int n = 8; };
template <> struct Vec16<float> { typedef f32x4 type; static constexpr int n = 4; };

template <typename T, int D, bool CAUSAL, bool PAGED>
__global__ __launch_bounds__(kThreads) void decode_partial_kernel(DecodeArgs a) {
  typedef typename Vec16<T>::type vec;
  constexpr int VEC = Vec16<T>::n;
  constexpr int LPR = D / VEC;          // lanes per key row
  constexpr int G = kThreads / LPR;     // lane groups per workgroup
  constexpr int U = 4;                  // key rows per group per step

  __shared__ float sm[G], sl[G];
  __shared__ float sa[G * D];

  const int row = blockIdx.x;  // (b*H + h)*Nq + i
  const int split = blockIdx.y;
  const int Nq = a.Nq;
  const int bh = row / Nq;
  const int i = row - bh * Nq;
  const int tid = threadIdx.x;
  const int g = tid / LPR;
  const int sub = tid - g * LPR;
  const float c = a.c;

  // Query head (b, h) reads K/V head (b, h / group): bh / group.
  int Nk = a.Nk;
  const T* __restrict__ Kh;
  const T* __restrict__ Vh;
  const int* trow = nullptr;
  int hk = 0;
  if (PAGED) {
    const int b = bh / a.H;
    hk = (bh - b * a.H) / a.group;
    trow = a.table + (int64_t)b * a.max_pages;
    Nk = min(max(a.lens[b], 0), a.max_pages << a.page_shift);
    Kh = static_cast<const T*>(a.k);
    Vh = static_cast<const T*>(a.v);
  } else {
    Kh = static_cast<const T*>(a.k) + (int64_t)(bh / a.group) * Nk * D;
    Vh = static_cast<const T*>(a.v) + (int64_t)(bh / a.group) * Nk * D;
  }
  float qv[VEC];
  {
    const vec q = *reinterpret_cast<const vec*>(static_cast<const T*>(a.q) + (int64_t)row * D + sub * VEC);
#pragma unroll
    for (int e = 0; e < VEC; ++e) qv[e] = to_f32<T>(q[e]);
  }

  int kend = Nk;
  if (CAUSAL) kend = min(Nk, i + (Nk - Nq) + 1);
  const int kbeg = a.window > 0 ? max(0, i + (Nk - Nq) - a.window + 1) : 0;
  const int kb = kbeg + split * a.kps;
  const int ke = min(kend, kb + a.kps);

  float m_run = kNegInf, l_run = 0.f;
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;

  // Paged: the page indices of a step are fetched one step ahead, so the
  // table read is not in series with the key reads it addresses.
  int pg[U];
  auto fetch_pages = [&](int j) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jj = j + u * G;
      pg[u] = PAGED && jj < ke ? trow[jj >> a.page_shift] : 0;
    }
  };
  if (PAGED) fetch_pages(kb + g);
  for (int j = kb + g; j < ke; j += G * U) {
    vec kv[U], vv[U];
    bool in[U];
    int cur[U];
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = pg[u];
    if (PAGED) fetch_pages(j + G * U);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jj = j + u * G;
      int64_t ko = -1;
      if (jj < ke) {
        if (!PAGED) {
          ko = (int64_t)jj * D;
        } else if (cur[u] >= 0 && cur[u] < a.num_pages) {
          const int r = jj & ((1 << a.page_shift) - 1);
          ko = ((((int64_t)cur[u] * a.Hkv + hk) << a.page_shift) + r) * D;
        }
      }
      in[u] = ko >= 0;
      kv[u] = in[u] ? *reinterpret_cast<const vec*>(Kh + ko + sub * VEC) : vec{};
      vv[u] = in[u] ? *reinterpret_cast<const vec*>(Vh + ko + sub * VEC) : vec{};
    }
    float s[U];
    float mx = kNegInf;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) dot = __builtin_fmaf(qv[e], to_f32<T>(kv[u][e]), dot);
#pragma unroll
      for (int o = LPR / 2; o >= 1; o >>= 1) dot += __shfl_xor(dot, o);
      // Rounded product kept apart from the later subtraction, so the
      // largest score gives exactly 2^0 = 1.
      s[u] = in[u] ? dot * c : kNegInf;
      mx = fmaxf(mx, s[u]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float ref = pinned_ref(m_new);
    const float alpha = exp2_hw(m_run - ref);
    float rs = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      s[u] = exp2_hw(s[u] - ref);
      rs += s[u];
    }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float x = acc[e] * alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) x = __builtin_fmaf(s[u], to_f32<T>(vv[u][e]), x);
      acc[e] = x;
    }
    m_run = m_new;
  }

  // Fold the G lane-group states of this workgroup (A1 merge).
  if (sub == 0) {
    sm[g] = m_run;
    sl[g] = l_run;
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) sa[g * D + sub * VEC + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float M = kNegInf, L = 0.f, A = 0.f;
    for (int gg = 0; gg < G; ++gg) {
      const MergeWeights w = merge_weights_log2(M, sm[gg]);
      L = L * w.w1 + sl[gg] * w.w2;
      A = A * w.w1 + sa[gg * D + tid] * w.w2;
      M = w.m;
    }
    float* dst = a.part + ((int64_t)row * a.S + split) * (D + 2);
    dst[2 + tid] = A;
    if (tid == 0) {
      dst[0] = M;
      dst[1] = L;
    }
  }
}

// Folds the S split states of each row into out and (m, l), merge A1 over
// groups of G splits: a group's states are loaded at once (one round
// of memory latency per group), then weighted by 2^(m_s - M) against the
// exact maximum M so far, the running sums rescaled when M grows.  D / 2
// lanes per row, two features per lane (8-byte loads: a split's a[D] starts
// 8 bytes into its D + 2 floats).
constexpr int kCombineThreads = 256;

template <typename T, int D, int G>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(DecodeArgs a, int rows) {
  constexpr int LPR = D / 2;
  constexpr int RPB = kCombineThreads / LPR;
  const int lr = threadIdx.x % LPR;
  const int row = blockIdx.x * RPB + threadIdx.x / LPR;
  if (row >= rows) return;
  const float* src = a.part + (int64_t)row * a.S * (D + 2);
  float M = kNegInf, L = 0.f;
  f32x2 acc = {0.f, 0.f};
  for (int s0 = 0; s0 < a.S; s0 += G) {
    float m[G], l[G];
    f32x2 x[G];
    // Past the last split the loads repeat it (no branches between the
    // loads) and its maximum is masked out; its weight below is 0.
  #pragma unroll
    for (int j = 0; j < G; ++j) {
      const float* st = src + min(s0 + j, a.S - 1) * (D + 2);
      m[j] = s0 + j < a.S ? st[0] : kNegInf;
      l[j] = st[1];
      x[j] = *reinterpret_cast<const f32x2*>(st + 2 + 2 * lr);
    }
    float mg = M;
  #pragma unroll
    for (int j = 0; j < G; ++j) mg = fmaxf(mg, m[j]);
    if (mg == kNegInf) continue;  // no visible key in any split so far
    const float r = exp2_hw(M - mg);  // 0 while M = -inf (L and acc are 0)
    L *= r;
    acc *= r;
  #pragma unroll
    for (int j = 0; j < G; ++j) {
      const float w = exp2_hw(m[j] - mg);  // 0 for a split with no visible key
      L += w * l[j];
      acc += w * x[j];
    }
    M = mg;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  T* orow = static_cast<T*>(a.o) + (int64_t)row * D + 2 * lr;
  orow[0] = from_f32<T>(acc[0] * inv);
  orow[1] = from_f32<T>(acc[1] * inv);
  if (lr == 0) {
    if (a.m_out) a.m_out[row] = M * kLn2;
    if (a.l_out) a.l_out[row] = L;
  }
}

template <typename T, int D, bool CAUSAL, bool PAGED>
hipError_t launch_typed(const Problem& p, const DecodePlan& plan, float* scratch) {
  DecodeArgs a;
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.o = p.o;
  a.m_out = p.m_out;
  a.l_out = p.l_out;
  a.part = scratch;
  a.H = (int)p.H;
  a.group = (int)(p.H / p.Hkv);
  a.Nq = (int)p.Nq;
  a.Nk = (int)p.Nk;
  a.S = plan.splits;
  a.kps = plan.keys_per_split;
  a.window = (int)p.window;
  a.c = p.scale * kLog2e;
  a.table = p.table;
  a.lens = p.lens;
  a.Hkv = (int)p.Hkv;
  a.max_pages = (int)p.max_pages;
  a.page_shift = 0;
  while ((int64_t(1) << a.page_shift) < p.page_size) ++a.page_shift;
  a.num_pages = p.num_pages;
  const int64_t rows = p.B * p.H * p.Nq;
  hipError_t e;
  if (plan.gqa_mfma) {
    e = launch_decode_gqa_partial(p, plan, scratch);  // decode_gqa.hip
  } else {
    hipLaunchKernelGGL((decode_partial_kernel<T, D, CAUSAL, PAGED>), dim3((unsigned)rows, plan.splits),
                       dim3(kThreads), 0, p.stream, a);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  constexpr int RPB = kCombineThreads / (D / 2);
  const dim3 grid((unsigned)((rows + RPB - 1) / RPB));
  // Groups no larger than the splits (a group past the last split repeats
  // its loads): 4, 8 or 16.
  if (plan.splits <= 4)
    hipLaunchKernelGGL((decode_combine_kernel<T, D, 4>), grid, dim3(kCombineThreads), 0, p.stream,
                       a, (int)rows);
  else if (plan.splits <= 8)
    hipLaunchKernelGGL((decode_combine_kernel<T, D, 8>), grid, dim3(kCombineThreads), 0, p.stream,
                       a, (int)rows);
  else
    hipLaunchKernelGGL((decode_combine_kernel<T, D, 16>), grid, dim3(kCombineThreads), 0, p.stream,
                       a, (int)rows);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const Problem& p, const DecodePlan& plan, float* scratch) {
  if (p.table)
    return p.causal ? launch_typed<T, D, true, true>(p, plan, scratch)
                    : launch_typed<T, D, false, true>(p, plan, scratch);
  return p.causal ? launch_typed<T, D, true, false>(p, plan, scratch)
                  : launch_typed<T, D, false, false>(p, plan, scratch);
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

// Two or more query rows per K/V head (grouped heads, or Nq > 1), bf16/f16,
// any page size: the partial states come from the matrix-core kernel of
// decode_gqa.hip, which reads each K/V tile once per 32 of the G * Nq query
// rows of a K/V head.  Its workgroups are (b, K/V head, split, chunk of 32
// rows): aim for ATTN_GQA_WANT_WGS of them with >= 2 tiles per wave in each
// split.  The splits cover the longest key range a K/V head's rows can need:
// the whole sequence, or with a window the keys from row 0's lower bound
// (rounded down to a 64-key tile) to the end.
static bool decode_gqa_eligible(const Problem& p) {
  if (p.dtype != DType::BF16 && p.dtype != DType::F16) return false;
  // One row per K/V head (plain decode) streams its keys on the vector
  // ALUs at the HBM rate; two or more rows share the matrix tiles.
  if (p.Hkv <= 0 || (p.H / p.Hkv) * p.Nq <= 1) return false;
  return true;
}

// Workgroups the grouped decode plan aims for: one per CU (a workgroup's
// double-buffered tiles take most of a CU's LDS, so 256 run as one round
// with no tail; 512, 768 and 1024 measured up to 40 % slower); a build-time
// knob.
#ifndef ATTN_GQA_WANT_WGS
#define ATTN_GQA_WANT_WGS 256
#endif

static DecodePlan plan_decode_gqa(const Problem& p, int64_t max_splits) {
  const int64_t kv_rows = p.B * p.Hkv * (((p.H / p.Hkv) * p.Nq + 31) / 32);
  const int64_t waves = p.D > 64 ? 2 : 4;
  int64_t range = p.table ? p.max_pages * p.page_size : p.Nk;
  if (p.window > 0 && p.window + p.Nq + 62 < range) range = p.window + p.Nq + 62;
  const int64_t want = (ATTN_GQA_WANT_WGS + kv_rows - 1) / kv_rows;
  int64_t kps = (range + want - 1) / want;
  const int64_t min_kps = 64 * waves * 2;
  if (kps < min_kps) kps = min_kps;
  kps = (kps + 63) / 64 * 64;
  int64_t splits = (range + kps - 1) / kps;
  if (splits < 1) splits = 1;
  if (splits > max_splits) {
    splits = max_splits;
    kps = ((range + splits - 1) / splits + 63) / 64 * 64;
    splits = (range + kps - 1) / kps;
    if (splits < 1) splits = 1;
  }
  DecodePlan plan;
  plan.splits = (int)splits;
  plan.keys_per_split = (int)kps;
  plan.scratch_bytes = (size_t)(p.B * p.H * p.Nq) * (size_t)splits * (size_t)(p.D + 2) * sizeof(float);
  plan.gqa_mfma = true;
  return plan;
}

// Measured at B16 H32 D128 bf16 over 32768 keys: 16 / 32 rows per head
// take 1527 / 1460 us here against 1570 / 1545 us in the prefill kernel, and
// 16 rows with 4 query heads per K/V head 440 us against 1002 (the prefill
// kernel reads K/V once per query head).  With 64 rows per head, 256 per K/V
// head, or 4096 keys and fewer, the prefill kernel is faster.
bool decode_route(const Problem& p) {
  if (p.Nq <= kDecodeMaxNq) return true;
  if (p.dtype == DType::F32 || p.Hkv <= 0) return false;
  return p.Nq <= 32 && (p.H / p.Hkv) * p.Nq <= 64 && p.Nk >= 8192;
}

DecodePlan plan_decode(const Problem& p, int64_t max_splits) {
  // The grid's y extent bounds the splits of the row-streaming kernel.
  if (max_splits > 65535) max_splits = 65535;
  if (max_splits < 1) max_splits = 1;
  if (decode_gqa_eligible(p)) {
    // One block per (work item, row chunk) in a 1-D grid of int-sized indices.
    const DecodePlan g = plan_decode_gqa(p, max_splits);
    const int64_t chunks = ((p.H / p.Hkv) * p.Nq + 31) / 32;
    const int64_t work8 = (p.B * p.Hkv * g.splits + 7) / 8 * 8;
    if (work8 <= INT32_MAX / chunks) return g;
  }
  // Aim for >= 4096 workgroups (16 per CU) so the HBM stream is deep enough,
  // but give each split at least 256 keys so the merge stays cheap.  The
  // splits cover the longest visible key range a row can have.
  const int64_t rows = p.B * p.H * p.Nq;
  int64_t range = p.table ? p.max_pages * p.page_size : p.Nk;
  if (p.window > 0 && p.window < range) range = p.window;
  const int64_t want = (4096 + rows - 1) / rows;
  int64_t kps = (range + want - 1) / want;
  if (kps < 256) kps = 256;
  int64_t splits = (range + kps - 1) / kps;
  if (splits < 1) splits = 1;
  if (splits > max_splits) {
    splits = max_splits;
    kps = (range + splits - 1) / splits;
    splits = (range + kps - 1) / kps;
    if (splits < 1) splits = 1;
  }
  DecodePlan plan;
  plan.splits = (int)splits;
  plan.keys_per_split = (int)kps;
  plan.scratch_bytes = (size_t)rows * (size_t)splits * (size_t)(p.D + 2) * sizeof(float);
  return plan;
}

hipError_t launch_decode(const Problem& p, const DecodePlan& plan, float* scratch) {
  if (p.dtype == DType::BF16) return launch_t<__bf16>(p, plan, scratch);
  if (p.dtype == DType::F16) return launch_t<_Float16>(p, plan, scratch);
  return launch_t<float>(p, plan, scratch);
}

}  // namespace attn
