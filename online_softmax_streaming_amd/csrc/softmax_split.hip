// Wide-row split softmax: y = softmax(x) over each row of a contiguous
// [M, N] matrix, for rows too wide for one workgroup to hold.
//
// The method is the split_softmax row of the workshops page ("Intermediate
// and advanced kernel workshops", section "Scope and contracts") as the
// answer-key page ("Compare reasoning after your own attempt") describes it
// in table row A2: three kernels ordered by one stream and a per-call
// scratch array.
//   kernel 1 (partial):   workgroup (row, chunk) reduces its C elements to a
//                         partial state (m_c, l_c) with
//                         l_c = sum exp(x - m_c), the sum of exponentials
//                         relative to the chunk's own maximum.
//   kernel 2 (merge):     one wave per row folds the T = ceil(N / C) partial
//                         states into the row's (m, l) with the A1 merge:
//                         each partial is re-expressed relative to the
//                         common maximum (answer-key row A1).
//   kernel 3 (normalise): workgroup (row, chunk) re-reads its elements and
//                         writes exp(x - m) / l, one cast at the end.
// Chunk-local probabilities cannot simply be concatenated (answer-key row
// A2): only the merged (m, l) normalises the whole row.
//
// Scratch is FP32 (m, l) per chunk and per row, 8 * M * (T + 1) bytes (the
// answer-key page's worked answer A2 prints 1088 for M = 4, N = 32769,
// C = 1024).  m is kept in the input's natural units so the exponent is
// formed from the difference x - m, which stays accurate for large |x|.
//
// Each pass is a stream over HBM (the path is bandwidth bound): lanes read
// 16-byte vectors when rows are 16-byte aligned, single elements otherwise.

#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {
namespace {

constexpr int kSmThreads = 256;

template <typename T> struct SmVec;
template <> struct SmVec<__bf16> { typedef bf16x8 type; static constexpr int n = 8; };
template <> struct SmVec<_Float16> { typedef f16x8 type; static constexpr int n = 8; };
template <> struct SmVec<float> { typedef f32x4 type; static constexpr int n = 4; };

struct SoftmaxArgs {
  const void* x;
  void* y;
  float* pm;  // [M * T] partial maxima (natural units)
  float* pl;  // [M * T] partial sums relative to pm
  float* rm;  // [M] row maxima
  float* rl;  // [M] row sums relative to rm
  int64_t M, N;
  int C;      // chunk size (elements)
  int T;      // chunks per row
  int vec;    // 1: 16-byte vector loads are aligned
};

// (m, l) pairs in natural units; an empty state is (-inf, 0).
struct State {
  float m, l;
};
__device__ __forceinline__ State merge(State a, State b) {
  const float m = fmaxf(a.m, b.m);
  const float ref = pinned_ref(m);
  State r;
  r.m = m;
  r.l = a.l * exp2_hw((a.m - ref) * kLog2e) + b.l * exp2_hw((b.m - ref) * kLog2e);
  return r;
}
__device__ __forceinline__ State wave_merge(State s) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    State t;
    t.m = __shfl_xor(s.m, o);
    t.l = __shfl_xor(s.l, o);
    s = merge(s, t);
  }
  return s;
}

// Folds elements [e0, e1) of row `row` into a per-thread state: within each
// vector the local maximum is taken first, so one extra exponential per
// vector rescales the running sum.
template <typename T>
__device__ __forceinline__ State chunk_state(const T* __restrict__ xr, int64_t e0, int64_t e1,
                                             bool vec) {
  typedef typename SmVec<T>::type vt;
  constexpr int VEC = SmVec<T>::n;
  State s{kNegInf, 0.f};
  if (vec) {
    // Two vectors per step (both loads in flight), one maximum over their
    // 2*VEC elements, then one exponential per element against it.
    constexpr int64_t STEP = (int64_t)kSmThreads * VEC;
    for (int64_t e = e0 + (int64_t)threadIdx.x * VEC; e < e1; e += 2 * STEP) {
      const bool two = e + STEP < e1;
      const vt v0 = *reinterpret_cast<const vt*>(xr + e);
      const vt v1 = two ? *reinterpret_cast<const vt*>(xr + e + STEP) : vt{};
      float f[2 * VEC];
      float mv = kNegInf;
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        f[i] = to_f32<T>(v0[i]);
        f[VEC + i] = two ? to_f32<T>(v1[i]) : kNegInf;
        mv = fmaxf(mv, fmaxf(f[i], f[VEC + i]));
      }
      // A run of masked (-inf) entries is the empty state (-inf, 0): its
      // exponents are taken against the pinned reference 0, never
      // (-inf) - (-inf).
      const float rv = pinned_ref(mv);
      float lv = 0.f;
#pragma unroll
      for (int i = 0; i < 2 * VEC; ++i) lv += exp2_hw((f[i] - rv) * kLog2e);
      s = merge(s, State{mv, lv});
    }
  } else {
    for (int64_t e = e0 + threadIdx.x; e < e1; e += kSmThreads) {
      const float f = to_f32<T>(xr[e]);
      s = merge(s, State{f, 1.f});
    }
  }
  return s;
}

template <typename T>
__global__ __launch_bounds__(kSmThreads) void softmax_partial_kernel(SoftmaxArgs a) {
  __shared__ float sm[kSmThreads / 64], sl[kSmThreads / 64];
  const int64_t wg = blockIdx.x;  // row * T + chunk
  const int64_t row = wg / a.T;
  const int chunk = (int)(wg - row * a.T);
  const T* __restrict__ xr = static_cast<const T*>(a.x) + row * a.N;
  const int64_t e0 = (int64_t)chunk * a.C;
  const int64_t e1 = e0 + a.C < a.N ? e0 + a.C : a.N;
  State s = wave_merge(chunk_state<T>(xr, e0, e1, a.vec != 0));
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    sm[wave] = s.m;
    sl[wave] = s.l;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    State r{sm[0], sl[0]};
#pragma unroll
    for (int w = 1; w < kSmThreads / 64; ++w) r = merge(r, State{sm[w], sl[w]});
    a.pm[wg] = r.m;
    a.pl[wg] = r.l;
  }
}

// One wave per row: lane i folds partials i, i + 64, ..., then the wave folds
// the lanes.
__global__ __launch_bounds__(64) void softmax_merge_kernel(SoftmaxArgs a) {
  const int64_t row = blockIdx.x;
  State s{kNegInf, 0.f};
  for (int c = threadIdx.x; c < a.T; c += 64) s = merge(s, State{a.pm[row * a.T + c], a.pl[row * a.T + c]});
  s = wave_merge(s);
  if (threadIdx.x == 0) {
    a.rm[row] = s.m;
    a.rl[row] = s.l;
  }
}

template <typename T>
__global__ __launch_bounds__(kSmThreads) void softmax_normalise_kernel(SoftmaxArgs a) {
  typedef typename SmVec<T>::type vt;
  constexpr int VEC = SmVec<T>::n;
  const int64_t wg = blockIdx.x;
  const int64_t row = wg / a.T;
  const int chunk = (int)(wg - row * a.T);
  const T* __restrict__ xr = static_cast<const T*>(a.x) + row * a.N;
  T* __restrict__ yr = static_cast<T*>(a.y) + row * a.N;
  // A row whose entries are all masked (-inf) has l = 0: it is written as
  // zeros, its reference pinned at 0 ("Kernel Notes & Checklist", gotchas
  // ledger: empty rows must not produce NaN).
  const float m = pinned_ref(a.rm[row]);
  const float rl = a.rl[row];
  const float inv = rl > 0.f ? 1.f / rl : 0.f;
  const int64_t e0 = (int64_t)chunk * a.C;
  const int64_t e1 = e0 + a.C < a.N ? e0 + a.C : a.N;
  if (a.vec) {
    for (int64_t e = e0 + (int64_t)threadIdx.x * VEC; e < e1; e += (int64_t)kSmThreads * VEC) {
      const vt v = *reinterpret_cast<const vt*>(xr + e);
      vt o;
#pragma unroll
      for (int i = 0; i < VEC; ++i) o[i] = from_f32<T>(exp2_hw((to_f32<T>(v[i]) - m) * kLog2e) * inv);
      *reinterpret_cast<vt*>(yr + e) = o;
    }
  } else {
    for (int64_t e = e0 + threadIdx.x; e < e1; e += kSmThreads)
      yr[e] = from_f32<T>(exp2_hw((to_f32<T>(xr[e]) - m) * kLog2e) * inv);
  }
}

template <typename T>
hipError_t launch_t(const SoftmaxArgs& a, hipStream_t stream) {
  const int64_t wgs = a.M * a.T;
  hipLaunchKernelGGL(softmax_partial_kernel<T>, dim3((unsigned)wgs), dim3(kSmThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(softmax_merge_kernel, dim3((unsigned)a.M), dim3(64), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(softmax_normalise_kernel<T>, dim3((unsigned)wgs), dim3(kSmThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

int64_t softmax_chunks(int64_t N, int64_t C) { return (N + C - 1) / C; }

int64_t softmax_scratch_bytes(int64_t M, int64_t N, int64_t C) {
  return 8 * M * (softmax_chunks(N, C) + 1);
}

hipError_t launch_softmax_split(const void* x, void* y, int64_t M, int64_t N, int C, DType dtype,
                                float* scratch, hipStream_t stream) {
  SoftmaxArgs a;
  a.x = x;
  a.y = y;
  a.M = M;
  a.N = N;
  a.C = C;
  a.T = (int)softmax_chunks(N, C);
  a.pm = scratch;
  a.pl = scratch + M * a.T;
  a.rm = scratch + 2 * M * a.T;
  a.rl = scratch + 2 * M * a.T + M;
  const int esize = dtype == DType::F32 ? 4 : 2;
  const bool aligned = (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                       (reinterpret_cast<uintptr_t>(y) % 16 == 0) && ((N * esize) % 16 == 0);
  a.vec = aligned ? 1 : 0;
  if (dtype == DType::BF16) return launch_t<__bf16>(a, stream);
  if (dtype == DType::F16) return launch_t<_Float16>(a, stream);
  return launch_t<float>(a, stream);
}

}  // namespace attn
