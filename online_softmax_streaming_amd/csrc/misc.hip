// Small kernels around the attention path.
//
//   fill_empty:   Nk == 0 -- every row has no visible key, so out = 0 and the
//                 row state is the empty A1 state (-inf, 0) (answer-key page,
//                 row A1: the empty state must never turn into NaN).
//   merge_batch:  the A1 merge of two (m, l) arrays, elementwise, in natural-
//                 log units (answer-key page, row A1 and its worked answer).
// Both are grid-stride loops over a 1-D range, so any size fits the grid.

#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {
namespace {

__global__ __launch_bounds__(256) void fill_empty_kernel(uint32_t* o, int64_t words, float* m_out,
                                                         float* l_out, int64_t rows) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += stride) o[i] = 0u;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows; i += stride) {
    if (m_out) m_out[i] = kNegInf;
    if (l_out) l_out[i] = 0.f;
  }
}

__global__ __launch_bounds__(256) void merge_batch_kernel(const float* m1, const float* l1,
                                                          const float* m2, const float* l2,
                                                          float* m, float* l, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float a_m = m1[i], a_l = l1[i], b_m = m2[i], b_l = l2[i];
    const float mm = fmaxf(a_m, b_m);
    const float ref = pinned_ref(mm);
    // Natural-log units; expf(-inf) = 0 empties a side.
    const float ll = a_l * expf(a_m - ref) + b_l * expf(b_m - ref);
    m[i] = mm;
    l[i] = mm == kNegInf ? 0.f : ll;
  }
}

unsigned grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return (unsigned)g;
}

}  // namespace

hipError_t launch_fill_empty(const Problem& p) {
  const int64_t elem = p.dtype == DType::F32 ? 4 : 2;
  const int64_t bytes = p.B * p.H * p.Nq * p.D * elem;  // multiple of 4: D >= 16
  const int64_t rows = p.B * p.H * p.Nq;
  const int64_t n = bytes / 4 > rows ? bytes / 4 : rows;
  hipLaunchKernelGGL(fill_empty_kernel, dim3(grid_for(n)), dim3(256), 0, p.stream,
                     static_cast<uint32_t*>(p.o), bytes / 4, p.m_out, p.l_out, rows);
  return hipGetLastError();
}

hipError_t launch_merge_batch(const float* m1, const float* l1, const float* m2, const float* l2,
                              float* m, float* l, int64_t n, hipStream_t stream) {
  hipLaunchKernelGGL(merge_batch_kernel, dim3(grid_for(n)), dim3(256), 0, stream, m1, l1, m2, l2,
                     m, l, n);
  return hipGetLastError();
}

}  // namespace attn
