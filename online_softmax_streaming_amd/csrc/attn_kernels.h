// Internal launcher interface between the C ABI (api.hip) and the kernels.
// Every launcher assumes the problem has already been validated by the ABI
// layer: pointers aligned and non-null where used, sizes within the limits
// stated in include/attn.h, D in {16, 32, 64, 128}, B*H*Nq > 0 and Nk > 0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

enum class DType : int { F32 = 0, F16 = 1, BF16 = 2 };

struct Problem {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* m_out;  // optional [B*H*Nq]
  float* l_out;  // optional [B*H*Nq]
  int64_t B, H, Nq, Nk, D;
  int64_t Hkv;  // K/V heads; query head h reads K/V head h / (H / Hkv)
  bool causal;
  float scale;
  DType dtype;
  hipStream_t stream;
  // Decode options: a sliding window (0 = none) and a paged K/V cache
  // (table == nullptr: the contiguous layout above).
  int64_t window = 0;
  const int* table = nullptr;  // [B, max_pages] physical page of each logical page
  const int* lens = nullptr;   // [B] keys per sequence
  int64_t max_pages = 0, page_size = 0, num_pages = 0;
  // Packed variable-length sequences (prefill kernels; cu_q == nullptr: the
  // batched layout).  Q/out [total_q, H, D], K/V [total_k, Hkv, D]; Nq is
  // the longest query sequence; row states [H, total_q].
  const int* cu_q = nullptr;  // [B + 1]
  const int* cu_k = nullptr;  // [B + 1]
  int64_t total_q = 0, total_k = 0;
  // Arbitrary mask (prefill kernels, batched layout): bit j % 32 of word
  // j / 32 of row (b, h, i) at mask + b*mask_sb + h*mask_sh + i*ceil(Nk/32);
  // with `window` > 0 the prefill kernels also apply the sliding window.
  const uint32_t* mask = nullptr;
  int64_t mask_sb = 0, mask_sh = 0;
  // Dropout on the probabilities (prefill kernels, batched layout): keep
  // key j of row i of head bh iff 16-bit field j % 16 of Philox4x64-10 on
  // counter (j / 16, i, bh, offset), key (seed, 0), is >= drop_t.
  bool dropout = false;
  uint64_t seed = 0, offset = 0;
  uint32_t drop_t = 0;
  // Keys split over workgroups (launch_prefill_splitkv): `splits` splits of
  // `split_tiles` 64-key tiles; FP32 partial states in `part`: a[D] as
  // [rows][splits][D], then (m, l) as [rows][splits][2], rows in row-state
  // order (B*H*Nq batched, H*total_q packed).
  float* part = nullptr;
  int64_t splits = 0, split_tiles = 0;
};

// Streaming prefill on bf16/f16 matrix cores (prefill_mfma.hip).
hipError_t launch_prefill_mfma(const Problem& p);
// Plain prefill with the keys of each query tile split over workgroups, for
// few long rows (prefill_mfma.hip): whether to take it, and its splits; then
// the tiled kernel (bf16/f16) or the FP32 kernel writes partial states to
// p.part and a combine kernel folds them, on p.stream.
struct SplitKvPlan {
  int64_t splits;
  int64_t split_tiles;
  size_t scratch_bytes;
};
bool plan_prefill_splitkv(const Problem& p, SplitKvPlan* plan);
hipError_t launch_prefill_splitkv(const Problem& p);
// The FP32 form (prefill_f32.hip): plan, and the vector-ALU kernel's
// partial states (launch_prefill_splitkv then combines them).
bool plan_prefill_f32_splitkv(const Problem& p, SplitKvPlan* plan);
hipError_t launch_prefill_f32_partials(const Problem& p);
// Streaming prefill for FP32 inputs on the vector ALUs (prefill_f32.hip).
hipError_t launch_prefill_f32(const Problem& p);

// Split-key decode path (decode_splitk.hip): partial states per key split
// into `scratch`, then a merge kernel on the same stream.
struct DecodePlan {
  int splits;           // key splits per query row
  int keys_per_split;   // keys each split streams
  size_t scratch_bytes; // partial (m, l, a[D]) states, FP32
  bool gqa_mfma = false;  // partial states from the grouped-head matrix-core kernel
};
// At most `max_splits` key splits (fewer keys per split beyond that are
// not taken); the grid bounds it at 65535.
DecodePlan plan_decode(const Problem& p, int64_t max_splits = 65535);
hipError_t launch_decode(const Problem& p, const DecodePlan& plan, float* scratch);
// Partial states of the split-key decode for grouped K/V heads on the matrix
// cores (decode_gqa.hip); plan from plan_decode.
hipError_t launch_decode_gqa_partial(const Problem& p, const DecodePlan& plan, float* scratch);

// Nk == 0: out = 0, (m, l) = (-inf, 0) (misc.hip).
hipError_t launch_fill_empty(const Problem& p);

// Elementwise A1 merge of FP32 device arrays, natural-log units (misc.hip).
hipError_t launch_merge_batch(const float* m1, const float* l1, const float* m2,
                              const float* l2, float* m, float* l, int64_t n,
                              hipStream_t stream);

// Wide-row split softmax (softmax_split.hip): chunks per row, scratch bytes
// (FP32 (m, l) per chunk and per row) and the three ordered kernels.
int64_t softmax_chunks(int64_t N, int64_t C);
int64_t softmax_scratch_bytes(int64_t M, int64_t N, int64_t C);
hipError_t launch_softmax_split(const void* x, void* y, int64_t M, int64_t N, int C, DType dtype,
                                float* scratch, hipStream_t stream);

// Attention backward on bf16/f16 matrix cores (bwd_mfma.hip): a dQ kernel
// that also writes each row's (base-2 lse, Delta) to `scratch`, then a
// dK/dV kernel that reads them, on p.stream.
struct BwdProblem {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* m;  // [B*H*Nq] forward row state, natural units
  const float* l;
  void* dq;
  void* dk;
  void* dv;
  int64_t B, H, Hkv, Nq, Nk, D;
  bool causal;
  float scale;
  DType dtype;
  hipStream_t stream;
};
size_t bwd_scratch_bytes(const BwdProblem& p);
hipError_t launch_bwd_mfma(const BwdProblem& p, float* scratch);
// Plain batched bf16/f16 prefill with the keys of each 32-row block split
// over the waves of a workgroup and merged in LDS (prefill_splitk.hip), for
// problems too small to fill the GPU.
hipError_t launch_prefill_splitk(const Problem& p);
// FP32 inputs: the same two-kernel backward on the vector ALUs (bwd_f32.hip),
// same scratch layout.
hipError_t launch_bwd_f32(const BwdProblem& p, float* scratch);

// Row count up to which attn_fwd always takes the split-key decode path.
constexpr int64_t kDecodeMaxNq = 8;
// Whether attn_fwd takes the split-key decode path: Nq <= kDecodeMaxNq, or
// (bf16/f16) up to 32 rows per head and 64 per K/V head over >= 8192 keys,
// where reading each K/V tile once per 32 rows beats the prefill kernel.
bool decode_route(const Problem& p);

}  // namespace attn
