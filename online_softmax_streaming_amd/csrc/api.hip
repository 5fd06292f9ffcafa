// C ABI of the attention library: argument checks, path selection and the
// host form of the A1 merge.  The contract of each call is documented in
// include/attn.h; the checks below are the "validate metadata, never scan
// values" rule of the workshops page ("Scope and contracts").

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdint.h>
#include <string.h>

#include <map>
#include <mutex>
#include <utility>

#include "../../include/attn.h"
#include "attn_kernels.h"

namespace {

thread_local char g_last_error[256] = "";

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(ATTN_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

constexpr int64_t kI32Max = 2147483647;

// Keep freed stream-ordered scratch in the device's default pool instead of
// returning it to the driver at every synchronisation.
void keep_pool_memory() {
  static std::mutex mu;
  static bool done[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return;
  std::lock_guard<std::mutex> lock(mu);
  if (done[dev]) return;
  hipMemPool_t pool;
  if (hipDeviceGetDefaultMemPool(&pool, dev) == hipSuccess) {
    uint64_t threshold = UINT64_MAX;
    (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &threshold);
  }
  done[dev] = true;
}

// Scratch of the paths that keep partial states (split-key decode, split-KV
// prefill, backward, wide-row softmax).  A stream-ordered hipMallocAsync /
// hipFreeAsync pair per call left the GPU idle ~5.6 us before the next
// call's first kernel, so outside graph capture each (device, stream) keeps
// one buffer, grown on demand (in 1 MiB steps) and never shrunk, until the
// process ends.  Work on one stream runs in issue order, so a call's kernels
// use the buffer only after the previous call's kernels on that stream; the
// lock is held from the lookup to the last launch, so another host thread
// cannot grow (free) the buffer between them.  Streams are keyed by handle:
// a stream destroyed while such a call may still run on it must be
// synchronised first, as a new stream may take over its handle (and
// buffer).  Under graph capture each call takes its own hipMallocAsync /
// hipFreeAsync pair, which capture records as the graph's allocation nodes.
constexpr size_t kScratchGrain = size_t(1) << 20;

struct StreamScratch {
  void* ptr = nullptr;
  size_t bytes = 0;
};

std::mutex g_scratch_mu;

std::map<std::pair<int, uintptr_t>, StreamScratch>& scratch_map() {
  static std::map<std::pair<int, uintptr_t>, StreamScratch> m;
  return m;
}

class ScratchLease {
 public:
  ScratchLease() = default;
  ScratchLease(const ScratchLease&) = delete;
  ScratchLease& operator=(const ScratchLease&) = delete;
  ~ScratchLease() { (void)release(); }

  // `bytes` of device scratch for work queued on `s` until release().
  hipError_t acquire(hipStream_t s, size_t bytes) {
    s_ = s;
    if (bytes == 0) return hipSuccess;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(s, &cs);
    if (e != hipSuccess) return e;
    keep_pool_memory();
    if (cs != hipStreamCaptureStatusNone) {
      owned_ = true;
      return hipMallocAsync(&ptr_, bytes, s);
    }
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    lock_ = std::unique_lock<std::mutex>(g_scratch_mu);
    StreamScratch& b = scratch_map()[std::make_pair(dev, reinterpret_cast<uintptr_t>(s))];
    if (b.bytes < bytes) {
      if (b.ptr) {
        e = hipFreeAsync(b.ptr, s);
        b.ptr = nullptr;
        b.bytes = 0;
        if (e != hipSuccess) return e;
      }
      const size_t want = (bytes + kScratchGrain - 1) / kScratchGrain * kScratchGrain;
      e = hipMallocAsync(&b.ptr, want, s);
      if (e != hipSuccess) {
        b.ptr = nullptr;
        return e;
      }
      b.bytes = want;
    }
    ptr_ = b.ptr;
    return hipSuccess;
  }

  float* ptr() const { return static_cast<float*>(ptr_); }

  // After the last launch that uses the scratch.
  hipError_t release() {
    hipError_t e = hipSuccess;
    if (owned_ && ptr_) e = hipFreeAsync(ptr_, s_);
    owned_ = false;
    ptr_ = nullptr;
    if (lock_.owns_lock()) lock_.unlock();
    return e;
  }

 private:
  std::unique_lock<std::mutex> lock_;
  void* ptr_ = nullptr;
  hipStream_t s_ = nullptr;
  bool owned_ = false;
};

// The split-KV prefill (plan from plan_prefill_splitkv): partial states in
// the stream's scratch, then their combine.
int run_splitkv(attn::Problem& p, const attn::SplitKvPlan& sk) {
  ScratchLease scratch;
  hipError_t e = scratch.acquire(p.stream, sk.scratch_bytes);
  if (e != hipSuccess) return hip_fail(e, "split-key scratch allocation");
  p.part = scratch.ptr();
  p.splits = sk.splits;
  p.split_tiles = sk.split_tiles;
  e = attn::launch_prefill_splitkv(p);
  const hipError_t ef = scratch.release();
  if (e != hipSuccess) return hip_fail(e, "split-key prefill launch");
  if (ef != hipSuccess) return hip_fail(ef, "hipFreeAsync of split-key scratch");
  return ATTN_OK;
}

int run_attention(const void* Q, const void* K, const void* V, void* out, int64_t B, int64_t H,
                  int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, int causal, float scale,
                  int dtype, float* m_out, float* l_out, void* stream,
                  const uint32_t* mask = nullptr, int64_t mask_sb = 0, int64_t mask_sh = 0,
                  int64_t window = 0, const attn::Problem* dropout = nullptr,
                  bool tiled_only = false) {
  g_last_error[0] = '\0';
  if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16)
    return fail(ATTN_E_INVALID, "dtype %d is not ATTN_F32, ATTN_F16 or ATTN_BF16", dtype);
  if (causal != 0 && causal != 1) return fail(ATTN_E_INVALID, "causal must be 0 or 1, got %d", causal);
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0)
    return fail(ATTN_E_INVALID, "negative size (B=%lld H=%lld Nq=%lld Nk=%lld)", (long long)B,
                (long long)H, (long long)Nq, (long long)Nk);
  if (H > 0 && (Hkv < 1 || Hkv > H || H % Hkv != 0))
    return fail(ATTN_E_INVALID, "Hkv=%lld must divide H=%lld", (long long)Hkv, (long long)H);
  if (D <= 0) return fail(ATTN_E_INVALID, "D must be positive, got %lld", (long long)D);
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(ATTN_E_INVALID, "scale must be finite and > 0, got %g", (double)scale);
  if (D != 16 && D != 32 && D != 64 && D != 128)
    return fail(ATTN_E_UNSUPPORTED, "head size D=%lld not built (16, 32, 64, 128)", (long long)D);
  if (B > kI32Max || H > kI32Max || Nq > kI32Max || Nk > kI32Max || B * H > kI32Max ||
      Nq * D > kI32Max || Nk * D > kI32Max || B * H * Nq > kI32Max)
    return fail(ATTN_E_INVALID,
                "sizes exceed the 32-bit per-head limits (B*H, Nq*D, Nk*D, B*H*Nq < 2^31)");
  if (window < 0) return fail(ATTN_E_INVALID, "window must be >= 0, got %lld", (long long)window);
  if (window > 0 && causal != 1) return fail(ATTN_E_INVALID, "a sliding window needs causal = 1");
  if (mask_sb < 0 || mask_sh < 0) return fail(ATTN_E_INVALID, "mask strides must be >= 0");
  if (B == 0 || H == 0 || Nq == 0) return ATTN_OK;

  const int64_t elem = dtype == ATTN_F32 ? 4 : 2;
  if (!Q || !out) return fail(ATTN_E_INVALID, "Q and out must be non-NULL");
  if (Nk > 0 && (!K || !V)) return fail(ATTN_E_INVALID, "K and V must be non-NULL when Nk > 0");
  if (!aligned(Q, 16) || !aligned(out, 16) || (Nk > 0 && (!aligned(K, 16) || !aligned(V, 16))))
    return fail(ATTN_E_INVALID, "Q, K, V and out must be 16-byte aligned");
  if ((m_out && !aligned(m_out, 4)) || (l_out && !aligned(l_out, 4)))
    return fail(ATTN_E_INVALID, "m_out and l_out must be 4-byte aligned");
  const int64_t qbytes = B * H * Nq * D * elem;
  const int64_t kbytes = B * Hkv * Nk * D * elem;
  const int64_t sbytes = B * H * Nq * 4;
  if (overlaps(out, qbytes, Q, qbytes) || overlaps(out, qbytes, K, kbytes) ||
      overlaps(out, qbytes, V, kbytes))
    return fail(ATTN_E_INVALID, "out overlaps Q, K or V");
  if (overlaps(m_out, sbytes, out, qbytes) || overlaps(l_out, sbytes, out, qbytes) ||
      overlaps(m_out, sbytes, l_out, sbytes))
    return fail(ATTN_E_INVALID, "m_out / l_out overlap out or each other");
  if (mask) {
    if (!aligned(mask, 4)) return fail(ATTN_E_INVALID, "mask must be 4-byte aligned");
    const int64_t words = (Nk + 31) / 32;
    if (mask_sb > INT64_MAX / 8 / (B + 1) || mask_sh > INT64_MAX / 8 / (H + 1) ||
        Nq > INT64_MAX / 8 / (words + 1))
      return fail(ATTN_E_INVALID, "mask extent overflows 64 bits");
    const int64_t mbytes = 4 * ((B - 1) * mask_sb + (H - 1) * mask_sh + Nq * words);
    if (overlaps(out, qbytes, mask, mbytes) || overlaps(m_out, sbytes, mask, mbytes) ||
        overlaps(l_out, sbytes, mask, mbytes))
      return fail(ATTN_E_INVALID, "out, m_out or l_out overlaps the mask");
  }

  attn::Problem p;
  p.q = Q;
  p.k = K;
  p.v = V;
  p.o = out;
  p.m_out = m_out;
  p.l_out = l_out;
  p.B = B;
  p.H = H;
  p.Hkv = Hkv;
  p.Nq = Nq;
  p.Nk = Nk;
  p.D = D;
  p.causal = causal != 0;
  p.scale = scale;
  p.dtype = static_cast<attn::DType>(dtype);
  p.stream = static_cast<hipStream_t>(stream);
  p.mask = mask;
  p.mask_sb = mask_sb;
  p.mask_sh = mask_sh;
  p.window = window;
  if (dropout) {
    p.dropout = true;
    p.seed = dropout->seed;
    p.offset = dropout->offset;
    p.drop_t = dropout->drop_t;
  }

  hipError_t e;
  if (Nk == 0) {
    e = attn::launch_fill_empty(p);
    return e == hipSuccess ? ATTN_OK : hip_fail(e, "fill kernel launch");
  }
  // The masked and dropout entry points always take the tiled kernels (and
  // so allocate nothing).
  const bool plain = !tiled_only && !mask && window == 0 && !dropout;
  if (plain && attn::decode_route(p)) {
    const attn::DecodePlan plan = attn::plan_decode(p);
    ScratchLease scratch;
    e = scratch.acquire(p.stream, plan.scratch_bytes);
    if (e != hipSuccess) return hip_fail(e, "decode scratch allocation");
    e = attn::launch_decode(p, plan, scratch.ptr());
    const hipError_t ef = scratch.release();
    if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
    if (ef != hipSuccess) return hip_fail(ef, "hipFreeAsync of decode scratch");
    return ATTN_OK;
  }
  attn::SplitKvPlan sk;
  if (plain && attn::plan_prefill_splitkv(p, &sk)) return run_splitkv(p, sk);
  e = dtype == ATTN_F32 ? attn::launch_prefill_f32(p) : attn::launch_prefill_mfma(p);
  return e == hipSuccess ? ATTN_OK : hip_fail(e, "prefill kernel launch");
}

// Chunk size for softmax_rows: the caller's, or (chunk == 0) the largest of
// 4096, 2048, ..., 256 that still gives >= 2048 workgroups per pass, so
// narrow matrices with few rows still spread over the CUs.
int64_t pick_chunk(int64_t M, int64_t N, int64_t chunk) {
  if (chunk != 0) return chunk;
  int64_t c = 4096;
  while (c > 256 && M * attn::softmax_chunks(N, c) < 2048) c /= 2;
  return c;
}

bool valid_chunk(int64_t c) {
  return c == 0 || c == 256 || c == 512 || c == 1024 || c == 2048 || c == 4096;
}

// Fixed device buffer for attn_decode_paged_noalloc, for callers that
// cannot allocate.  Each GPU the library runs on holds its own copy until
// the process ends.  Host code must never pass the array's name to a
// kernel or a copy (on the host it is only a stand-in for the symbol): the
// device address comes from hipGetSymbolAddress, looked up once per device
// with that device current and kept per device.
constexpr int64_t kNoallocScratchBytes = int64_t(4) << 20;
static __device__ __align__(256) unsigned char noalloc_scratch[kNoallocScratchBytes];

int noalloc_scratch_ptr(void** out) {
  static std::mutex mu;
  static void* ptrs[64] = {};
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(ATTN_E_UNSUPPORTED, "device ordinal %d is not below 64", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    const hipError_t es = hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch));
    if (es != hipSuccess) return hip_fail(es, "hipGetSymbolAddress of the fixed decode buffer");
    if (!p) return fail(ATTN_E_HIP, "hipGetSymbolAddress gave a NULL fixed decode buffer");
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return ATTN_OK;
}

// attn_decode_paged and its variant for callers that cannot allocate
// (`noalloc`: the partial states go to the fixed buffer instead of
// stream-ordered scratch).
int run_paged(const void* Q, const void* K_cache, const void* V_cache,
              const int32_t* block_table, const int32_t* seq_lens, void* out, int64_t B,
              int64_t H, int64_t Hkv, int64_t Nq, int64_t D, int64_t num_pages,
              int64_t page_size, int64_t max_pages, int causal, int64_t window, float scale,
              int dtype, float* m_out, float* l_out, void* stream, bool noalloc) {
  g_last_error[0] = '\0';
  if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16)
    return fail(ATTN_E_INVALID, "dtype %d is not ATTN_F32, ATTN_F16 or ATTN_BF16", dtype);
  if (causal != 0 && causal != 1) return fail(ATTN_E_INVALID, "causal must be 0 or 1, got %d", causal);
  if (B < 0 || H < 0 || Nq < 0)
    return fail(ATTN_E_INVALID, "negative size (B=%lld H=%lld Nq=%lld)", (long long)B,
                (long long)H, (long long)Nq);
  if (H > 0 && (Hkv < 1 || Hkv > H || H % Hkv != 0))
    return fail(ATTN_E_INVALID, "Hkv=%lld must divide H=%lld", (long long)Hkv, (long long)H);
  if (D <= 0) return fail(ATTN_E_INVALID, "D must be positive, got %lld", (long long)D);
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(ATTN_E_INVALID, "scale must be finite and > 0, got %g", (double)scale);
  if (window < 0) return fail(ATTN_E_INVALID, "window must be >= 0, got %lld", (long long)window);
  if (window > 0 && causal != 1)
    return fail(ATTN_E_INVALID, "a sliding window needs causal = 1");
  if (page_size < 1 || (page_size & (page_size - 1)) != 0 || page_size > (1 << 20))
    return fail(ATTN_E_INVALID, "page_size must be a power of two in [1, 2^20], got %lld",
                (long long)page_size);
  if (num_pages < 1 || max_pages < 1 || num_pages > kI32Max || max_pages * page_size > kI32Max)
    return fail(ATTN_E_INVALID, "need num_pages >= 1, max_pages >= 1, num_pages < 2^31 and "
                                "max_pages * page_size < 2^31");
  if (D != 16 && D != 32 && D != 64 && D != 128)
    return fail(ATTN_E_UNSUPPORTED, "head size D=%lld not built (16, 32, 64, 128)", (long long)D);
  if (B > kI32Max || H > kI32Max || Nq > kI32Max || B * H > kI32Max || B * H * Nq > kI32Max ||
      B > kI32Max / max_pages)
    return fail(ATTN_E_INVALID, "sizes exceed the 32-bit limits (B*H*Nq, B*max_pages < 2^31)");
  if (B == 0 || H == 0 || Nq == 0) return ATTN_OK;

  const int64_t elem = dtype == ATTN_F32 ? 4 : 2;
  if (!Q || !K_cache || !V_cache || !block_table || !seq_lens || !out)
    return fail(ATTN_E_INVALID, "Q, K_cache, V_cache, block_table, seq_lens and out must be non-NULL");
  if (!aligned(Q, 16) || !aligned(K_cache, 16) || !aligned(V_cache, 16) || !aligned(out, 16))
    return fail(ATTN_E_INVALID, "Q, K_cache, V_cache and out must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(seq_lens, 4) || (m_out && !aligned(m_out, 4)) ||
      (l_out && !aligned(l_out, 4)))
    return fail(ATTN_E_INVALID, "block_table, seq_lens, m_out and l_out must be 4-byte aligned");
  if (num_pages > INT64_MAX / Hkv / page_size / D / elem)
    return fail(ATTN_E_INVALID, "cache size overflows 64 bits");
  const int64_t qbytes = B * H * Nq * D * elem;
  const int64_t cbytes = num_pages * Hkv * page_size * D * elem;
  const int64_t sbytes = B * H * Nq * 4;
  if (overlaps(out, qbytes, Q, qbytes) || overlaps(out, qbytes, K_cache, cbytes) ||
      overlaps(out, qbytes, V_cache, cbytes) || overlaps(out, qbytes, block_table, B * max_pages * 4) ||
      overlaps(out, qbytes, seq_lens, B * 4))
    return fail(ATTN_E_INVALID, "out overlaps an input");
  if (overlaps(m_out, sbytes, out, qbytes) || overlaps(l_out, sbytes, out, qbytes) ||
      overlaps(m_out, sbytes, l_out, sbytes))
    return fail(ATTN_E_INVALID, "m_out / l_out overlap out or each other");

  attn::Problem p;
  p.q = Q;
  p.k = K_cache;
  p.v = V_cache;
  p.o = out;
  p.m_out = m_out;
  p.l_out = l_out;
  p.B = B;
  p.H = H;
  p.Hkv = Hkv;
  p.Nq = Nq;
  p.Nk = max_pages * page_size;
  p.D = D;
  p.causal = causal != 0;
  p.scale = scale;
  p.dtype = static_cast<attn::DType>(dtype);
  p.stream = static_cast<hipStream_t>(stream);
  p.window = window;
  p.table = block_table;
  p.lens = seq_lens;
  p.max_pages = max_pages;
  p.page_size = page_size;
  p.num_pages = num_pages;

  if (noalloc) {
    // One key split needs B*H*Nq*(D+2) FP32 values; fewer splits than the
    // usual plan are taken when that plan does not fit the fixed buffer.
    const int64_t per_split = B * H * Nq * (D + 2) * 4;
    if (per_split > kNoallocScratchBytes)
      return fail(ATTN_E_UNSUPPORTED,
                  "attn_decode_paged_noalloc: one key split of B*H*Nq=%lld rows needs %lld bytes, "
                  "the fixed buffer holds %lld",
                  (long long)(B * H * Nq), (long long)per_split, (long long)kNoallocScratchBytes);
    void* fixed = nullptr;
    const int rc = noalloc_scratch_ptr(&fixed);
    if (rc != ATTN_OK) return rc;
    const attn::DecodePlan plan = attn::plan_decode(p, kNoallocScratchBytes / per_split);
    if ((int64_t)plan.scratch_bytes > kNoallocScratchBytes)
      return fail(ATTN_E_UNSUPPORTED, "attn_decode_paged_noalloc: plan exceeds the fixed buffer");
    const hipError_t e = attn::launch_decode(p, plan, static_cast<float*>(fixed));
    return e == hipSuccess ? ATTN_OK : hip_fail(e, "paged decode kernel launch");
  }
  const attn::DecodePlan plan = attn::plan_decode(p);
  ScratchLease scratch;
  hipError_t e = scratch.acquire(p.stream, plan.scratch_bytes);
  if (e != hipSuccess) return hip_fail(e, "decode scratch allocation");
  e = attn::launch_decode(p, plan, scratch.ptr());
  const hipError_t ef = scratch.release();
  if (e != hipSuccess) return hip_fail(e, "paged decode kernel launch");
  if (ef != hipSuccess) return hip_fail(ef, "hipFreeAsync of decode scratch");
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd(const void* Q, const void* K, const void* V, void* out, int64_t B, int64_t H,
             int64_t Nq, int64_t Nk, int64_t D, int causal, float scale, int dtype, void* stream) {
  return run_attention(Q, K, V, out, B, H, H, Nq, Nk, D, causal, scale, dtype, nullptr, nullptr,
                       stream);
}

int attn_fwd_stats(const void* Q, const void* K, const void* V, void* out, int64_t B, int64_t H,
                   int64_t Nq, int64_t Nk, int64_t D, int causal, float scale, int dtype,
                   float* m_out, float* l_out, void* stream) {
  return run_attention(Q, K, V, out, B, H, H, Nq, Nk, D, causal, scale, dtype, m_out, l_out,
                       stream);
}

int attn_fwd_gqa(const void* Q, const void* K, const void* V, void* out, int64_t B, int64_t H,
                 int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, int causal, float scale,
                 int dtype, float* m_out, float* l_out, void* stream) {
  return run_attention(Q, K, V, out, B, H, Hkv, Nq, Nk, D, causal, scale, dtype, m_out, l_out,
                       stream);
}

int attn_fwd_masked(const void* Q, const void* K, const void* V, void* out, const uint32_t* mask,
                    int64_t mask_stride_b, int64_t mask_stride_h, int64_t B, int64_t H,
                    int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, int causal, int64_t window,
                    float scale, int dtype, float* m_out, float* l_out, void* stream) {
  return run_attention(Q, K, V, out, B, H, Hkv, Nq, Nk, D, causal, scale, dtype, m_out, l_out,
                       stream, mask, mask_stride_b, mask_stride_h, window, nullptr, true);
}

int attn_fwd_dropout(const void* Q, const void* K, const void* V, void* out, int64_t B, int64_t H,
                     int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, int causal, float scale,
                     float p, uint64_t seed, uint64_t offset, int dtype, float* m_out,
                     float* l_out, void* stream) {
  g_last_error[0] = '\0';
  if (!(p >= 0.f) || !(p < 1.f))
    return fail(ATTN_E_INVALID, "dropout p must satisfy 0 <= p < 1, got %g", (double)p);
  const double t = floor((double)p * 65536.0 + 0.5);
  if (t > 65535.0)
    return fail(ATTN_E_INVALID, "dropout p=%g rounds to a threshold of 65536 (drop everything)",
                (double)p);
  attn::Problem d;
  d.seed = seed;
  d.offset = offset;
  d.drop_t = (uint32_t)t;
  return run_attention(Q, K, V, out, B, H, Hkv, Nq, Nk, D, causal, scale, dtype, m_out, l_out,
                       stream, nullptr, 0, 0, 0, &d);
}

int attn_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
             const float* m, const float* l, void* dQ, void* dK, void* dV, int64_t B, int64_t H,
             int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, int causal, float scale, int dtype,
             void* stream) {
  g_last_error[0] = '\0';
  if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16)
    return fail(ATTN_E_INVALID, "dtype %d is not ATTN_F32, ATTN_F16 or ATTN_BF16", dtype);
  if (causal != 0 && causal != 1) return fail(ATTN_E_INVALID, "causal must be 0 or 1, got %d", causal);
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0)
    return fail(ATTN_E_INVALID, "negative size (B=%lld H=%lld Nq=%lld Nk=%lld)", (long long)B,
                (long long)H, (long long)Nq, (long long)Nk);
  if (H > 0 && (Hkv < 1 || Hkv > H || H % Hkv != 0))
    return fail(ATTN_E_INVALID, "Hkv=%lld must divide H=%lld", (long long)Hkv, (long long)H);
  if (D <= 0) return fail(ATTN_E_INVALID, "D must be positive, got %lld", (long long)D);
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(ATTN_E_INVALID, "scale must be finite and > 0, got %g", (double)scale);
  if (D != 16 && D != 32 && D != 64 && D != 128)
    return fail(ATTN_E_UNSUPPORTED, "head size D=%lld not built (16, 32, 64, 128)", (long long)D);
  if (B > kI32Max || H > kI32Max || Nq > kI32Max || Nk > kI32Max || B * H > kI32Max ||
      Nq * D > kI32Max || Nk * D > kI32Max || B * H * Nq > kI32Max || B * Hkv * Nk > kI32Max)
    return fail(ATTN_E_INVALID, "sizes exceed the 32-bit limits (B*H, Nq*D, Nk*D, B*H*Nq, "
                                "B*Hkv*Nk < 2^31)");
  if (B == 0 || H == 0 || (Nq == 0 && Nk == 0)) return ATTN_OK;

  const int64_t elem = dtype == ATTN_F32 ? 4 : 2;
  const int64_t qbytes = B * H * Nq * D * elem;
  const int64_t kbytes = B * Hkv * Nk * D * elem;
  const int64_t sbytes = B * H * Nq * 4;
  if (Nq > 0 && (!Q || !O || !dO || !m || !l || !dQ))
    return fail(ATTN_E_INVALID, "Q, O, dO, m, l and dQ must be non-NULL when Nq > 0");
  if (Nk > 0 && (!K || !V || !dK || !dV))
    return fail(ATTN_E_INVALID, "K, V, dK and dV must be non-NULL when Nk > 0");
  const void* a16[8] = {Q, K, V, O, dO, dQ, dK, dV};
  for (const void* p : a16)
    if (p && !aligned(p, 16)) return fail(ATTN_E_INVALID, "Q, K, V, O, dO, dQ, dK, dV must be 16-byte aligned");
  if ((m && !aligned(m, 4)) || (l && !aligned(l, 4)))
    return fail(ATTN_E_INVALID, "m and l must be 4-byte aligned");
  // Outputs must not overlap any input or each other.
  struct Span {
    const void* p;
    int64_t n;
  };
  const Span outs[3] = {{dQ, Nq > 0 ? qbytes : 0}, {dK, kbytes}, {dV, kbytes}};
  const Span ins[7] = {{Q, qbytes}, {K, kbytes}, {V, kbytes}, {O, qbytes},
                       {dO, qbytes}, {m, sbytes}, {l, sbytes}};
  for (int i = 0; i < 3; ++i) {
    for (const Span& in : ins)
      if (overlaps(outs[i].p, outs[i].n, in.p, in.n))
        return fail(ATTN_E_INVALID, "dQ, dK and dV must not overlap an input");
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n))
        return fail(ATTN_E_INVALID, "dQ, dK and dV must not overlap each other");
  }

  attn::BwdProblem p;
  p.q = Q;
  p.k = K;
  p.v = V;
  p.o = O;
  p.dout = dO;
  p.m = m;
  p.l = l;
  p.dq = dQ;
  p.dk = dK;
  p.dv = dV;
  p.B = B;
  p.H = H;
  p.Hkv = Hkv;
  p.Nq = Nq;
  p.Nk = Nk;
  p.D = D;
  p.causal = causal != 0;
  p.scale = scale;
  p.dtype = static_cast<attn::DType>(dtype);
  p.stream = static_cast<hipStream_t>(stream);

  const size_t sb = attn::bwd_scratch_bytes(p);
  ScratchLease scratch;
  hipError_t e = scratch.acquire(p.stream, sb);
  if (e != hipSuccess) return hip_fail(e, "backward scratch allocation");
  e = dtype == ATTN_F32 ? attn::launch_bwd_f32(p, scratch.ptr())
                        : attn::launch_bwd_mfma(p, scratch.ptr());
  const hipError_t ef = scratch.release();
  if (e != hipSuccess) return hip_fail(e, "backward kernel launch");
  if (ef != hipSuccess) return hip_fail(ef, "hipFreeAsync of backward scratch");
  return ATTN_OK;
}

int attn_decode_paged(const void* Q, const void* K_cache, const void* V_cache,
                      const int32_t* block_table, const int32_t* seq_lens, void* out, int64_t B,
                      int64_t H, int64_t Hkv, int64_t Nq, int64_t D, int64_t num_pages,
                      int64_t page_size, int64_t max_pages, int causal, int64_t window,
                      float scale, int dtype, float* m_out, float* l_out, void* stream) {
  return run_paged(Q, K_cache, V_cache, block_table, seq_lens, out, B, H, Hkv, Nq, D, num_pages,
                   page_size, max_pages, causal, window, scale, dtype, m_out, l_out, stream,
                   false);
}

int attn_decode_paged_noalloc(const void* Q, const void* K_cache, const void* V_cache,
                              const int32_t* block_table, const int32_t* seq_lens, void* out,
                              int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t D,
                              int64_t num_pages, int64_t page_size, int64_t max_pages,
                              int causal, int64_t window, float scale, int dtype, float* m_out,
                              float* l_out, void* stream) {
  return run_paged(Q, K_cache, V_cache, block_table, seq_lens, out, B, H, Hkv, Nq, D, num_pages,
                   page_size, max_pages, causal, window, scale, dtype, m_out, l_out, stream,
                   true);
}

int attn_fwd_varlen(const void* Q, const void* K, const void* V, void* out,
                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int64_t B,
                    int64_t H, int64_t Hkv, int64_t total_q, int64_t total_k,
                    int64_t max_seqlen_q, int64_t D, int causal, float scale, int dtype,
                    float* m_out, float* l_out, void* stream) {
  g_last_error[0] = '\0';
  if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16)
    return fail(ATTN_E_INVALID, "dtype %d is not ATTN_F32, ATTN_F16 or ATTN_BF16", dtype);
  if (causal != 0 && causal != 1) return fail(ATTN_E_INVALID, "causal must be 0 or 1, got %d", causal);
  if (B < 0 || H < 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0)
    return fail(ATTN_E_INVALID, "negative size (B=%lld H=%lld total_q=%lld total_k=%lld "
                "max_seqlen_q=%lld)", (long long)B, (long long)H, (long long)total_q,
                (long long)total_k, (long long)max_seqlen_q);
  if (H > 0 && (Hkv < 1 || Hkv > H || H % Hkv != 0))
    return fail(ATTN_E_INVALID, "Hkv=%lld must divide H=%lld", (long long)Hkv, (long long)H);
  if (D <= 0) return fail(ATTN_E_INVALID, "D must be positive, got %lld", (long long)D);
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(ATTN_E_INVALID, "scale must be finite and > 0, got %g", (double)scale);
  if (max_seqlen_q > total_q)
    return fail(ATTN_E_INVALID, "max_seqlen_q=%lld exceeds total_q=%lld", (long long)max_seqlen_q,
                (long long)total_q);
  if (D != 16 && D != 32 && D != 64 && D != 128)
    return fail(ATTN_E_UNSUPPORTED, "head size D=%lld not built (16, 32, 64, 128)", (long long)D);
  if (B > kI32Max - 1 || H > kI32Max || total_q > kI32Max || total_k > kI32Max ||
      B * H > kI32Max || B * H * max_seqlen_q > kI32Max)
    return fail(ATTN_E_INVALID, "sizes exceed the 32-bit limits (B*H*max_seqlen_q, total_q, "
                                "total_k < 2^31)");
  const int64_t elem = dtype == ATTN_F32 ? 4 : 2;
  if (total_k * Hkv * D * elem > 4294967295LL)
    return fail(ATTN_E_UNSUPPORTED, "packed K and V above 4 GiB each are not supported");
  if (B == 0 || H == 0 || total_q == 0) return ATTN_OK;

  if (!Q || !out || !cu_seqlens_q || !cu_seqlens_k)
    return fail(ATTN_E_INVALID, "Q, out, cu_seqlens_q and cu_seqlens_k must be non-NULL");
  if (total_k > 0 && (!K || !V))
    return fail(ATTN_E_INVALID, "K and V must be non-NULL when total_k > 0");
  if (!aligned(Q, 16) || !aligned(out, 16) || (total_k > 0 && (!aligned(K, 16) || !aligned(V, 16))))
    return fail(ATTN_E_INVALID, "Q, K, V and out must be 16-byte aligned");
  if (!aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4) || (m_out && !aligned(m_out, 4)) ||
      (l_out && !aligned(l_out, 4)))
    return fail(ATTN_E_INVALID, "cu_seqlens_q/k, m_out and l_out must be 4-byte aligned");
  const int64_t qbytes = total_q * H * D * elem;
  const int64_t kbytes = total_k * Hkv * D * elem;
  const int64_t sbytes = total_q * H * 4;
  if (overlaps(out, qbytes, Q, qbytes) || overlaps(out, qbytes, K, kbytes) ||
      overlaps(out, qbytes, V, kbytes) || overlaps(out, qbytes, cu_seqlens_q, (B + 1) * 4) ||
      overlaps(out, qbytes, cu_seqlens_k, (B + 1) * 4))
    return fail(ATTN_E_INVALID, "out overlaps an input");
  if (overlaps(m_out, sbytes, out, qbytes) || overlaps(l_out, sbytes, out, qbytes) ||
      overlaps(m_out, sbytes, l_out, sbytes))
    return fail(ATTN_E_INVALID, "m_out / l_out overlap out or each other");
  if (max_seqlen_q == 0) return ATTN_OK;  // every sequence is empty

  attn::Problem p;
  p.q = Q;
  p.k = K;
  p.v = V;
  p.o = out;
  p.m_out = m_out;
  p.l_out = l_out;
  p.B = B;
  p.H = H;
  p.Hkv = Hkv;
  p.Nq = max_seqlen_q;
  p.Nk = 0;
  p.D = D;
  p.causal = causal != 0;
  p.scale = scale;
  p.dtype = static_cast<attn::DType>(dtype);
  p.stream = static_cast<hipStream_t>(stream);
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.total_q = total_q;
  p.total_k = total_k;
  attn::SplitKvPlan sk;
  if (dtype != ATTN_F32 && total_k > 0 && attn::plan_prefill_splitkv(p, &sk))
    return run_splitkv(p, sk);
  const hipError_t e =
      dtype == ATTN_F32 ? attn::launch_prefill_f32(p) : attn::launch_prefill_mfma(p);
  return e == hipSuccess ? ATTN_OK : hip_fail(e, "varlen prefill kernel launch");
}

int online_merge(double m1, double l1, double m2, double l2, double* m, double* l) {
  g_last_error[0] = '\0';
  if (!m || !l) return fail(ATTN_E_INVALID, "online_merge: m and l must be non-NULL");
  if (isnan(m1) || isnan(m2) || m1 == INFINITY || m2 == INFINITY)
    return fail(ATTN_E_INVALID, "online_merge: m must be finite or -inf");
  if (!(l1 >= 0.0) || !(l2 >= 0.0) || isinf(l1) || isinf(l2))
    return fail(ATTN_E_INVALID, "online_merge: l must be finite and >= 0");
  const double mm = m1 > m2 ? m1 : m2;
  if (mm == -INFINITY) {  // empty with empty: the empty state, not NaN
    *m = -INFINITY;
    *l = 0.0;
    return ATTN_OK;
  }
  *m = mm;
  *l = l1 * exp(m1 - mm) + l2 * exp(m2 - mm);
  return ATTN_OK;
}

int online_merge_batch(const float* m1, const float* l1, const float* m2, const float* l2,
                       float* m, float* l, int64_t n, void* stream) {
  g_last_error[0] = '\0';
  if (n < 0) return fail(ATTN_E_INVALID, "online_merge_batch: n < 0");
  if (n == 0) return ATTN_OK;
  if (!m1 || !l1 || !m2 || !l2 || !m || !l)
    return fail(ATTN_E_INVALID, "online_merge_batch: NULL array");
  const void* ptrs[6] = {m1, l1, m2, l2, m, l};
  for (const void* q : ptrs)
    if (!aligned(q, 4)) return fail(ATTN_E_INVALID, "online_merge_batch: misaligned array");
  const hipError_t e =
      attn::launch_merge_batch(m1, l1, m2, l2, m, l, n, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : hip_fail(e, "merge kernel launch");
}

int64_t softmax_rows_scratch_bytes(int64_t M, int64_t N, int64_t chunk) {
  if (M < 0 || N < 1 || !valid_chunk(chunk)) return -1;
  return attn::softmax_scratch_bytes(M, N, pick_chunk(M, N, chunk));
}

int softmax_rows(const void* x, void* y, int64_t M, int64_t N, int64_t chunk, int dtype,
                 void* stream) {
  g_last_error[0] = '\0';
  if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16)
    return fail(ATTN_E_INVALID, "dtype %d is not ATTN_F32, ATTN_F16 or ATTN_BF16", dtype);
  if (M < 0) return fail(ATTN_E_INVALID, "softmax_rows: M < 0");
  if (N < 1) return fail(ATTN_E_INVALID, "softmax_rows: N must be >= 1, got %lld", (long long)N);
  if (!valid_chunk(chunk))
    return fail(ATTN_E_INVALID, "softmax_rows: chunk must be 0, 256, 512, 1024, 2048 or 4096");
  if (M == 0) return ATTN_OK;
  if (!x || !y) return fail(ATTN_E_INVALID, "softmax_rows: x and y must be non-NULL");
  const int64_t elem = dtype == ATTN_F32 ? 4 : 2;
  if (!aligned(x, elem) || !aligned(y, elem))
    return fail(ATTN_E_INVALID, "softmax_rows: x and y must be aligned to their element size");
  if (N > INT64_MAX / elem / M) return fail(ATTN_E_INVALID, "softmax_rows: M*N overflows");
  const int64_t bytes = M * N * elem;
  if (x != y && overlaps(x, bytes, y, bytes))
    return fail(ATTN_E_INVALID, "softmax_rows: y overlaps x without being equal to it");
  const int64_t c = pick_chunk(M, N, chunk);
  const int64_t T = attn::softmax_chunks(N, c);
  if (M > kI32Max || T > kI32Max / M)
    return fail(ATTN_E_UNSUPPORTED, "softmax_rows: M * ceil(N / chunk) must be < 2^31");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  ScratchLease scratch;
  hipError_t e = scratch.acquire(s, (size_t)attn::softmax_scratch_bytes(M, N, c));
  if (e != hipSuccess) return hip_fail(e, "softmax scratch allocation");
  e = attn::launch_softmax_split(x, y, M, N, (int)c, static_cast<attn::DType>(dtype),
                                 scratch.ptr(), s);
  const hipError_t ef = scratch.release();
  if (e != hipSuccess) return hip_fail(e, "softmax kernel launch");
  if (ef != hipSuccess) return hip_fail(ef, "hipFreeAsync of softmax scratch");
  return ATTN_OK;
}

const char* attn_strerror(int code) {
  switch (code) {
    case ATTN_OK: return "success";
    case ATTN_E_INVALID: return "invalid argument";
    case ATTN_E_UNSUPPORTED: return "unsupported configuration";
    case ATTN_E_HIP: return "HIP runtime error";
    default: return "unknown status code";
  }
}

const char* attn_last_error(void) { return g_last_error; }

}  // extern "C"
