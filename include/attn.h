/*
 * attn.h -- C ABI of the streaming (online-softmax) attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * Sources for what the calls compute (three web pages on one subject):
 *   [W]  "Intermediate and advanced kernel workshops", section "Scope and
 *        contracts", rows streaming_attention and split_softmax, and the
 *        paragraph after the table (single-head, forward only, P cast to the
 *        input precision before the P.V product).
 *   [AK] "Compare reasoning after your own attempt" (the answer key): table
 *        rows A1, A2, A3 and "Worked answers worth memorizing by derivation".
 *   [KN] "Kernel Notes & Checklist", section 4, "The gotchas ledger".
 *
 * Conventions shared by every call:
 *   - Plain pointers and sizes only.  Device pointers point to memory of the
 *     current HIP device; the caller owns every buffer and keeps it alive
 *     until the work queued on `stream` has finished.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device work is queued asynchronously; no call synchronises the host.
 *   - Argument errors are found on the host before anything is queued and
 *     returned synchronously; nothing is written in that case.  Input
 *     *values* are never scanned: non-finite inputs are outside the contract
 *     ([W], "Scope and contracts": wrappers validate metadata only).
 *   - Status codes: ATTN_OK, ATTN_E_INVALID (bad argument), ATTN_E_UNSUPPORTED
 *     (valid but not built: head size, grid limits), ATTN_E_HIP (a HIP runtime call or
 *     kernel launch failed; the HIP error text is in attn_last_error()).
 */
#ifndef ONLINE_SOFTMAX_STREAMING_ATTN_H
#define ONLINE_SOFTMAX_STREAMING_ATTN_H

#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define ATTN_API __attribute__((visibility("default")))
#else
#define ATTN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of Q, K, V and out (all four share one type). */
#define ATTN_F32 0  /* IEEE binary32 */
#define ATTN_F16 1  /* IEEE binary16 */
#define ATTN_BF16 2 /* bfloat16 */

#define ATTN_OK 0
#define ATTN_E_INVALID 1
#define ATTN_E_UNSUPPORTED 2
#define ATTN_E_HIP 3

/*
 * attn_fwd -- scaled-dot-product attention forward, streaming over key tiles.
 *
 * Computes, for every batch b < B, head h < H and query row i < Nq,
 *
 *     out[b,h,i,:] = sum_{j visible} softmax_j(scale * Q[b,h,i,:] . K[b,h,j,:]) V[b,h,j,:]
 *
 * carrying the running state (max m, sum l, unnormalised output a) across
 * key tiles and rescaling both l and a by exp(m_old - m_new) when the max
 * rises ([AK] row A3); the full score matrix is never formed.  Masked and
 * padded scores are -inf before the max and contribute 0 to the sums; rows
 * with nothing visible yet are pinned so they cannot produce NaN ([KN]).
 *
 * Visibility: every j < Nk when causal == 0.  When causal == 1, key j is
 * visible to query i iff j <= i + (Nk - Nq): the diagonal is included ([W],
 * streaming_attention row) and, for Nq != Nk, keys are aligned to the end
 * of the query block.  A row with no visible key gets out = +0.
 *
 * Layout: Q and out are contiguous [B, H, Nq, D]; K and V are contiguous
 * [B, H, Nk, D]; row-major, D fastest.  All four use `dtype`; out is
 * written with one round-to-nearest-even cast from the FP32 result.
 * Arithmetic: FP32 accumulation throughout; for F16/BF16 the products
 * Q.K^T and P.V run on bf16/f16 matrix cores, with P rounded to the input
 * type before P.V ([W], paragraph after the contracts table).
 *
 * Arguments:
 *   Q, K, V, out  device pointers, 16-byte aligned; out must not overlap
 *                 Q, K or V.  K and V may be NULL when Nk == 0.
 *   B, H, Nq, Nk  >= 0.  B, H or Nq == 0 is a no-op returning ATTN_OK.
 *                 Nk == 0 writes out = 0.  Per head, Nq*D and Nk*D must be
 *                 < 2^31, and B*H and B*H*Nq (rows) < 2^31; element offsets
 *                 across heads are 64-bit, so whole tensors may exceed 2^31
 *                 elements.
 *   D             head size: 16, 32, 64 or 128 (else ATTN_E_UNSUPPORTED).
 *   causal        0 or 1.
 *   scale         logit scale, finite and > 0 (the pages use 1/sqrt(D)).
 *   dtype         ATTN_F32, ATTN_F16 or ATTN_BF16.
 *   stream        hipStream_t the work is queued on.
 *
 * Paths: Nq <= 8 takes the split-key decode path (keys split across
 * workgroups, partial states merged); so does bf16/f16 with Nq <= 32,
 * (H / Hkv) * Nq <= 64 and Nk >= 8192.  Problems whose rows alone would
 * leave CUs idle (bf16/f16: at most 64 query tiles of 256 rows over at
 * least 2048 keys; FP32: fewer than 512 default workgroups over at least
 * 1024 keys) split each query tile's keys over workgroups the same way
 * (split-KV prefill).  Everything else takes the tiled prefill kernels.
 * Memory: the tiled prefill kernels allocate nothing.  The split-key decode
 * path and the split-KV prefill need a scratch array of partial states
 * (FP32, (D + 2) floats per query row and split).  The library keeps one
 * such buffer per (device, stream), taken with hipMallocAsync on `stream`,
 * grown on demand in 1 MiB steps and held until the process ends; calls on
 * one stream reuse it in stream order, and every call that takes scratch
 * (this one, attn_fwd_varlen, attn_bwd, attn_decode_paged, softmax_rows)
 * shares it.  A stream on which such a call may still run must be
 * synchronised before it is destroyed (a new stream may receive its
 * handle, and with it the buffer).  Under HIP graph capture each call instead takes its own hipMallocAsync /
 * hipFreeAsync pair, which become the graph's allocation nodes.  Callers
 * that cannot allocate at all use attn_decode_paged_noalloc.
 */
ATTN_API int attn_fwd(const void* Q, const void* K, const void* V, void* out,
             int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
             int causal, float scale, int dtype, void* stream);

/*
 * attn_fwd_stats -- attn_fwd that also returns each row's merge state.
 *
 * Same arguments and behaviour as attn_fwd, plus two optional FP32 device
 * arrays of B*H*Nq elements, row-major [B, H, Nq]:
 *   m_out[row]  the row's maximum scaled logit, natural-log units;
 *   l_out[row]  sum over visible keys of exp(scale * q.k - m_out).
 * Together they are the row's A1 state ([AK] row A1): the sum of
 * exp(scale * q.k) over visible keys equals l * exp(m).  A row with no
 * visible key has (m, l) = (-inf, 0).  Either pointer may be NULL.
 */
ATTN_API int attn_fwd_stats(const void* Q, const void* K, const void* V, void* out,
                   int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
                   int causal, float scale, int dtype,
                   float* m_out, float* l_out, void* stream);

/*
 * attn_fwd_gqa -- attn_fwd_stats with grouped K/V heads (grouped-query
 * attention): K and V are contiguous [B, Hkv, Nk, D] with Hkv dividing H,
 * and query head h attends with K/V head h / (H / Hkv).  Hkv == H is
 * attn_fwd_stats exactly.  m_out and l_out may each be NULL.  The pages
 * attend one head at a time; grouping only changes which K/V head a query
 * head reads, so the same streaming computation ([AK] row A3) runs per
 * head.  Errors as attn_fwd, plus ATTN_E_INVALID if Hkv < 1 or Hkv does not
 * divide H (for H > 0).
 */
ATTN_API int attn_fwd_gqa(const void* Q, const void* K, const void* V, void* out,
                          int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk,
                          int64_t D, int causal, float scale, int dtype,
                          float* m_out, float* l_out, void* stream);

/*
 * attn_bwd -- gradients of the attention forward (dQ, dK, dV), recomputing
 * the probabilities from each row's forward state instead of storing them.
 *
 * For out = attn_fwd_gqa(Q, K, V) with row states (m, l) and an upstream
 * gradient dO of out, per batch b, query head h, K/V head h / (H / Hkv):
 *     P  = exp(scale * Q K^T - lse) on visible keys (0 elsewhere), lse = m + ln l
 *     dV = sum over the query heads of the group of P^T dO
 *     dS = P * (dO V^T - Delta),  Delta[i] = sum_d dO[i, d] * O[i, d]
 *     dQ = scale * dS K,  dK = sum over the group of scale * dS^T Q
 * dS row by row is the softmax vector-Jacobian product y * (g - <y, g>) of
 * [W]'s intermediate workshop I2 (softmax backward; [AK] row I2 and its
 * worked answer), with y = P and g = dO V^T; <P, dO V^T> = Delta because
 * out = P V.  Visibility (causal or not) is attn_fwd's; a query row with no
 * visible key gets dQ = 0, a key no query sees gets dK = dV = 0.
 *
 * Layout: Q, O, dO, dQ contiguous [B, H, Nq, D]; K, V, dK, dV contiguous
 * [B, Hkv, Nk, D]; m, l FP32 [B, H, Nq] exactly as attn_fwd_stats /
 * attn_fwd_gqa write them (O too: the forward's rounded output).  All
 * tensors but m, l use `dtype` (ATTN_F32, ATTN_F16 or ATTN_BF16).
 * Arithmetic: for F16/BF16, Q K^T, dO V^T and every sum in FP32 on bf16/f16
 * matrix cores; P and dS are rounded to `dtype` as operands of the products
 * that form dV, dK and dQ; one round-to-nearest-even cast per output
 * element.  For F32, everything in FP32 on the vector ALUs with nothing
 * rounded to a narrower type.  No atomics: results are bitwise
 * reproducible from run to run.
 *
 * Arguments:
 *   Q, K, V, O, dO  device pointers, 16-byte aligned (K, V may be NULL if
 *                   Nk == 0; Q, O, dO, m, l may be NULL if Nq == 0).
 *   m, l            device FP32 arrays, 4-byte aligned.
 *   dQ, dK, dV      device outputs, 16-byte aligned, overwritten entirely;
 *                   none may overlap an input or another output.
 *   B, H, Hkv, Nq, Nk, D, causal, scale, dtype, stream: as attn_fwd_gqa
 *                   (D in {16, 32, 64, 128}); additionally B*Hkv*Nk < 2^31.
 *                   Nq == 0 writes dK = dV = 0; Nk == 0 writes dQ = 0.
 * Memory: a scratch array of 8 * B*H*Nq bytes (per row the base-2 lse and
 * Delta), the per-stream scratch described under attn_fwd.  Two kernels are queued: dQ (which also fills the scratch),
 * then dK and dV.
 * Returns ATTN_OK once queued, else the status codes of attn_fwd.
 */
ATTN_API int attn_bwd(const void* Q, const void* K, const void* V, const void* O,
                      const void* dO, const float* m, const float* l,
                      void* dQ, void* dK, void* dV,
                      int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk,
                      int64_t D, int causal, float scale, int dtype, void* stream);

/*
 * attn_fwd_masked -- attn_fwd_gqa with an arbitrary boolean mask and/or a
 * sliding window (the arbitrary masks that [W] "Scope and contracts" lists
 * as an extension opportunity; the per-row computation is [AK] row A3's).
 *
 * Key j is visible to query row i of head (b, h) iff the causal rule of
 * attn_fwd holds (when causal == 1), the window holds (when window > 0:
 * j > i + (Nk - Nq) - window, causal == 1 required), and, when mask is not
 * NULL, bit (j % 32) of word mask[b*mask_stride_b + h*mask_stride_h +
 * i*ceil(Nk/32) + j/32] is set.  Rows with no visible key get out = 0 and
 * (m, l) = (-inf, 0).  A window skips the key tiles before each query
 * tile's window.
 *
 * mask: NULL or a device array of uint32 words, 4-byte aligned, bit-packed
 *   row by row ([B or 1, H or 1, Nq, ceil(Nk/32)] with strides in words;
 *   a stride of 0 broadcasts over that dimension).  Bits past Nk in a row's
 *   last word are ignored.  Values are not scanned.
 * Other arguments, layout, errors and memory as attn_fwd_gqa (m_out, l_out
 * may be NULL; window >= 0, mask strides >= 0); out, m_out and l_out must
 * not overlap the mask.  Every Nq takes the tiled kernels (no split-key
 * decode path), so the call allocates nothing.
 */
ATTN_API int attn_fwd_masked(const void* Q, const void* K, const void* V, void* out,
                             const uint32_t* mask, int64_t mask_stride_b,
                             int64_t mask_stride_h, int64_t B, int64_t H, int64_t Hkv,
                             int64_t Nq, int64_t Nk, int64_t D, int causal, int64_t window,
                             float scale, int dtype, float* m_out, float* l_out,
                             void* stream);

/*
 * attn_fwd_dropout -- attn_fwd_gqa with dropout on the attention
 * probabilities (dropout is one of the extension opportunities [W] "Scope
 * and contracts" lists; the per-row computation is [AK] row A3's).
 *
 * With w_ij = exp(scale q_i.k_j - m_i) on visible keys and l_i = sum_j w_ij
 * (dropout does not change m, l):
 *     out_i = sum_j w_ij keep_ij V_j / l_i * 65536 / (65536 - T)
 * keep_ij: 16-bit field j % 16 of Philox4x64-10 (Salmon et al., SC 2011) on
 * counter (j / 16, i, b*H + h, offset) under key (seed, 0) is >= T, field t
 * at bits 16*(t % 4) of output word t / 4; T = round(p * 65536), so the
 * drop probability is T / 65536 and the output is unbiased.  Query row i
 * and key j are indices within the head.  The same (seed, offset) gives the
 * same mask on every call; advance `offset` between calls for fresh masks.
 *
 * p: 0 <= p < 1 and round(p * 65536) <= 65535 (else ATTN_E_INVALID); p = 0
 * gives attn_fwd_gqa's output bit for bit when that call also takes the
 * tiled kernels (a bf16/f16 problem too small to fill the GPU splits each
 * row's keys over several waves or workgroups there, which rounds
 * differently, within the same tolerances).  Other arguments, layout,
 * errors as attn_fwd_gqa; m_out, l_out may be NULL.  Every Nq takes the
 * tiled kernels; the call allocates nothing.
 */
ATTN_API int attn_fwd_dropout(const void* Q, const void* K, const void* V, void* out,
                              int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk,
                              int64_t D, int causal, float scale, float p, uint64_t seed,
                              uint64_t offset, int dtype, float* m_out, float* l_out,
                              void* stream);

/*
 * attn_fwd_varlen -- attention over a batch of packed sequences of
 * different lengths (the padding lengths that [W] "Scope and contracts"
 * lists as an extension opportunity, in packed form; per sequence the
 * computation is attn_fwd_gqa's, [AK] row A3).
 *
 * B sequences are concatenated along the token axis.  Sequence b owns query
 * rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key rows cu_seqlens_k[b] ..
 * cu_seqlens_k[b+1]-1, and attends only to its own keys; query head h reads
 * K/V head h / (H / Hkv); causal keys are aligned to the end of the
 * sequence's own query block (j <= i + Nk_b - Nq_b).  Empty sequences and
 * sequences with no keys are allowed (rows without a visible key get 0).
 *
 * Layout (token-major, D fastest): Q and out contiguous [total_q, H, D]; K
 * and V contiguous [total_k, Hkv, D]; cu_seqlens_q/k int32 [B + 1]
 * (non-decreasing, first 0, last total_q / total_k); m_out, l_out optional
 * FP32 [H, total_q] (head-major) with attn_fwd_stats' meaning.  dtype and
 * arithmetic as attn_fwd.
 *
 * Arguments:
 *   max_seqlen_q  the longest query sequence (sizes the grid; 0 <= it <=
 *                 total_q).  A longer sequence is outside the contract:
 *                 some of its rows may be left unwritten (none is written
 *                 wrong).
 *   cu_seqlens_*  device arrays, 4-byte aligned.  Values are not scanned:
 *                 each bound is clamped into [0, total] and made
 *                 non-decreasing, so no value addresses memory outside the
 *                 tensors.
 *   Q, K, V, out  16-byte aligned device pointers (K, V may be NULL if
 *                 total_k == 0); out must not overlap an input.
 *   Limits: total_q, total_k, B*H*max_seqlen_q < 2^31; packed K (and V)
 *   at most 4 GiB (else ATTN_E_UNSUPPORTED).  B, H or total_q == 0 is a
 *   no-op.  D, causal, scale, dtype, stream as attn_fwd.
 * Paths: bf16/f16 calls of at most 64 query tiles of 256 rows (B * H *
 * ceil(max_seqlen_q / 256)) over at least 2048 keys in all (total_k) split
 * each query tile's keys over workgroups when the rows alone would leave
 * CUs idle (the split-KV prefill of attn_fwd; the lengths are not read on
 * the host, so total_k stands in for the longest sequence's key count);
 * everything else takes the tiled prefill kernels.
 * Memory: the tiled kernels allocate nothing; the split-KV prefill uses the
 * per-stream scratch described under attn_fwd ((D + 2) FP32 values per
 * row of H * total_q and split).  Returns ATTN_OK once queued, else the
 * status codes of attn_fwd.
 */
ATTN_API int attn_fwd_varlen(const void* Q, const void* K, const void* V, void* out,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                             int64_t B, int64_t H, int64_t Hkv, int64_t total_q,
                             int64_t total_k, int64_t max_seqlen_q, int64_t D, int causal,
                             float scale, int dtype, float* m_out, float* l_out,
                             void* stream);

/*
 * attn_decode_paged -- attention of a few query rows per head over a paged
 * key/value cache, with an optional sliding window (a KV-cache slice and a
 * sliding window: the decode variants the workshops page plans for a later
 * week; the computation per row is attn_fwd_gqa's, [AK] row A3).
 *
 * Sequence b has seq_lens[b] keys (clamped to [0, max_pages * page_size]);
 * its key j lives in physical page block_table[b * max_pages + j / page_size]
 * at row j % page_size.  Query head h of sequence b attends with K/V head
 * h / (H / Hkv).  Visibility for query row i, with off = seq_lens[b] - Nq:
 * every key when causal == 0; keys j <= i + off when causal == 1; and with
 * window > 0 (causal == 1 only) also j > i + off - window, i.e. the `window`
 * keys ending at the row's diagonal.  A row with no visible key gets out = 0
 * and (m, l) = (-inf, 0).  Keys are split across workgroups and the partial
 * states folded with the A1 merge ([AK] rows A1, A2), as attn_fwd does for
 * Nq <= 8; any Nq >= 1 is accepted.  With (H / Hkv) * Nq > 1 query rows
 * per K/V head (bf16 or f16, any page size) each K/V tile read serves 32 of
 * them; otherwise each row streams its keys.
 *
 * Layout: Q and out contiguous [B, H, Nq, D]; K_cache and V_cache contiguous
 * [num_pages, Hkv, page_size, D] (one page of one head is contiguous);
 * block_table int32 [B, max_pages]; seq_lens int32 [B]; m_out, l_out
 * optional FP32 [B, H, Nq] as in attn_fwd_stats.  dtype as attn_fwd (FP32
 * accumulation; out written with one round-to-nearest-even cast).
 *
 * Arguments:
 *   Q, K_cache, V_cache, out  device pointers, 16-byte aligned; out must not
 *            overlap an input.
 *   block_table, seq_lens     device int32 arrays, 4-byte aligned.  Their
 *            values are not scanned: a table entry outside [0, num_pages) is
 *            read as an absent key (it contributes nothing); entries past a
 *            sequence's length are never read.
 *   page_size a power of two in [1, 2^20]; num_pages >= 1, max_pages >= 1,
 *            max_pages * page_size < 2^31, B * H * Nq < 2^31.
 *   causal   0 or 1; window >= 0 (0 = none; > 0 needs causal == 1).
 *   D, scale, dtype, stream: as attn_fwd.  B, H or Nq == 0 is a no-op.
 * Memory: partial states of the key splits in the per-stream scratch
 * described under attn_fwd.
 * Returns ATTN_OK once queued; ATTN_E_INVALID / ATTN_E_UNSUPPORTED /
 * ATTN_E_HIP as attn_fwd.
 */
ATTN_API int attn_decode_paged(const void* Q, const void* K_cache, const void* V_cache,
                               const int32_t* block_table, const int32_t* seq_lens,
                               void* out, int64_t B, int64_t H, int64_t Hkv, int64_t Nq,
                               int64_t D, int64_t num_pages, int64_t page_size,
                               int64_t max_pages, int causal, int64_t window, float scale,
                               int dtype, float* m_out, float* l_out, void* stream);

/*
 * attn_decode_paged_noalloc -- attn_decode_paged for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc / hipMallocAsync.  It makes no
 * allocation of any kind (no hipMalloc, hipMallocAsync, hipFree or
 * allocating library call).
 *
 * Arguments, layout, visibility rules, results and status codes are those
 * of attn_decode_paged.  The partial states of the key splits go to a fixed
 * library-owned device buffer of 4 MiB instead of stream-ordered scratch;
 * each GPU the library runs on holds its own copy until the process ends.
 * The first call on a device looks up that device's copy (with the device
 * current; no allocation).  When the usual split plan needs more than
 * 4 MiB (B*H*Nq*S*(D+2) FP32 values for S splits) fewer splits are taken,
 * which changes only the order of the FP32 sums (results stay within the
 * same bounds; with the usual plan they equal attn_decode_paged bit for
 * bit).  A problem whose single split needs more than 4 MiB, i.e.
 * B*H*Nq*(D+2)*4 > 4 MiB, returns ATTN_E_UNSUPPORTED before any device
 * work.
 * Sharing: every call on one GPU uses the same buffer.  Calls queued on one
 * stream are ordered and safe; calls that may run at the same time on one
 * GPU (other streams, other threads, without an ordering event between
 * them) race on the buffer and give wrong results.  The buffer keeps the
 * last call's contents; every slot a call reads it writes first, so nothing
 * needs clearing.
 */
ATTN_API int attn_decode_paged_noalloc(const void* Q, const void* K_cache, const void* V_cache,
                                       const int32_t* block_table, const int32_t* seq_lens,
                                       void* out, int64_t B, int64_t H, int64_t Hkv,
                                       int64_t Nq, int64_t D, int64_t num_pages,
                                       int64_t page_size, int64_t max_pages, int causal,
                                       int64_t window, float scale, int dtype, float* m_out,
                                       float* l_out, void* stream);

/*
 * online_merge -- merge two A1 summaries ([AK] row A1 and its worked answer).
 *
 * A state (m, l) stands for sum_j exp(x_j) = l * exp(m); (-inf, 0) is the
 * empty state.  The result re-expresses both relative to the common maximum:
 *     m = max(m1, m2),  l = l1 * exp(m1 - m) + l2 * exp(m2 - m),
 * and merging two empty states gives the empty state, never NaN.
 * Example: (2, 2) merged with (4, 1) is (4, 1 + 2 exp(-2)).
 *
 * Host call in double precision; m and l are host pointers, both non-NULL
 * (else ATTN_E_INVALID).  l1 and l2 must be >= 0 and the m's must not be
 * NaN or +inf (else ATTN_E_INVALID).  Touches no device.
 */
ATTN_API int online_merge(double m1, double l1, double m2, double l2,
                 double* m, double* l);

/*
 * online_merge_batch -- the same merge, elementwise on device arrays.
 *
 * m1, l1, m2, l2, m, l: FP32 device arrays of n elements (natural-log
 * units, as written by attn_fwd_stats).  Outputs may alias inputs
 * elementwise.  The split-key decode path folds its partial states with
 * the same merge, in base-2 units inside its kernels ([AK] row A2: partial
 * statistics, then a rescaled merge, on one stream).  Queued on `stream`;
 * n == 0 is a no-op; n < 0 or a NULL or misaligned array is
 * ATTN_E_INVALID.
 */
ATTN_API int online_merge_batch(const float* m1, const float* l1,
                       const float* m2, const float* l2,
                       float* m, float* l, int64_t n, void* stream);

/*
 * softmax_rows -- row softmax of a wide matrix by the split method
 * ([W] "Scope and contracts", split_softmax row; [AK] table row A2 and its
 * worked answer).
 *
 * y[i, :] = exp(x[i, :] - max x[i, :]) / sum_j exp(x[i, j] - max x[i, :])
 * for i < M, computed as three kernels queued on `stream`: per chunk of
 * `chunk` columns a partial (m, l); per row the A1 merge of the
 * ceil(N / chunk) partials; then a re-read of x that writes exp(x - m) / l
 * with one cast to the output type.
 *
 * x, y: device pointers to contiguous row-major [M, N] arrays of `dtype`
 *       (ATTN_F32 / ATTN_F16 / ATTN_BF16), aligned to the element size;
 *       16-byte aligned rows (x, y 16-byte aligned and N * element size a
 *       multiple of 16) take vector loads.  y may equal x (in place) but
 *       must not otherwise overlap it.  Caller-owned; the library allocates
 *       only the scratch below.
 * M >= 0 (M == 0 is a no-op), N >= 1 (the pages' contract stops at 131072
 *       columns; larger N is accepted), M * ceil(N / chunk) < 2^31.
 * chunk: 256, 512, 1024, 2048 or 4096 columns per chunk, or 0 to let the
 *       library choose (the largest that still gives 2048 chunks in all).
 * Values are not scanned.  -inf entries are masked positions ([KN]
 *       gotchas ledger): they get probability 0, and a row whose entries
 *       are all -inf is written as zeros.  NaN and +inf are outside the
 *       contract.
 * Scratch: FP32 (m, l) per chunk and per row, 8 * M * (T + 1) bytes with
 *       T = ceil(N / chunk), in the per-stream scratch described under
 *       attn_fwd.
 * Returns ATTN_OK once queued; ATTN_E_INVALID for bad arguments,
 * ATTN_E_UNSUPPORTED when M * T reaches 2^31, ATTN_E_HIP if a launch or
 * the scratch allocation fails.
 */
ATTN_API int softmax_rows(const void* x, void* y, int64_t M, int64_t N, int64_t chunk,
                          int dtype, void* stream);

/*
 * softmax_rows_scratch_bytes -- bytes of scratch softmax_rows takes for
 * these sizes ([AK] worked answer A2: 1088 for M = 4, N = 32769,
 * chunk = 1024), or -1 if M < 0, N < 1 or chunk is not accepted.  Host
 * only; no device work.
 */
ATTN_API int64_t softmax_rows_scratch_bytes(int64_t M, int64_t N, int64_t chunk);

/* Static text for a status code; never NULL. */
ATTN_API const char* attn_strerror(int code);

/* Detail of the last ATTN_E_INVALID / ATTN_E_HIP on the calling thread
 * (empty string if none); valid until the next call on that thread. */
ATTN_API const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ONLINE_SOFTMAX_STREAMING_ATTN_H */
