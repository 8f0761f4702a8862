/*
 * fp8mla.h -- C ABI of libfp8mla.so: MLA decode attention that reads a paged
 * FP8-E4M3FN latent KV cache directly, the two cast paths it replaces, and
 * the write path that quantises new BF16 KV rows into the cache.
 * Hand-written HIP kernels for gfx950 (MI355X).
 *
 * Source of the operations (the pages are three public write-ups):
 *  - "The KV Cache Cast Bottleneck: A Surgical Fix for 69% Decode Overhead"
 *    (magik.net), sections The Context and The Message: a per-layer KV pool
 *    [num_slots, 1, 576] of Float8_e4m3fn, 576 = 512 latent (kv_lora_rank)
 *    + 64 rope (qk_rope_head_dim), cast in full to BFloat16 with .to() on
 *    every decode step before an MLA kernel that reads only the slots named
 *    by kv_indices; the fix is an attention kernel that reads FP8 directly.
 *  - "The Gather-Then-Cast Pivot" (magik.net), Reasoning Process and
 *    Assumptions: gather only the active FP8 rows into a compact buffer, cast
 *    that, and run BF16 attention over sequential indices.
 *  - "When a Faster Kernel Doesn't Speed Up Serving: Profiling FP8 KV Cache
 *    on AMD Instinct MI308X" (ROCm blog), Step 3: CastFromFP8, the same
 *    FP8->BF16 history cast on the extend path, and CastToFP8, the BF16->FP8
 *    copy that writes new KV rows into the cache.
 *
 * Conventions for every call:
 *  - All tensor arguments are DEVICE pointers on the current HIP device,
 *    owned by the caller, row-major and contiguous, 16-byte aligned.  The
 *    library never allocates or frees device memory and keeps no state
 *    between calls beyond a per-device compute-unit count (and, for
 *    mla_decode_fp8_noalloc, a static scratch array per device).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue kernels on it and return; they never synchronise.  Kernel
 *    faults surface as errors of a later HIP call, as usual in HIP.
 *  - FP8 means OCP E4M3FN bytes (bias 7, max 448, NaN = 0x7F/0xFF, no inf).
 *    BF16 means raw bfloat16 bit patterns (uint16_t).
 *  - Every argument is checked on the host before any HIP call; a bad
 *    argument returns a negative status and launches nothing.  There is no
 *    silent fallback to another path.
 *  - Slot indices are the caller's contract (0 <= index < num_slots).  The
 *    reading kernels clamp every index into the pool, so an out-of-range
 *    index gives a wrong row, never an out-of-bounds access; the writing
 *    kernel (scatter_cast_bf16_fp8) skips rows whose slot is out of range.
 */
#ifndef FP8MLA_H
#define FP8MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8MLA_KV_WIDTH 576   /* latent row: 512 latent + 64 rope           */
#define FP8MLA_V_WIDTH 512    /* value operand = first 512 columns of a row */
#define FP8MLA_MAX_HEADS 256  /* query heads sharing the single KV head     */
#define FP8MLA_MAX_BATCH (1 << 24) /* requests per decode call                */

/* Status codes (0 = success, negative = error). */
#define FP8MLA_OK 0
#define FP8MLA_ERR_NULL_PTR (-1)        /* a required pointer is NULL                     */
#define FP8MLA_ERR_BAD_SHAPE (-2)       /* a size is negative, zero where not allowed, or too large */
#define FP8MLA_ERR_MISALIGNED (-3)      /* a tensor pointer is not 16-byte aligned         */
#define FP8MLA_ERR_WORKSPACE (-4)       /* workspace NULL or smaller than required         */
#define FP8MLA_ERR_BAD_SCALAR (-5)      /* a scale not finite, or scale / inv_scale <= 0   */
#define FP8MLA_ERR_HIP (-6)             /* a HIP runtime call or kernel launch failed      */
#define FP8MLA_ERR_NOT_DEBUG (-7)       /* fp8mla_debug_status called on the release build */

/*
 * cast_pool_fp8_bf16 -- the full-pool cast the pages measured
 * ("The KV Cache Cast Bottleneck", The Context: get_key_buffer(l).to(q.dtype)
 * on a [495552, 1, 576] Float8_e4m3fn pool, every layer, every step).
 *
 *   out[i, j] = bf16(e4m3fn(pool[i, j]))   for 0 <= i < num_slots, 0 <= j < 576
 *
 * A pure dtype cast, no scale.  Exact: every finite E4M3FN value is a BF16
 * value; -0 keeps its sign; both NaN codes give 0x7FC0.
 *   pool      uint8  [num_slots, 576]   read
 *   out       uint16 [num_slots, 576]   written (must not overlap pool)
 *   num_slots >= 0 (0 is a no-op)
 */
int cast_pool_fp8_bf16(const uint8_t* pool, int64_t num_slots, uint16_t* out, void* stream);

/*
 * gather_cast_fp8_bf16 -- gather-then-cast fallback
 * ("The Gather-Then-Cast Pivot", Reasoning Process: k_fp8[kv_indices], cast
 * of the compact buffer, then attention over sequential indices 0..n-1).
 *
 *   out[r, j] = bf16(e4m3fn(pool[indices[r], j]))   for 0 <= r < n
 *
 *   pool      uint8  [num_slots, 576]   read
 *   indices   int32  [n]                slot ids, each in [0, num_slots)
 *   out       uint16 [n, 576]           written, compact and in index order
 *   n >= 0 (0 is a no-op); num_slots >= 1 when n > 0
 */
int gather_cast_fp8_bf16(const uint8_t* pool, int64_t num_slots, const int32_t* indices,
                         int64_t n, uint16_t* out, void* stream);

/*
 * scatter_cast_bf16_fp8 -- the write path into the FP8 cache
 * ("When a Faster Kernel Doesn't Speed Up Serving", Step 3, CastToFP8:
 * set_kv_buffer stores freshly computed BF16 KV rows into the FP8 KV cache
 * through a BF16 -> Float8_e4m3fn copy).
 *
 *   pool[slots[r], j] = e4m3fn(float32(src[r, j]) * inv_scale)
 *                                       for 0 <= r < n, 0 <= j < 576
 *
 * The product is rounded to float32 first, then to the nearest E4M3FN value,
 * ties to the even code.  saturate == 0 is the copy's rule (torch's float ->
 * Float8_e4m3fn): magnitudes above 464, the midpoint between 448 and the next
 * step up, and infinities give NaN (0x7F / 0xFF); 464 itself gives 448.
 * saturate != 0 clamps magnitudes to 448 first, so overflow and infinities
 * give +-448 (0x7E / 0xFE).  In both modes NaN gives NaN, the sign bit is
 * kept (-0 -> 0x80), and 2^-9 multiples below 2^-6 are subnormal codes.
 * inv_scale = 1 is the pages' unscaled copy; a per-tensor dequant scale s
 * of the read path pairs with inv_scale = 1 / s.
 *   src       uint16 [n, src_row_stride] BF16, read; element (r, j) at
 *                                       src[r * src_row_stride + j], j < 576
 *   n >= 0 (0 is a no-op)
 *   src_row_stride >= 576, a multiple of 8 (elements)
 *   slots     int32  [n]                destination slot of each row
 *   pool      uint8  [num_slots, 576]   written in place, rows slots[r] only;
 *                                       every other byte is left unchanged
 *   num_slots >= 1 when n > 0
 *   inv_scale finite and > 0, else FP8MLA_ERR_BAD_SCALAR
 * Rows whose slot is negative or >= num_slots are not written.  Slots must
 * be distinct; with duplicates the bytes of a slot come from any one of its
 * rows, chunk by chunk.  src must not overlap pool.
 */
int scatter_cast_bf16_fp8(const uint16_t* src, int64_t n, int64_t src_row_stride,
                          const int32_t* slots, uint8_t* pool, int64_t num_slots,
                          float inv_scale, int32_t saturate, void* stream);

/*
 * mla_decode_fp8 -- fused MLA decode over the paged FP8 latent cache
 * (the fix of "The KV Cache Cast Bottleneck", The Message: the attention
 * kernel reads FP8 and computes in BF16 internally; only the slots named by
 * kv_indices are ever read, dequantised in-kernel).
 *
 * For request b (tokens kv_indices[kv_indptr[b] .. kv_indptr[b+1]-1]) and
 * query head h, with K[t,:] = scale * e4m3fn(kv_pool[slot_t, :]):
 *   s[t]        = sm_scale * sum_{d<576} q[b,h,d] * K[t,d]
 *   out[b,h,:]  = sum_t softmax(s)[t] * K[t, 0:512]          (BF16, round-to-nearest-even)
 * A request with no tokens gets a zero row.  All heads share one KV head.
 *
 *   q           uint16 [batch, num_heads, 576]  BF16 queries
 *   kv_pool     uint8  [num_slots, 576]         E4M3FN latent rows
 *   kv_indptr   int32  [batch + 1]              kv_indptr[0] = 0, non-decreasing,
 *                                               kv_indptr[batch] = total_tokens
 *   kv_indices  int32  [total_tokens]           token slot ids (page size 1; a paged
 *                                               layout is expressed slot by slot)
 *   scale       per-tensor KV dequantisation factor (> 0; 1.0 = plain E4M3 values)
 *   sm_scale    softmax scale, e.g. 1/sqrt(192)
 *   out         uint16 [batch, num_heads, 512]  BF16 output, written
 *   workspace   device scratch of at least mla_decode_fp8_workspace_bytes(...)
 *               bytes, owned by the caller; contents need no initialisation and
 *               are garbage afterwards.  Calls that may overlap (different
 *               streams) need different workspaces.  May be NULL when
 *               total_tokens == 0.
 *   1 <= batch <= FP8MLA_MAX_BATCH, 1 <= num_heads <= FP8MLA_MAX_HEADS,
 *   total_tokens >= 0, num_slots >= 1 (unless total_tokens == 0).
 * Each request's tokens are cut into 128-token tiles; the list of all tiles
 * is split into equal segments over the compute units (flash-decoding
 * split-K), and a second kernel merges the pieces of requests that span
 * several segments.  With 64 or more heads and at least 4 64-token tiles per
 * workgroup slot, 64-head workgroups walk 64-token tiles instead.  The host never reads kv_indptr, so the call stays
 * asynchronous.
 */
int mla_decode_fp8(const uint16_t* q, const uint8_t* kv_pool, int64_t num_slots,
                   const int32_t* kv_indptr, const int32_t* kv_indices, int64_t total_tokens,
                   int32_t batch, int32_t num_heads, float scale, float sm_scale,
                   uint16_t* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_decode_fp8_segments -- mla_decode_fp8 with its split-K partition
 * bounded: the list of request tiles is cut into at most num_segments
 * segments (never more than mla_decode_fp8 itself would use, which is one
 * per compute unit and head group, fewer for small calls).  The operation is
 * mla_decode_fp8's; the partition is this library's own flash-decoding split
 * (see there), which the result does not depend on beyond rounding.  For
 * tests of that invariance and for tuning; num_segments = 1 is an unsplit
 * decode with no merge kernel.  The workspace mla_decode_fp8_workspace_bytes
 * returns suffices for every num_segments.
 *   num_segments >= 1, else FP8MLA_ERR_BAD_SHAPE.
 * All other arguments, layouts, ownership and status codes as mla_decode_fp8
 * (which is this call with num_segments = INT32_MAX).
 */
int mla_decode_fp8_segments(const uint16_t* q, const uint8_t* kv_pool, int64_t num_slots,
                            const int32_t* kv_indptr, const int32_t* kv_indices,
                            int64_t total_tokens, int32_t batch, int32_t num_heads, float scale,
                            float sm_scale, uint16_t* out, void* workspace,
                            size_t workspace_bytes, int32_t num_segments, void* stream);

/*
 * Workspace size in bytes for mla_decode_fp8 on the CURRENT device with these
 * sizes (0 when total_tokens == 0: no workspace is needed).  Returns 0 for
 * invalid sizes.  For total_tokens > 0 the size depends only on batch and
 * num_heads (8 bytes per request plus two partial results per compute unit
 * and head), not on the number of tokens.  Host-only except for one query of
 * the device's compute-unit count (cached per device).
 */
size_t mla_decode_fp8_workspace_bytes(int32_t batch, int32_t num_heads, int64_t total_tokens);

/*
 * mla_decode_fp8_noalloc -- mla_decode_fp8 for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  Same computation, kernels and arguments
 * as mla_decode_fp8 minus the workspace: the split-K scratch is a static
 * device array of FP8MLA_NOALLOC_SCRATCH_BYTES inside the library, one per
 * GPU, held from the first call on that GPU until the process ends.  The
 * call allocates and frees nothing.  Every call on a GPU shares that GPU's
 * array, so calls that may overlap on one GPU (different streams, or
 * different host threads) race and must not be issued; serialise them or
 * use mla_decode_fp8 with separate workspaces.
 *   batch <= FP8MLA_NOALLOC_MAX_BATCH, else FP8MLA_ERR_BAD_SHAPE;
 *   FP8MLA_ERR_WORKSPACE if the call would need more scratch than the array
 *   holds (it is sized for every head count on devices of up to 256 compute
 *   units); FP8MLA_ERR_HIP if the array's device address cannot be found.
 * All other arguments, layouts, ownership and status codes as mla_decode_fp8.
 */
#define FP8MLA_NOALLOC_SCRATCH_BYTES (36u << 20)
#define FP8MLA_NOALLOC_MAX_BATCH 65536
int mla_decode_fp8_noalloc(const uint16_t* q, const uint8_t* kv_pool, int64_t num_slots,
                           const int32_t* kv_indptr, const int32_t* kv_indices,
                           int64_t total_tokens, int32_t batch, int32_t num_heads, float scale,
                           float sm_scale, uint16_t* out, void* stream);

/*
 * mla_decode_bf16 -- the same decode over BF16 latent rows: the attention
 * that follows a cast on the pages' fallback paths ("The Gather-Then-Cast
 * Pivot", Reasoning Process: gather, cast, attend over indices 0..n-1; "The
 * KV Cache Cast Bottleneck", The Context: cast the whole pool, attend with
 * the original indices).  Benchmark-only: it lets those paths be timed end to
 * end against mla_decode_fp8.
 *
 * Computes what mla_decode_fp8 computes, with the same arithmetic (BF16
 * scores, FP16 probabilities and values in P.V, fp32 accumulation), with
 * K[t,:] = scale * kv[kv_indices[t], :] read as BF16 instead of E4M3FN.
 *   kv          uint16 [num_rows, 576]  BF16 latent rows (e.g. the output of
 *                                       cast_pool_fp8_bf16 or gather_cast_fp8_bf16);
 *                                       values must lie within the fp16 range
 *                                       (|v| <= 65504), which cast E4M3 rows do
 *   num_rows    rows of kv (>= 1 unless total_tokens == 0)
 *   workspace   at least mla_decode_bf16_workspace_bytes(...) bytes of scratch
 * All other arguments, layouts, ownership and status codes as mla_decode_fp8.
 */
int mla_decode_bf16(const uint16_t* q, const uint16_t* kv, int64_t num_rows,
                    const int32_t* kv_indptr, const int32_t* kv_indices, int64_t total_tokens,
                    int32_t batch, int32_t num_heads, float scale, float sm_scale,
                    uint16_t* out, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace size in bytes for mla_decode_bf16 (as mla_decode_fp8_workspace_bytes). */
size_t mla_decode_bf16_workspace_bytes(int32_t batch, int32_t num_heads, int64_t total_tokens);

/*
 * mla_extend_fp8 -- extend (prefill) MLA attention reading the paged FP8 cache
 * directly ("When a Faster Kernel Doesn't Speed Up Serving", Step 3,
 * CastFromFP8: on every extend step the prefill attention reads each
 * request's whole KV history, which the original stack casts to BF16 first;
 * "The KV Cache Cast Bottleneck", The Message: the direct-FP8 MLA wrapper on
 * the extend path as well).
 *
 * Request b has the query rows qo_indptr[b] .. qo_indptr[b+1]-1 (q_len_b new
 * tokens) and the cache tokens kv_indices[kv_indptr[b] .. kv_indptr[b+1]-1]
 * (kv_len_b, the new tokens' own KV being the last q_len_b of them, written
 * before the call).  Query token i of request b sees the first n_i of them:
 *   causal != 0:  n_i = clamp(kv_len_b - q_len_b + i + 1, 0, kv_len_b)
 *   causal == 0:  n_i = kv_len_b
 * and, with K[t,:] = scale * e4m3fn(kv_pool[slot_t, :]) over those n_i tokens,
 *   out[qo_indptr[b] + i, h, :] = sum_t softmax_t(sm_scale * <q[qo_indptr[b] + i, h, :], K[t, :]>) * K[t, 0:512]
 * (BF16, round-to-nearest-even); n_i = 0 gives a zero row.  One token per
 * request (q_len_b = 1) is the decode of mla_decode_fp8.
 *   q           uint16 [total_q, num_heads, 576]   BF16, read
 *   kv_pool     uint8  [num_slots, 576]            E4M3FN bytes, read
 *   qo_indptr   int32  [batch + 1]  0 = qo_indptr[0] <= ... <= qo_indptr[batch] <= total_q
 *   kv_indptr   int32  [batch + 1]  0 = kv_indptr[0] <= ... <= kv_indptr[batch] <= total_kv
 *   kv_indices  int32  [total_kv]   slot ids in [0, num_slots)
 *   out         uint16 [total_q, num_heads, 512]   BF16, written (rows of
 *                                     requests in the indptr ranges only)
 *   workspace   at least mla_extend_fp8_workspace_bytes(batch, num_heads,
 *               total_q) bytes of scratch (no initialisation needed,
 *               garbage afterwards; NULL allowed when total_q == 0)
 *   1 <= batch, 1 <= num_heads <= FP8MLA_MAX_HEADS, 0 <= total_q < 2^23,
 *   total_q * num_heads <= 2^31 - 1,
 *   0 <= total_kv <= 2^31 - 1; num_slots >= 1 when total_kv > 0;
 *   scale finite > 0, sm_scale finite.
 * Work is organised in blocks of T query tokens of one request (T = 4 for
 * num_heads <= 16, 2 for <= 32, else 1), each reading its visible tokens in
 * 64-token tiles.  With NB = ceil(total_q / T) the call also requires
 *   batch + NB <= 2^25   and   (NB + 1) * ceil(total_kv / 64) + batch + NB <= 2^28,
 * a bound on the tiles read that holds for every index layout with these
 * sizes (e.g. a single causal prefill of up to ~128k tokens at 64 or more
 * heads, 4x that at 16 heads); larger calls return FP8MLA_ERR_BAD_SHAPE and
 * launch nothing.  Every accepted call writes every row of `out` it owns.
 * The index arrays are read on the device only.  Out-of-range indptr
 * entries are clamped into [0, total_q] / [0, total_kv] (a wrong row, never
 * an out-of-bounds access); with a decreasing indptr every row may come out
 * zero.
 */
int mla_extend_fp8(const uint16_t* q, const uint8_t* kv_pool, int64_t num_slots,
                   const int32_t* qo_indptr, const int32_t* kv_indptr, const int32_t* kv_indices,
                   int64_t total_q, int64_t total_kv, int32_t batch, int32_t num_heads,
                   float scale, float sm_scale, int32_t causal, uint16_t* out, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Workspace size in bytes for mla_extend_fp8 (0 when total_q == 0 or on bad
 * arguments); depends on batch, num_heads, total_q and the device's compute
 * unit count: O(batch + total_q) bytes of per-block records plus a fixed
 * partial-result area of two pieces per compute unit and head row. */
size_t mla_extend_fp8_workspace_bytes(int32_t batch, int32_t num_heads, int64_t total_q);

/*
 * fp8mla_check_indices -- on-device check of the index contract that the
 * reading calls assume but cannot afford to verify on their hot path.  They
 * clamp out-of-range entries (a wrong row, never an out-of-bounds access),
 * so a broken layout would otherwise fail silently -- the failure mode "The
 * KV Cache Cast Bottleneck" warns about (Assumptions, assumption 5: a
 * fallback that silently does nothing masks configuration errors).
 *
 * Checks, on the device, without a host read of the arrays:
 *   indptr[0] == 0, indptr[b] <= indptr[b+1], indptr[batch] == total, and
 *   0 <= indices[i] < num_slots for i < total.
 *   indptr    int32 [batch + 1] (NULL: only the slot ids are checked, as for
 *             gather_cast_fp8_bf16's index list)
 *   indices   int32 [total] (NULL: only indptr is checked, as for an extend
 *             call's qo_indptr against total_q)
 *   status    int32 [4] on the device, written: [0] FP8MLA_CHECK_* flags (0 =
 *             contract holds), [1] first request b with indptr[b+1] <
 *             indptr[b], [2] first position of an out-of-range slot id (both
 *             INT32_MAX if none), [3] number of out-of-range slot ids.
 * batch >= 1 when indptr is given; 0 <= total <= 2^31 - 1; num_slots >= 1
 * when indices are given.  Enqueues small kernels on `stream`, no sync.
 *
 * Debug build.  The library built with FP8MLA_DEBUG=1 (libfp8mla_debug.so,
 * same ABI) runs these checks inside every reading call -- mla_decode_fp8,
 * mla_decode_fp8_noalloc, mla_decode_bf16, mla_extend_fp8 (qo_indptr against
 * total_q, kv_indptr and kv_indices against total_kv) and
 * gather_cast_fp8_bf16 -- before its own kernels, accumulating into one
 * sticky status per device that fp8mla_debug_status reads.
 */
#define FP8MLA_CHECK_INDPTR_START 1  /* indptr[0] != 0                        */
#define FP8MLA_CHECK_INDPTR_ORDER 2  /* indptr decreases somewhere            */
#define FP8MLA_CHECK_INDPTR_END 4    /* indptr[batch] != total                */
#define FP8MLA_CHECK_SLOT_RANGE 8    /* a slot id outside [0, num_slots)      */
int fp8mla_check_indices(const int32_t* indptr, int32_t batch, int64_t total,
                         const int32_t* indices, int64_t num_slots, int32_t* status,
                         void* stream);

/*
 * fp8mla_debug_status -- debug build only: waits for the current device to
 * finish all work, copies its accumulated check status (layout as above)
 * into host memory status_out[4], and if `reset` clears it.  The release
 * build returns FP8MLA_ERR_NOT_DEBUG.
 */
int fp8mla_debug_status(int32_t* status_out, int32_t reset);

/* Static description of a status code; never NULL. */
const char* fp8mla_status_string(int status);

/* ABI version of this library (bumped on incompatible changes). */
int fp8mla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8MLA_H */
