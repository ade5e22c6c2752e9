/*
 * pagedkv.h — C ABI of the paged KV-cache attention library for AMD Instinct
 * MI355X (gfx950).
 *
 * What the library computes (reference pages, by title and section):
 *   - Paged KV cache: keys and values in fixed-size pages of one shared pool,
 *     allocated on demand; a per-sequence block table maps logical page i to a
 *     physical page, so storage is non-contiguous; repeated prompt prefixes may
 *     share pages.  "TensorRT-LLM框架解析与高性能推理优化实践" §4.2 (KV缓存管理细节:
 *     KVCacheBlock / KVCacheManager with allocate_blocks, free_blocks,
 *     get_block_table) and §6.2 (Paged Attention优化).
 *   - Attention: scaled dot-product softmax attention ("TensorRT-LLM性能调优：提升LLM
 *     推理效率", layer-fusion discussion: fused MHA with scaled dot-product
 *     attention and a causal mask), computed flash-style with a running max
 *     and running sum (first page, §6.1 Flash Attention实现).
 *   - KV-cache quantization with one scale per attention head, dequantised
 *     inside the attention kernel (first page, §7.2 KV Cache量化).
 *   - Chunked context: long prompts processed chunk by chunk, interleaved with
 *     decode requests (first page, §5.3 分块上下文处理); in-flight batching of
 *     mixed-length requests ("TensorRT-LLM内核融合与动态批处理", In-flight Batching
 *     section).
 *   - Launches are asynchronous and stream-ordered (first page, §2.2 GPU内存传输机制).
 *
 * Conventions for every call below:
 *   - Pointers named as device pointers are HIP device memory owned by the
 *     caller.  The library allocates no device memory and keeps no device state
 *     between calls; scratch space is passed in as `workspace` (the one
 *     exception: the fixed per-GPU array of pkv_paged_attn_decode_noalloc).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Launch
 *     calls enqueue work and return without synchronizing.
 *   - Host-side checks happen before anything is launched: on a non-OK status
 *     nothing was enqueued and pkv_last_error() (thread-local) says why.
 *   - Device-resident values (block-table entries, lengths, offsets) are trusted
 *     on the fast path: they must satisfy the documented ranges.  An entry
 *     point that reads them only on the device cannot check them;
 *     pkv_validate_block_tables() checks them (synchronously) for debugging.
 *
 * Layouts (row-major, element type given by the dtype):
 *   K pool, V pool : [num_pages][num_kv_heads][page_size][head_dim]
 *                    token t of a sequence with block-table row `bt` lives in
 *                    page bt[t / page_size], slot t % page_size.
 *   block tables   : int32 [rows][bt_stride]; unused entries may hold -1.
 *   decode q/out   : [num_seqs][num_q_heads][head_dim]
 *   packed tokens  : [num_tokens][heads][head_dim], rows laid end to end
 *                    (no padding), described by int32 offsets cu[rows+1].
 *   lse            : float [rows][num_q_heads], natural-log log-sum-exp of the
 *                    scaled scores (-inf for an empty context).
 *   Query head h reads KV head h / (num_q_heads / num_kv_heads).
 */
#ifndef PAGEDKV_H_
#define PAGEDKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1,     /* null pointer, negative size, bad combination */
  PKV_ERR_UNSUPPORTED = 2,     /* valid but not implemented (dtype, head_dim, page size) */
  PKV_ERR_OUT_OF_PAGES = 3,    /* allocator: not enough free pages (nothing taken) */
  PKV_ERR_BAD_BLOCK_TABLE = 4, /* validate: an entry outside the pool or a length too long */
  PKV_ERR_HIP = 5              /* a HIP runtime call failed; message has the HIP error */
} pkv_status;

typedef enum pkv_dtype {
  PKV_F32 = 0,
  PKV_BF16 = 1,
  PKV_FP8_E4M3FN = 2,          /* OCP e4m3fn: bias 7, max 448, no inf, NaN = 0x7F/0xFF */
  PKV_INT8 = 3                 /* symmetric int8 code c in [-127, 127] standing for c * scale
                                  ("TensorRT-LLM框架解析与高性能推理优化实践" §7.2; the KV-cache
                                  quantization plugin of "4. TensorRT-LLM架构与核心组件…" §4.3) */
} pkv_dtype;

/* One layer's paged cache.  Supported: kv_dtype F32, BF16, FP8_E4M3FN or INT8;
 * head_dim 64 or 128; page_size 16, 32, 64, 128 or 256; num_kv_heads >= 1.
 * k_scale / v_scale: device float[num_kv_heads], required iff kv_dtype is
 * FP8_E4M3FN or INT8 (stored code = encode(x / scale), dequantised value =
 * code * scale; the division in float32; fp8 rounds to nearest even and
 * saturates at +-448, int8 rounds half to even and saturates at +-127, NaN
 * encodes as 0). */
typedef struct pkv_cache_desc {
  void* k_pool;
  void* v_pool;
  const float* k_scale;
  const float* v_scale;
  int32_t num_pages;
  int32_t num_kv_heads;
  int32_t page_size;
  int32_t head_dim;
  int32_t kv_dtype;            /* a pkv_dtype */
} pkv_cache_desc;

/* Library version string (static storage). */
const char* pkv_version(void);

/* Message for the last non-OK status returned on this thread (static,
 * thread-local storage; overwritten by the next failing call). */
const char* pkv_last_error(void);

/* ------------------------------------------------------------------------ *
 * Host page allocator — "TensorRT-LLM框架解析与高性能推理优化实践" §4.2 (KVCacheManager:
 * allocate_blocks / free_blocks; block reuse and prefix sharing) and §5.2
 * (OutOfMemoryError when no pages remain).  CPU only; every call is
 * serialised by an internal mutex.  Page ids are 0..num_pages-1.  A page's
 * refcount is 1 after allocation, +1 per share, -1 per free; it returns to the
 * free list at 0.  Which free ids an allocation receives is unspecified.
 * ------------------------------------------------------------------------ */

/* Create an allocator for `num_pages` (> 0) pages; *out_alloc receives the handle. */
pkv_status pkv_allocator_create(int32_t num_pages, void** out_alloc);

/* Destroy an allocator (NULL is ignored). */
void pkv_allocator_destroy(void* alloc);

/* Allocate `n` (>= 0) pages into host array out_ids[n].  All or nothing:
 * PKV_ERR_OUT_OF_PAGES leaves the allocator unchanged. */
pkv_status pkv_alloc_pages(void* alloc, int32_t n, int32_t* out_ids);

/* Add one reference to each of the n allocated pages ids[n] (shared prefix).
 * PKV_ERR_INVALID_ARG (and no change) if an id is out of range or free. */
pkv_status pkv_share_pages(void* alloc, int32_t n, const int32_t* ids);

/* Drop one reference from each of ids[n]; pages reaching 0 become free.
 * PKV_ERR_INVALID_ARG (and no change) if an id is out of range, free, or
 * would be released more times than it is referenced. */
pkv_status pkv_free_pages(void* alloc, int32_t n, const int32_t* ids);

/* Number of free pages, or -1 for a NULL handle. */
int32_t pkv_num_free_pages(const void* alloc);

/* Reference count of page `id` (0 = free), or -1 if the handle or id is invalid. */
int32_t pkv_page_refcount(const void* alloc, int32_t id);

/* ------------------------------------------------------------------------ *
 * kv_cache_append — scatter new tokens' K and V into their page slots
 * ("TensorRT-LLM内核融合与动态批处理", In-flight Batching section: a request's KV
 * is placed as it joins and grows; first page §7.2 for the fp8 path).
 *
 * k_new, v_new : device [num_new_tokens][num_kv_heads][head_dim], packed rows.
 *                in_dtype must equal the cache dtype for F32/BF16 caches (a copy);
 *                an FP8 cache takes F32 input and stores
 *                e4m3fn(x / scale[head]): IEEE float32 division, round to
 *                nearest even, saturating to +-448; NaN stays NaN.  An INT8
 *                cache takes F32 input and stores the integer nearest to
 *                x / scale[head] (float32 division, ties to even),
 *                saturated to [-127, 127]; NaN stores 0.
 * cu_new_tokens: device int32[num_rows+1], cu[0] = 0, non-decreasing,
 *                cu[num_rows] = num_new_tokens.
 * start_pos    : device int32[num_rows]; row r's token i goes to logical
 *                position start_pos[r] + i of block-table row r.
 * block_tables : device int32[num_rows][bt_stride]; every page the new tokens
 *                land in must be a valid id.
 * Pages written must not be shared with another row that reads them in the
 * same stream step (shared prefixes are full pages, never appended to).
 * Bytes of the pool other than the written slots are left unchanged.
 * ------------------------------------------------------------------------ */
pkv_status pkv_kv_cache_append(const pkv_cache_desc* cache,
                               const void* k_new, const void* v_new, int32_t in_dtype,
                               const int32_t* cu_new_tokens, const int32_t* start_pos,
                               const int32_t* block_tables, int32_t bt_stride,
                               int32_t num_rows, int32_t num_new_tokens, void* stream);

/* ------------------------------------------------------------------------ *
 * paged_attn_decode — one query token per sequence over its paged context
 * ("TensorRT-LLM框架解析与高性能推理优化实践" §6.2: the kernel walks the sequence's
 * block table; §6.1: running max / running sum).  Work is split along the
 * context into ranges of `split_tokens` tokens (flash-decoding); each range
 * leaves a partial (max, sum, unnormalised accumulator) in the workspace and
 * a log-sum-exp merge combines them.  Sequences that fit in one range are
 * written directly.
 *
 * Supported (q_dtype, kv_dtype, out_dtype): (F32, F32, F32), (BF16, BF16, BF16),
 * (BF16, FP8_E4M3FN, BF16), (BF16, INT8, BF16).  8-bit codes are widened
 * exactly to bf16 in the kernel; the per-head scales multiply the scores and
 * the output.  num_q_heads must be a multiple of num_kv_heads
 * with group size G = num_q_heads / num_kv_heads <= 16.
 *
 * q            : device [num_seqs][num_q_heads][head_dim]
 * out          : device [num_seqs][num_q_heads][head_dim]
 * lse          : device float[num_seqs][num_q_heads] or NULL
 * block_tables : device int32[num_seqs][bt_stride]
 * context_lens : device int32[num_seqs], 0 <= L <= min(max_context_len,
 *                bt_stride * page_size); L counts the query's own token.
 *                L = 0 gives out = 0 and lse = -inf.
 * sm_scale     : score scale, finite and > 0 (1/sqrt(head_dim) for standard
 *                attention).
 * split_tokens : context range per work item, a positive multiple of
 *                page_size; 0 selects pkv_decode_split_tokens().
 * workspace    : device scratch of at least pkv_decode_workspace_bytes(...)
 *                bytes (may be NULL when that size is 0); contents on entry
 *                are ignored.  It holds the partials and, for
 *                pkv_mixed_step, the decode work list.
 * ------------------------------------------------------------------------ */

/* Default split length for a decode batch: a multiple of page_size chosen
 * from the batch shape so that the launch has enough work items to fill the
 * device.  Pure host function; returns 0 on invalid arguments. */
int32_t pkv_decode_split_tokens(const pkv_cache_desc* cache, int32_t num_seqs,
                                int32_t num_q_heads, int32_t max_context_len);

/* Workspace bytes needed by a decode call with these arguments (split_tokens
 * resolved as in pkv_paged_attn_decode; 0 when no sequence can need more than
 * one range). */
size_t pkv_decode_workspace_bytes(const pkv_cache_desc* cache, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t max_context_len,
                                  int32_t split_tokens);

/* Partial pass followed by the merge pass. */
pkv_status pkv_paged_attn_decode(const pkv_cache_desc* cache,
                                 const void* q, int32_t q_dtype,
                                 void* out, int32_t out_dtype, float* lse,
                                 const int32_t* block_tables, int32_t bt_stride,
                                 const int32_t* context_lens, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t max_context_len,
                                 float sm_scale, int32_t split_tokens,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* The partial pass alone: writes out/lse of single-range sequences and the
 * workspace partials of the others.  pkv_lse_merge with the same arguments
 * completes the call. */
pkv_status pkv_paged_attn_decode_partial(const pkv_cache_desc* cache,
                                         const void* q, int32_t q_dtype,
                                         void* out, int32_t out_dtype, float* lse,
                                         const int32_t* block_tables, int32_t bt_stride,
                                         const int32_t* context_lens, int32_t num_seqs,
                                         int32_t num_q_heads, int32_t max_context_len,
                                         float sm_scale, int32_t split_tokens,
                                         void* workspace, size_t workspace_bytes,
                                         void* stream);

/* Decode work list for separate calls (pkv_mixed_step builds its own).
 * pkv_decode_work_list orders the (sequence, context range) work items of a
 * decode call with these arguments by token count, longest first, into the
 * work-list area of `workspace` (one single-workgroup kernel on `stream`;
 * it reads only context_lens).  pkv_paged_attn_decode_partial_listed, with
 * the same cache, context_lens contents, num_seqs, num_q_heads,
 * max_context_len, split_tokens and workspace, later on the same stream,
 * then takes its items in that order, so that the launch ends on its
 * shortest items; its results are bit for bit those of
 * pkv_paged_attn_decode_partial.  Calls of fewer than 1024 (sequence, range,
 * KV head) work items, or needing no workspace, use no list: the builder
 * then does nothing and the listed pass walks its grid as the plain one.
 * A list written for other arguments gives wrong results (items outside
 * the call are skipped, so nothing is accessed out of bounds).  Arguments
 * and errors as for pkv_paged_attn_decode_partial. */
pkv_status pkv_decode_work_list(const pkv_cache_desc* cache, const int32_t* context_lens,
                                int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                                int32_t split_tokens, void* workspace, size_t workspace_bytes,
                                void* stream);
pkv_status pkv_paged_attn_decode_partial_listed(const pkv_cache_desc* cache,
                                                const void* q, int32_t q_dtype,
                                                void* out, int32_t out_dtype, float* lse,
                                                const int32_t* block_tables, int32_t bt_stride,
                                                const int32_t* context_lens, int32_t num_seqs,
                                                int32_t num_q_heads, int32_t max_context_len,
                                                float sm_scale, int32_t split_tokens,
                                                void* workspace, size_t workspace_bytes,
                                                void* stream);

/* The log-sum-exp merge pass: for every sequence with more than one range,
 * M = max_s m_s, w_s = exp(m_s - M), out = sum_s w_s acc_s / sum_s w_s l_s,
 * lse = M + ln(sum_s w_s l_s).  Sequences with one range are untouched. */
pkv_status pkv_lse_merge(const pkv_cache_desc* cache, void* out, int32_t out_dtype, float* lse,
                         const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                         int32_t max_context_len, int32_t split_tokens,
                         const void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * decode_step — one generation step of a decode batch in one attention
 * launch: every sequence's newest token is written into its page slot and
 * the sequence's query attends its whole context, that token included.
 * Each step of in-flight batching places the new token's K/V as the request
 * grows ("TensorRT-LLM内核融合与动态批处理", In-flight Batching section;
 * "TensorRT-LLM框架解析与高性能推理优化实践" §4.2 and §6.2 for the block-table
 * write and walk), and joining the write to the attention kernel removes a
 * launch per step (Kernel Fusion section of "TensorRT-LLM内核融合与动态批处理";
 * layer-fusion paragraph of "TensorRT-LLM性能调优：提升LLM推理效率" on the
 * cost of each launch).
 *
 * Equivalent, bit for bit in pools, out and lse, to
 *   pkv_kv_cache_append(k_new, v_new, cu = {0, 1, .., num_seqs},
 *                       start_pos[s] = context_lens[s] - 1)
 * followed by pkv_paged_attn_decode with the remaining arguments, for
 * sequences with context_lens[s] >= 1; a sequence with context_lens[s] = 0
 * appends nothing and gets out = 0, lse = -inf.
 *
 * k_new, v_new : device [num_seqs][num_kv_heads][head_dim], the new token of
 *                each sequence (position context_lens[s] - 1 of block-table
 *                row s); in_dtype and the stored encoding as for
 *                pkv_kv_cache_append.  Row s is read only if
 *                context_lens[s] >= 1.
 * The remaining arguments, the supported dtypes, split_tokens, the
 * workspace and its size are those of pkv_paged_attn_decode.  The page that
 * receives a sequence's new token must not be shared with another sequence
 * of the call.  Calls of at least 1024 (sequence, range, KV head) work
 * items first write a longest-first work list into the workspace (one small
 * launch, as pkv_decode_work_list); smaller calls are one attention launch
 * (plus the merge when a sequence spans several ranges).
 * Errors: the checks of pkv_paged_attn_decode; in_dtype other than the
 * append's (PKV_ERR_UNSUPPORTED); k_new or v_new NULL with num_seqs > 0
 * (PKV_ERR_INVALID_ARG).  Nothing is launched on error.
 * ------------------------------------------------------------------------ */
pkv_status pkv_decode_step(const pkv_cache_desc* cache,
                           const void* k_new, const void* v_new, int32_t in_dtype,
                           const void* q, int32_t q_dtype,
                           void* out, int32_t out_dtype, float* lse,
                           const int32_t* block_tables, int32_t bt_stride,
                           const int32_t* context_lens, int32_t num_seqs,
                           int32_t num_q_heads, int32_t max_context_len,
                           float sm_scale, int32_t split_tokens,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * paged_attn_decode_noalloc — pkv_paged_attn_decode for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid allocation): the same kernels and results, with the
 * partials kept in a fixed device array of the library
 * (PKV_NOALLOC_SCRATCH_BYTES per GPU, held from module load until the
 * process ends) instead of a caller workspace.  The call itself allocates
 * nothing; its first call on a device looks up that device's array once.
 *
 * Arguments, supported types and results as for pkv_paged_attn_decode
 * without workspace / workspace_bytes.  A call whose partials
 * (pkv_decode_workspace_bytes with the same arguments) exceed
 * PKV_NOALLOC_SCRATCH_BYTES returns PKV_ERR_INVALID_ARG and launches nothing
 * (longer split_tokens need fewer partials).  Nothing in the array needs to
 * start at zero; it keeps the last call's contents.  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from several threads without ordering) race and give
 * wrong results; calls on one stream are ordered and safe.  The array used
 * is the current device's, so `stream` must belong to the current device;
 * a stream of another device returns PKV_ERR_INVALID_ARG.
 * ------------------------------------------------------------------------ */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
pkv_status pkv_paged_attn_decode_noalloc(const pkv_cache_desc* cache,
                                         const void* q, int32_t q_dtype,
                                         void* out, int32_t out_dtype, float* lse,
                                         const int32_t* block_tables, int32_t bt_stride,
                                         const int32_t* context_lens, int32_t num_seqs,
                                         int32_t num_q_heads, int32_t max_context_len,
                                         float sm_scale, int32_t split_tokens, void* stream);

/* ------------------------------------------------------------------------ *
 * paged_attn_chunked_prefill — causal attention of context chunks over the
 * pages already cached for their request plus the chunk itself
 * (first page §5.3 分块上下文处理; causal mask of the fused-MHA pseudocode in
 * "TensorRT-LLM性能调优：提升LLM推理效率").  The chunk's own K/V must already be
 * in the pages (pkv_kv_cache_append).  Row i of request r (absolute position
 * ctx_before[r] + i) attends keys 0 .. ctx_before[r] + i inclusive.
 *
 * As in decode, the keys are cut into ranges of split_tokens; a row whose
 * keys span several ranges gets per-range partials in the workspace and the
 * same log-sum-exp merge (launched by this call on the same stream).  Long
 * contexts so spread over many workgroups instead of one long serial walk.
 *
 * q, out        : device packed [num_q_tokens][num_q_heads][head_dim]
 * lse           : device float[num_q_tokens][num_q_heads] or NULL
 * cu_q_lens     : device int32[num_reqs+1], chunk row offsets, cu[0] = 0,
 *                 every chunk length <= max_chunk_len, cu[num_reqs] = num_q_tokens
 * ctx_before    : device int32[num_reqs], tokens cached before the chunk;
 *                 ctx_before[r] + chunk_len(r) <= max_total_len
 * max_total_len : host bound on ctx_before[r] + chunk_len(r) over the batch,
 *                 max_chunk_len <= max_total_len <= bt_stride * page_size
 * split_tokens  : key range per work item, a positive multiple of 64; 0
 *                 selects pkv_prefill_split_tokens().  F32 caches take one
 *                 range only (split_tokens >= max_total_len, or 0).  With
 *                 bf16 / 8-bit caches a range spans at most 511 pages
 *                 (split_tokens / page_size + 1 <= 512); a longer one
 *                 leaves only the one-range generic path, so several such
 *                 ranges give PKV_ERR_UNSUPPORTED.
 * workspace     : device scratch of at least pkv_prefill_workspace_bytes(...)
 *                 bytes (NULL when that is 0); contents on entry are ignored.
 * Supported dtypes as for decode.
 * ------------------------------------------------------------------------ */
pkv_status pkv_paged_attn_chunked_prefill(const pkv_cache_desc* cache,
                                          const void* q, int32_t q_dtype,
                                          void* out, int32_t out_dtype, float* lse,
                                          const int32_t* cu_q_lens, const int32_t* ctx_before,
                                          const int32_t* block_tables, int32_t bt_stride,
                                          int32_t num_reqs, int32_t num_q_tokens,
                                          int32_t num_q_heads, int32_t max_chunk_len,
                                          int32_t max_total_len, float sm_scale,
                                          int32_t split_tokens, void* workspace,
                                          size_t workspace_bytes, void* stream);

/* Default key range for a prefill batch (a multiple of 64).  One range
 * (no partials, no merge) for F32 caches, and for bf16 / 8-bit caches when
 * even the least work the batch can have — its longest chunk with nothing
 * cached — keeps the device's workgroup slots busy for twice the longest
 * row's walk over max_total_len keys (and the block-table slice of that
 * range fits the kernel's 512-entry copy); otherwise about 3/5 of
 * max_total_len (at least 1024), so the longest rows are cut in two.  Pure
 * host function; returns 0 on invalid arguments. */
int32_t pkv_prefill_split_tokens(const pkv_cache_desc* cache, int32_t num_reqs,
                                 int32_t num_q_heads, int32_t max_chunk_len,
                                 int32_t max_total_len);

/* Workspace bytes a prefill call with these arguments needs (split_tokens
 * resolved as in pkv_paged_attn_chunked_prefill; 0 for one range). */
size_t pkv_prefill_workspace_bytes(const pkv_cache_desc* cache, int32_t num_reqs,
                                   int32_t num_q_tokens, int32_t num_q_heads,
                                   int32_t max_chunk_len, int32_t max_total_len,
                                   int32_t split_tokens);

/* ------------------------------------------------------------------------ *
 * context_fmha — causal attention of whole prompts over their own contiguous
 * K/V, no pages (the fused multi-head attention of a context phase:
 * "TensorRT-LLM性能调优：提升LLM推理效率", layer fusion, fused MHA = scaled
 * dot-product attention with a causal mask; the context_fmha build option of
 * "如何用TensorRT-LLM和Triton Server实现LLM的高效推理？…" §2; the FMHA plugin of
 * "4. TensorRT-LLM架构与核心组件…" §4.3).  Token i of sequence s attends tokens
 * 0..i of s.  The same kernel as chunked prefill with K/V addressed directly,
 * key ranges and merge included.
 *
 * q, out     : device bf16 packed [num_tokens][num_q_heads][head_dim]
 * k, v       : device bf16 packed [num_tokens][num_kv_heads][head_dim]
 * dtype      : PKV_BF16 (the only supported type)
 * lse        : device float[num_tokens][num_q_heads] or NULL
 * cu_seqlens : device int32[num_seqs+1], cu[0] = 0, every length <= max_seqlen,
 *              cu[num_seqs] = num_tokens
 * split_tokens, workspace: as for pkv_paged_attn_chunked_prefill, with
 *              max_seqlen in place of max_total_len; the default (0) takes
 *              one range when the least work of num_tokens tokens over
 *              num_seqs prompts (num_tokens^2 / num_seqs squared lengths)
 *              keeps the device busy for twice the longest row's walk.
 * head_dim 64 or 128, num_q_heads a multiple of num_kv_heads, group <= 16.
 * ------------------------------------------------------------------------ */
pkv_status pkv_context_fmha(const void* q, const void* k, const void* v, int32_t dtype, void* out,
                            float* lse, const int32_t* cu_seqlens, int32_t num_seqs,
                            int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t max_seqlen, float sm_scale,
                            int32_t split_tokens, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Workspace bytes of a context_fmha call (0: one key range, none needed;
 * also 0 on invalid arguments). */
size_t pkv_context_fmha_workspace_bytes(int32_t num_seqs, int32_t num_tokens,
                                        int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t max_seqlen,
                                        int32_t split_tokens);

/* ------------------------------------------------------------------------ *
 * mixed_step — one in-flight batching step in one call: new tokens join the
 * cache, then decode sequences and prefill chunks attend it
 * ("TensorRT-LLM内核融合与动态批处理", In-flight Batching: requests at different
 * phases share a step; first page §5.3 for the chunks).  The three parts are
 * the arguments of pkv_kv_cache_append, pkv_paged_attn_decode and
 * pkv_paged_attn_chunked_prefill gathered in structs; any part may be NULL.
 *
 * Order: the append runs on `stream`; decode (partial + merge) and prefill
 * (+ merge) follow it.  With side_stream non-NULL (and different from
 * stream) the prefill runs on side_stream concurrently with the decode —
 * the decode reads HBM while the prefill keeps the matrix cores busy — and
 * `stream` waits for it before the call's work is complete; the fork and
 * join are stream events, so a graph captured from `stream` records all of
 * it.  Both streams belong to the current device.  With side_stream NULL (or
 * equal to stream) the parts run one after another on `stream`: append,
 * decode (partial + merge), then prefill (+ merge); the decode has consumed
 * its workspace before the prefill writes, so the two parts may then share
 * one workspace buffer.
 *
 * Decode work list: when the step has an append part and the decode does
 * not run beside a prefill, a decode of at least 1024 (sequence, context
 * range, KV head) work items takes its (sequence, range) items longest
 * first, so that the launch ends on its shortest items; one extra workgroup
 * of the append launch sorts them by token count (it reads only
 * context_lens).  The list lives in the decode workspace
 * (pkv_decode_workspace_bytes counts it).  Results are bit for bit those of
 * pkv_paged_attn_decode with the same arguments.
 *
 * Every part is checked on the host before anything is launched.  When the
 * two attention parts run concurrently their workspaces must not overlap
 * (PKV_ERR_INVALID_ARG).  The library keeps two events per host thread and
 * device for the fork and join, created on first use and kept until the
 * process ends; calls from one thread are ordered, calls from several
 * threads do not share events.
 * ------------------------------------------------------------------------ */
typedef struct {
  const void* k_new;
  const void* v_new;
  int32_t in_dtype;
  const int32_t* cu_new_tokens;
  const int32_t* start_pos;
  const int32_t* block_tables;
  int32_t bt_stride;
  int32_t num_rows;
  int32_t num_new_tokens;
} pkv_append_batch;

typedef struct {
  const void* q;
  int32_t q_dtype;
  void* out;
  int32_t out_dtype;
  float* lse;
  const int32_t* block_tables;
  int32_t bt_stride;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t max_context_len;
  int32_t split_tokens;
  void* workspace;
  size_t workspace_bytes;
} pkv_decode_batch;

typedef struct {
  const void* q;
  int32_t q_dtype;
  void* out;
  int32_t out_dtype;
  float* lse;
  const int32_t* cu_q_lens;
  const int32_t* ctx_before;
  const int32_t* block_tables;
  int32_t bt_stride;
  int32_t num_reqs;
  int32_t num_q_tokens;
  int32_t num_q_heads;
  int32_t max_chunk_len;
  int32_t max_total_len;
  int32_t split_tokens;
  void* workspace;
  size_t workspace_bytes;
} pkv_prefill_batch;

pkv_status pkv_mixed_step(const pkv_cache_desc* cache, const pkv_append_batch* append,
                          const pkv_decode_batch* decode, const pkv_prefill_batch* prefill,
                          float sm_scale, void* stream, void* side_stream);

/* ------------------------------------------------------------------------ *
 * Step scheduler with the KV-cache manager — host only, produces the block
 * tables and positions the kernels above consume
 * ("TensorRT-LLM框架解析与高性能推理优化实践" §4.2 KVCacheManager, §5.1
 * capacity / micro-batch scheduling, §5.2 LIFO preemption, §5.3 chunked
 * context, §4.1 slot manager).
 *
 * Per request: num_tokens = prompt + generated tokens, num_computed = tokens
 * with K/V in the cache.  pkv_sched_schedule plans one step:
 *   1. running requests, oldest admitted first, each computing its next
 *      prefill chunk (min(chunk_size, num_tokens - num_computed)) or, with
 *      one token pending, one decode token, within max_num_tokens per step.
 *      A request short of pages evicts the most recently admitted running
 *      request (possibly itself): its pages are freed and it returns to the
 *      front of the waiting queue, to be recomputed from its prefix on resume.
 *   2. waiting requests from the front, while they fit (max_batch_size
 *      running, the token budget, and pages: the next chunk's pages in the
 *      aggressive policy; every running request's remaining worst case plus
 *      the new one's in the conservative policy, which therefore never
 *      evicts).  Admission never evicts and never skips the queue front.
 * pkv_sched_commit then records the step as executed: num_computed advances,
 * a request whose cache caught up with num_tokens gains one generated token,
 * and one with max_new_tokens generated finishes (pages freed).
 *
 * A request whose worst case (prompt + max_new_tokens - 1 cached tokens)
 * cannot fit the pool beside the registered prefixes is refused with
 * PKV_ERR_OUT_OF_PAGES at pkv_sched_add_request.  Shared prefixes are whole
 * pages registered once (the caller fills their K/V); requests naming one
 * start with those pages (refcounted) and num_computed = the prefix length.
 * All functions are thread-safe (one mutex per scheduler).
 * ------------------------------------------------------------------------ */
typedef enum { PKV_SCHED_CONSERVATIVE = 0, PKV_SCHED_AGGRESSIVE = 1 } pkv_sched_policy;
typedef enum { PKV_WORK_PREFILL = 0, PKV_WORK_DECODE = 1 } pkv_work_kind;

typedef struct {
  int32_t num_pages;        /* cache pages managed */
  int32_t page_size;        /* tokens per page */
  int32_t max_batch_size;   /* running requests (compute slots) */
  int32_t max_num_tokens;   /* tokens computed per step, decode + prefill */
  int32_t chunk_size;       /* prefill tokens per request per step */
  int32_t policy;           /* pkv_sched_policy */
} pkv_sched_config;

typedef struct {
  int64_t req_id;
  int32_t slot;             /* compute slot, 0 .. max_batch_size-1 */
  int32_t kind;             /* pkv_work_kind */
  int32_t start_pos;        /* tokens already cached (= append start_pos) */
  int32_t num_tokens;       /* tokens appended and attended this step */
} pkv_sched_item;

typedef struct {
  int32_t num_tokens, num_computed, generated, num_pages, slot, running;
} pkv_sched_request_state;

typedef struct {
  int32_t waiting, running, free_pages;
  int64_t preemptions;      /* evictions since creation */
} pkv_sched_counts;

pkv_status pkv_sched_create(const pkv_sched_config* cfg, void** out_sched);
void       pkv_sched_destroy(void* sched);
/* Registers num_tokens (a positive multiple of page_size) of shared prefix;
 * out_pages receives its num_tokens / page_size page ids. */
pkv_status pkv_sched_add_prefix(void* sched, int64_t prefix_id, int32_t num_tokens,
                                int32_t* out_pages);
/* Fails while a request references the prefix. */
pkv_status pkv_sched_remove_prefix(void* sched, int64_t prefix_id);
/* Queues a request at the back of the waiting queue; prefix_id -1 = none
 * (else prompt_len counts the prefix and must exceed it). */
pkv_status pkv_sched_add_request(void* sched, int64_t req_id, int32_t prompt_len,
                                 int32_t max_new_tokens, int64_t prefix_id);
/* Plans one step into items[] (capacity >= max_batch_size) and lists the
 * requests evicted by it in preempted[] (capacity >= max_batch_size).
 * Must be followed by pkv_sched_commit before the next call.
 * PKV_ERR_OUT_OF_PAGES (nothing planned) when the queue front cannot be
 * admitted even into an empty batch. */
pkv_status pkv_sched_schedule(void* sched, pkv_sched_item* items, int32_t items_cap,
                              int32_t* num_items, int64_t* preempted, int32_t preempted_cap,
                              int32_t* num_preempted);
/* Copies up to cap page ids of the request's block table into out (may be
 * NULL) and returns its page count, or -1 for an unknown request. */
int32_t    pkv_sched_block_table(const void* sched, int64_t req_id, int32_t* out, int32_t cap);
/* Records the planned step as executed; finished[] (capacity >= items of the
 * step) receives the requests that completed and were removed. */
pkv_status pkv_sched_commit(void* sched, int64_t* finished, int32_t finished_cap,
                            int32_t* num_finished);
/* Removes a request early (stop token, cancellation) and frees its pages. */
pkv_status pkv_sched_finish(void* sched, int64_t req_id);
pkv_status pkv_sched_query(const void* sched, int64_t req_id, pkv_sched_request_state* out);
pkv_status pkv_sched_stats(const void* sched, pkv_sched_counts* out);

/* ------------------------------------------------------------------------ *
 * Utilities
 * ------------------------------------------------------------------------ */

/* Debug check of the block-table address map that every kernel above trusts
 * ("TensorRT-LLM框架解析与高性能推理优化实践" §4.2: get_block_table maps a
 * sequence's logical pages to physical ones; §6.2: the attention kernel
 * reaches each token through it, shared prefix pages included).
 * Synchronous on `stream`: copies block_tables and lens to the host and
 * checks 0 <= lens[s] <= bt_stride * page_size and that every entry covering
 * tokens 0..lens[s]-1 is in [0, num_pages).  PKV_ERR_BAD_BLOCK_TABLE names the
 * first offending row.  Device pointers; lens is int32[num_seqs]. */
pkv_status pkv_validate_block_tables(const pkv_cache_desc* cache, const int32_t* block_tables,
                                     int32_t bt_stride, const int32_t* lens, int32_t num_seqs,
                                     void* stream);

/* The in-kernel dequantisation of the fp8 KV cache on its own
 * ("TensorRT-LLM框架解析与高性能推理优化实践" §7.2: 8-bit KV codes dequantised
 * inside the attention kernel): decode n fp8 e4m3fn codes (device uint8[n],
 * 4-byte aligned) to float (device float[n]) with the conversion the
 * matrix-core attention kernels use (fp8 -> bf16, exact), so that it can be
 * checked against the format's definition. */
pkv_status pkv_fp8_e4m3fn_to_f32(const uint8_t* codes, float* out, int64_t n, void* stream);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* PAGEDKV_H_ */
