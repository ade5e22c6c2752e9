// C ABI front end: argument checks, split planning, workspace carving,
// launches.  Nothing here touches the device before every host-side check
// has passed, so a failing call enqueues nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <limits>
#include <string>
#include <vector>

#include "../../include/pagedkv.h"
#include "pkv_launch.h"

namespace {

thread_local std::string g_err;

pkv_status fail(pkv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

pkv_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PKV_OK;
  return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kNumCUs = 256;          // MI355X compute units
constexpr int kMaxGridYZ = 65535;

pkv_status check_cache(const pkv_cache_desc* c) {
  if (!c) return fail(PKV_ERR_INVALID_ARG, "cache descriptor is NULL");
  if (!c->k_pool || !c->v_pool) return fail(PKV_ERR_INVALID_ARG, "k_pool/v_pool is NULL");
  if (c->num_pages <= 0 || c->num_kv_heads <= 0)
    return fail(PKV_ERR_INVALID_ARG, "num_pages (%d) and num_kv_heads (%d) must be positive",
                c->num_pages, c->num_kv_heads);
  if (c->kv_dtype < PKV_F32 || c->kv_dtype > PKV_INT8)
    return fail(PKV_ERR_INVALID_ARG, "kv_dtype %d is not a pkv_dtype", c->kv_dtype);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", c->head_dim);
  // Any power of two from 16 (a 16-token tile never straddles two pages) to
  // 256 tokens.
  if (c->page_size < 16 || c->page_size > 256 || (c->page_size & (c->page_size - 1)) != 0)
    return fail(PKV_ERR_UNSUPPORTED, "page_size %d (supported: 16, 32, 64, 128, 256)",
                c->page_size);
  const bool coded = c->kv_dtype == PKV_FP8_E4M3FN || c->kv_dtype == PKV_INT8;
  if (coded && (!c->k_scale || !c->v_scale))
    return fail(PKV_ERR_INVALID_ARG, "an fp8 or int8 cache needs k_scale and v_scale");
  if (!coded && (c->k_scale || c->v_scale))
    return fail(PKV_ERR_INVALID_ARG, "k_scale/v_scale are only for an fp8 or int8 cache");
  return PKV_OK;
}

pkv_status check_qo_dtypes(const pkv_cache_desc* c, int32_t q_dtype, int32_t out_dtype) {
  const bool ok = (c->kv_dtype == PKV_F32 && q_dtype == PKV_F32 && out_dtype == PKV_F32) ||
                  (c->kv_dtype == PKV_BF16 && q_dtype == PKV_BF16 && out_dtype == PKV_BF16) ||
                  ((c->kv_dtype == PKV_FP8_E4M3FN || c->kv_dtype == PKV_INT8) &&
                   q_dtype == PKV_BF16 && out_dtype == PKV_BF16);
  if (!ok)
    return fail(PKV_ERR_UNSUPPORTED, "dtype combination q=%d kv=%d out=%d not supported", q_dtype,
                c->kv_dtype, out_dtype);
  return PKV_OK;
}

pkv_status check_heads(const pkv_cache_desc* c, int32_t num_q_heads) {
  if (num_q_heads <= 0 || num_q_heads % c->num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                num_q_heads, c->num_kv_heads);
  const int G = num_q_heads / c->num_kv_heads;
  if (G > 16) return fail(PKV_ERR_UNSUPPORTED, "query group size %d > 16", G);
  if (c->num_kv_heads > kMaxGridYZ) return fail(PKV_ERR_UNSUPPORTED, "too many KV heads");
  return PKV_OK;
}

pkv::CacheView view(const pkv_cache_desc* c) {
  pkv::CacheView v;
  v.k_pool = c->k_pool;
  v.v_pool = c->v_pool;
  v.k_pool_w = c->k_pool;
  v.v_pool_w = c->v_pool;
  v.k_scale = c->k_scale;
  v.v_scale = c->v_scale;
  v.num_pages = c->num_pages;
  v.num_kv_heads = c->num_kv_heads;
  v.page_size = c->page_size;
  v.head_dim = c->head_dim;
  v.kv_dtype = c->kv_dtype;
  return v;
}

int32_t ceil_div(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }

int32_t default_split(const pkv_cache_desc* c, int32_t num_seqs, int32_t num_q_heads,
                      int32_t max_len) {
  const int gran = std::max(16, (int)c->page_size);
  const int64_t pairs = (int64_t)std::max(1, num_seqs) * c->num_kv_heads;
  const int G = num_q_heads / c->num_kv_heads;
  int split;
  if (G >= 3 && c->kv_dtype != PKV_F32) {
    // Matrix-core path: long ranges amortise each work item's start-up,
    // but the grid must keep enough items.  With only the longest context
    // known, the expected item count assumes contexts average half of it.
    // (A range's block-table slice, at most 512 entries, is staged in LDS.)
    const bool coded = c->kv_dtype == PKV_FP8_E4M3FN || c->kv_dtype == PKV_INT8;
    split = 512;
    if (coded) {
      // 8-bit codes: the longest range, in steps of 1024 tokens up to 16384,
      // that still leaves about 5/3 items per workgroup slot (three per CU,
      // 768 in all) when contexts spread evenly up to the longest, i.e.
      // max_len / (2 split) + 1/2 ranges per sequence and KV head.  A decode
      // that has the GPU to itself takes its items longest first, which
      // balances fewer, longer items: on 128 sequences of 1024..16384 tokens
      // (8 KV heads) this picks 10240, ahead of 8192, 9216, 11264 and 12288.
      for (int s = 16384; s >= 1024; s -= 1024) {
        if (s / c->page_size + 2 > 512) continue;
        const double items =
            (double)pairs * ((double)std::max(1, max_len) / (2.0 * s) + 0.5);
        if (items >= 1280.0) {
          split = s;
          break;
        }
      }
    } else {
      // 16-bit caches: ranges of 512 tokens up to 1 MiB of K+V per KV head
      // and item (2048 tokens at head_dim 128) while ~2048 items remain.
      while (split < 2048 && (2 * split) / c->page_size + 2 <= 512 &&
             pairs * ceil_div(std::max(1, max_len), 2 * split) / 2 >= 2048)
        split *= 2;
    }
  } else {
    // Vector path: 1 MiB of 16-bit K+V per KV head and item (2048 tokens at
    // head_dim 128), 1024 tokens of other formats (8-bit codes measured no
    // better with longer ranges); shorter ranges when the batch would give
    // fewer than ~8 items per CU, never below 256 tokens (the merge would cost
    // more than the parallelism gains).
    split = c->kv_dtype == PKV_BF16 ? 2048 : 1024;
    if (c->head_dim == 64) split *= 2;
    const int floor_split = 256;
    while (split / 2 >= floor_split && pairs * ceil_div(std::max(1, max_len), split) < 8 * kNumCUs)
      split /= 2;
  }
  split = std::max(gran, split / gran * gran);
  if (max_len <= split) split = std::max(gran, ceil_div(std::max(1, max_len), gran) * gran);
  return split;
}

pkv_status resolve_split(const pkv_cache_desc* c, int32_t num_seqs, int32_t num_q_heads,
                         int32_t max_len, int32_t split_tokens, int32_t* out) {
  if (split_tokens == 0) {
    *out = default_split(c, num_seqs, num_q_heads, max_len);
    return PKV_OK;
  }
  if (split_tokens < 0 || split_tokens % c->page_size != 0 || split_tokens % 16 != 0)
    return fail(PKV_ERR_INVALID_ARG, "split_tokens %d must be a positive multiple of page_size %d",
                split_tokens, c->page_size);
  *out = split_tokens;
  return PKV_OK;
}

size_t workspace_bytes(const pkv_cache_desc* c, int32_t num_seqs, int32_t num_q_heads,
                       int32_t max_len, int32_t split) {
  const int32_t ms = ceil_div(std::max(0, max_len), split);
  if (ms <= 1 || num_seqs <= 0) return 0;
  // acc [rows][Hq][ms][D] + (m, l) [rows][Hq][ms][2], float32, + the work
  // list {count, 0, (row, range) x rows*ms}, int32; each 256-byte aligned
  const size_t n = (size_t)num_seqs * num_q_heads * ms;
  const size_t acc = (n * c->head_dim * 4 + 255) / 256 * 256;
  const size_t ml = (n * 2 * 4 + 255) / 256 * 256;
  const size_t list = ((2 + 2 * (size_t)num_seqs * ms) * 4 + 255) / 256 * 256;
  return acc + ml + list;
}

// The work-list area of a decode workspace laid out by workspace_bytes.
int32_t* decode_list_area(const pkv::AttnArgs& a) {
  const size_t n = (size_t)a.num_rows * a.num_q_heads * a.max_splits;
  const size_t acc = (n * a.c.head_dim * 4 + 255) / 256 * 256;
  const size_t ml = (n * 2 * 4 + 255) / 256 * 256;
  return reinterpret_cast<int32_t*>(reinterpret_cast<char*>(a.ws_acc) + acc + ml);
}

struct DecodeSetup {
  pkv::AttnArgs a;
};

pkv_status prepare_decode(const pkv_cache_desc* cache, const void* q, int32_t q_dtype, void* out,
                          int32_t out_dtype, float* lse, const int32_t* block_tables,
                          int32_t bt_stride, const int32_t* context_lens, int32_t num_seqs,
                          int32_t num_q_heads, int32_t max_context_len, float sm_scale,
                          int32_t split_tokens, const void* workspace, size_t workspace_bytes_in,
                          bool need_q, pkv::AttnArgs* a) {
  pkv_status st;
  if ((st = check_cache(cache)) != PKV_OK) return st;
  if ((st = check_qo_dtypes(cache, q_dtype, out_dtype)) != PKV_OK) return st;
  if ((st = check_heads(cache, num_q_heads)) != PKV_OK) return st;
  if (num_seqs < 0 || max_context_len < 0)
    return fail(PKV_ERR_INVALID_ARG, "num_seqs %d / max_context_len %d negative", num_seqs,
                max_context_len);
  if (num_seqs > kMaxGridYZ) return fail(PKV_ERR_UNSUPPORTED, "num_seqs %d > %d", num_seqs, kMaxGridYZ);
  if (num_seqs > 0) {
    if ((need_q && !q) || !out || !context_lens || (need_q && !block_tables))
      return fail(PKV_ERR_INVALID_ARG, "q/out/block_tables/context_lens must not be NULL");
    if (need_q && bt_stride <= 0) return fail(PKV_ERR_INVALID_ARG, "bt_stride %d", bt_stride);
    if (need_q && (int64_t)bt_stride * cache->page_size < max_context_len)
      return fail(PKV_ERR_INVALID_ARG, "max_context_len %d exceeds bt_stride*page_size %lld",
                  max_context_len, (long long)bt_stride * cache->page_size);
  }
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f))
    return fail(PKV_ERR_INVALID_ARG, "sm_scale must be finite and positive");
  int32_t split;
  if ((st = resolve_split(cache, num_seqs, num_q_heads, max_context_len, split_tokens, &split)) !=
      PKV_OK)
    return st;
  const size_t need = workspace_bytes(cache, num_seqs, num_q_heads, max_context_len, split);
  if (need > 0 && (!workspace || workspace_bytes_in < need))
    return fail(PKV_ERR_INVALID_ARG, "workspace of %zu bytes needed, %zu given", need,
                workspace_bytes_in);
  const int32_t ms = std::max(1, ceil_div(std::max(0, max_context_len), split));
  if (ms > kMaxGridYZ)
    return fail(PKV_ERR_UNSUPPORTED, "%d context ranges per sequence (max %d)", ms, kMaxGridYZ);
  std::memset(a, 0, sizeof *a);
  a->c = view(cache);
  a->q = q;
  a->out = out;
  a->lse = lse;
  a->bt = block_tables;
  a->bt_stride = bt_stride;
  a->context_lens = context_lens;
  a->num_rows = num_seqs;
  a->num_q_heads = num_q_heads;
  a->split_tokens = split;
  a->max_splits = ms;
  a->sm_scale = sm_scale;
  a->page_shift = __builtin_ctz((unsigned)cache->page_size);
  if (need > 0) {
    char* w = static_cast<char*>(const_cast<void*>(workspace));
    const size_t n = (size_t)num_seqs * num_q_heads * ms;
    a->ws_acc = reinterpret_cast<float*>(w);
    a->ws_ml = reinterpret_cast<float*>(w + (n * cache->head_dim * 4 + 255) / 256 * 256);
  }
  return PKV_OK;
}

// Prefill key ranges.  Matrix-core path: about 3/5 of the longest context,
// at least 1024 keys.  Rows of the longest requests then split into two
// uneven ranges — halving the longest serial walk, which bounds a step whose
// contexts differ widely — while shorter requests stay in one range and need
// no merge.  Contexts of up to 1024 keys take one range.  F32 caches
// (generic path) always take one range.
int32_t split_for_keys(int32_t max_total, bool one_range) {
  const int32_t one = std::max<int32_t>(64, (max_total + 63) / 64 * 64);
  if (one_range) return one;
  const int32_t part = (int32_t)(((int64_t)max_total * 3 / 5 + 63) / 64 * 64);
  return std::min<int32_t>(one, std::max<int32_t>(1024, part));
}

// One key range per row — no partials to write and merge — pays once the
// call has enough work that heaviest-first order balances it anyway: when
// the least work the call can have (in tiles of 128 rows x 32 keys) keeps
// every workgroup slot of the device (two per CU, 256 CUs) busy for at
// least twice the longest item, a row's walk over max_keys keys.  A causal
// sequence of n tokens at G query heads per KV head costs G n^2 / 8192 tiles
// per KV head.
constexpr long long kPrefillSlots = 2LL * 256;

bool one_range_pays(long double min_tiles, int32_t max_keys) {
  return min_tiles >= 2.0L * kPrefillSlots * ((max_keys + 31) / 32);
}

long double causal_tiles(long double n_sq, int32_t num_q_heads, int32_t num_kv_heads) {
  const int32_t G = num_kv_heads > 0 ? num_q_heads / num_kv_heads : 0;
  return (long double)num_kv_heads * G * n_sq / 8192.0L;
}

// Chunked prefill: the least work is the longest chunk with nothing cached
// before it (the host knows neither the other chunks nor the cached lengths).
// A range's block-table slice must fit the kernel's LDS copy (512 entries).
int32_t default_prefill_split(const pkv_cache_desc* c, int32_t num_q_heads, int32_t max_chunk,
                              int32_t max_total) {
  const int32_t whole = std::max<int32_t>(64, (max_total + 63) / 64 * 64);
  if (c->kv_dtype != PKV_F32 && whole / c->page_size + 1 <= 512 &&
      one_range_pays(causal_tiles((long double)max_chunk * max_chunk, num_q_heads,
                                  c->num_kv_heads), max_total))
    return whole;
  const int32_t split = split_for_keys(max_total, c->kv_dtype == PKV_F32);
  if (c->kv_dtype == PKV_F32) return split;
  // at most 511 pages per range (multiple of 64 tokens)
  const int32_t cap = std::max<int32_t>(64, 511 * c->page_size / 64 * 64);
  return std::min(split, cap);
}

size_t ranges_ws_bytes(int32_t head_dim, int32_t num_q_tokens, int32_t num_q_heads, int32_t ms) {
  if (ms <= 1 || num_q_tokens <= 0) return 0;
  const size_t n = (size_t)num_q_tokens * num_q_heads * ms;
  const size_t acc = (n * head_dim * 4 + 255) / 256 * 256;
  const size_t ml = (n * 2 * 4 + 255) / 256 * 256;
  return acc + ml;
}

size_t prefill_ws_bytes(const pkv_cache_desc* c, int32_t num_q_tokens, int32_t num_q_heads,
                        int32_t ms) {
  return ranges_ws_bytes(c->head_dim, num_q_tokens, num_q_heads, ms);
}

// Host checks of a context-attention call (contiguous bf16 q/k/v); fills `a`
// (pointers included when given) and *need_out with the workspace bytes.
pkv_status prepare_context(const void* q, const void* k, const void* v, int32_t dtype, void* out,
                           float* lse, const int32_t* cu_seqlens, int32_t num_seqs,
                           int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t max_seqlen, float sm_scale,
                           int32_t split_tokens, bool check_ptrs, pkv::AttnArgs* a,
                           size_t* need_out) {
  if (dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "context attention takes bf16 q/k/v/out (dtype %d)", dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", head_dim);
  if (num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "num_q_heads %d must be a positive multiple of num_kv_heads %d",
                num_q_heads, num_kv_heads);
  if (num_q_heads / num_kv_heads > 16)
    return fail(PKV_ERR_UNSUPPORTED, "group size %d > 16", num_q_heads / num_kv_heads);
  if (num_seqs < 0 || num_tokens < 0 || max_seqlen < 0 || split_tokens < 0)
    return fail(PKV_ERR_INVALID_ARG, "negative size");
  if (num_seqs > kMaxGridYZ) return fail(PKV_ERR_UNSUPPORTED, "num_seqs %d > %d", num_seqs, kMaxGridYZ);
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f))
    return fail(PKV_ERR_INVALID_ARG, "sm_scale must be finite and positive");
  std::memset(a, 0, sizeof *a);
  a->c.k_pool = k;
  a->c.v_pool = v;
  a->c.num_kv_heads = num_kv_heads;
  a->c.head_dim = head_dim;
  a->c.page_size = 16;
  a->c.kv_dtype = PKV_BF16;
  a->prefill = 1;
  a->contiguous = 1;
  a->num_rows = num_seqs;
  a->num_tokens = num_tokens;
  a->max_chunk = max_seqlen;
  a->num_q_heads = num_q_heads;
  a->max_splits = 1;
  a->split_tokens = 64;
  if (need_out) *need_out = 0;
  if (num_seqs == 0 || num_tokens == 0) return PKV_OK;
  if (max_seqlen <= 0) return fail(PKV_ERR_INVALID_ARG, "max_seqlen must be positive");
  // Whole prompts: num_tokens over num_seqs sequences cost at least
  // num_tokens^2 / num_seqs (squared lengths, Cauchy-Schwarz).
  const bool one = one_range_pays(
      causal_tiles((long double)num_tokens * num_tokens / num_seqs, num_q_heads, num_kv_heads),
      max_seqlen);
  const int32_t split = split_tokens ? split_tokens
                        : one ? std::max<int32_t>(64, (max_seqlen + 63) / 64 * 64)
                              : split_for_keys(max_seqlen, false);
  if (split % 64 != 0)
    return fail(PKV_ERR_INVALID_ARG, "split_tokens %d is not a positive multiple of 64", split);
  const int32_t ms = ceil_div(max_seqlen, split);
  if (ms > kMaxGridYZ) return fail(PKV_ERR_UNSUPPORTED, "%d key ranges per row", ms);
  a->split_tokens = split;
  a->max_splits = std::max(1, ms);
  if (pkv::prefill_mfma_grid(*a) > 0x7FFFFFFFLL) return fail(PKV_ERR_UNSUPPORTED, "grid too large");
  const size_t need = ranges_ws_bytes(head_dim, num_tokens, num_q_heads, a->max_splits);
  if (need_out) *need_out = need;
  if (!check_ptrs) return PKV_OK;
  if (!q || !k || !v || !out || !cu_seqlens)
    return fail(PKV_ERR_INVALID_ARG, "context attention pointers must not be NULL");
  a->q = q;
  a->out = out;
  a->lse = lse;
  a->cu_q = cu_seqlens;
  a->sm_scale = sm_scale;
  return PKV_OK;
}

// Shape checks shared by the prefill call and its planning functions; fills
// the size fields of `a` (pointers are left NULL).
pkv_status prepare_prefill(const pkv_cache_desc* cache, int32_t q_dtype, int32_t out_dtype,
                           int32_t num_reqs, int32_t num_q_tokens, int32_t num_q_heads,
                           int32_t max_chunk_len, int32_t max_total_len, int32_t split_tokens,
                           pkv::AttnArgs* a) {
  pkv_status st;
  if ((st = check_cache(cache)) != PKV_OK) return st;
  if ((st = check_qo_dtypes(cache, q_dtype, out_dtype)) != PKV_OK) return st;
  if ((st = check_heads(cache, num_q_heads)) != PKV_OK) return st;
  if (num_reqs < 0 || num_q_tokens < 0 || max_chunk_len < 0 || max_total_len < 0 ||
      split_tokens < 0)
    return fail(PKV_ERR_INVALID_ARG, "negative size");
  std::memset(a, 0, sizeof *a);
  a->c = view(cache);
  a->num_rows = num_reqs;
  a->num_tokens = num_q_tokens;
  a->max_chunk = max_chunk_len;
  a->num_q_heads = num_q_heads;
  a->prefill = 1;
  a->page_shift = __builtin_ctz((unsigned)cache->page_size);
  a->max_splits = 1;
  a->split_tokens = 64;
  if (num_q_tokens == 0 || num_reqs == 0) return PKV_OK;
  if (max_chunk_len <= 0) return fail(PKV_ERR_INVALID_ARG, "max_chunk_len must be positive");
  if (num_reqs > kMaxGridYZ) return fail(PKV_ERR_UNSUPPORTED, "num_reqs %d > %d", num_reqs, kMaxGridYZ);
  if (max_total_len < max_chunk_len)
    return fail(PKV_ERR_INVALID_ARG, "max_total_len %d < max_chunk_len %d", max_total_len,
                max_chunk_len);
  const int32_t split =
      split_tokens ? split_tokens
                   : default_prefill_split(cache, num_q_heads, max_chunk_len, max_total_len);
  if (split % 64 != 0)
    return fail(PKV_ERR_INVALID_ARG, "split_tokens %d is not a positive multiple of 64", split);
  const int32_t ms = ceil_div(max_total_len, split);
  if (ms > kMaxGridYZ)
    return fail(PKV_ERR_UNSUPPORTED, "%d key ranges per row (max %d)", ms, kMaxGridYZ);
  a->split_tokens = split;
  a->max_splits = std::max(1, ms);
  if (!pkv::prefill_mfma_supported(*a)) {
    // generic path: one workgroup per (KV head, chunk row), one range
    if (ms > 1)
      return fail(PKV_ERR_UNSUPPORTED, "this cache takes one key range (split_tokens >= %d)",
                  max_total_len);
    if ((int64_t)num_reqs * max_chunk_len > kMaxGridYZ)
      return fail(PKV_ERR_UNSUPPORTED, "num_reqs * max_chunk_len > %d", kMaxGridYZ);
  } else if (pkv::prefill_mfma_grid(*a) > 0x7FFFFFFFLL) {
    return fail(PKV_ERR_UNSUPPORTED, "prefill grid too large");
  }
  return PKV_OK;
}

// New K/V rows come in the cache's own dtype for F32/BF16 caches and as
// float32 for 8-bit caches (encoded on the way in).
pkv_status check_append_input(const pkv_cache_desc* cache, int32_t in_dtype) {
  const int32_t want_in =
      (cache->kv_dtype == PKV_FP8_E4M3FN || cache->kv_dtype == PKV_INT8) ? PKV_F32 : cache->kv_dtype;
  if (in_dtype != want_in)
    return fail(PKV_ERR_UNSUPPORTED, "append into kv_dtype %d takes in_dtype %d, got %d",
                cache->kv_dtype, want_in, in_dtype);
  return PKV_OK;
}

pkv_status prepare_append(const pkv_cache_desc* cache, const void* k_new, const void* v_new,
                          int32_t in_dtype, const int32_t* cu_new_tokens,
                          const int32_t* start_pos, const int32_t* block_tables,
                          int32_t bt_stride, int32_t num_rows, int32_t num_new_tokens,
                          pkv::AppendArgs* a) {
  pkv_status st;
  if ((st = check_cache(cache)) != PKV_OK) return st;
  if ((st = check_append_input(cache, in_dtype)) != PKV_OK) return st;
  if (num_rows < 0 || num_new_tokens < 0)
    return fail(PKV_ERR_INVALID_ARG, "num_rows %d / num_new_tokens %d negative", num_rows,
                num_new_tokens);
  if (num_new_tokens > 0) {
    if (num_rows == 0) return fail(PKV_ERR_INVALID_ARG, "tokens given but no rows");
    if (!k_new || !v_new || !cu_new_tokens || !start_pos || !block_tables)
      return fail(PKV_ERR_INVALID_ARG, "append pointers must not be NULL");
    if (bt_stride <= 0) return fail(PKV_ERR_INVALID_ARG, "bt_stride %d", bt_stride);
  }
  std::memset(a, 0, sizeof *a);
  a->c = view(cache);
  a->k_new = k_new;
  a->v_new = v_new;
  a->in_dtype = in_dtype;
  a->cu = cu_new_tokens;
  a->start_pos = start_pos;
  a->bt = block_tables;
  a->bt_stride = bt_stride;
  a->num_rows = num_rows;
  a->num_tokens = num_new_tokens;
  return PKV_OK;
}

// All host checks of a prefill call; on success `a` is ready to launch and
// *need holds the workspace bytes it uses.
pkv_status prepare_prefill_call(const pkv_cache_desc* cache, const void* q, int32_t q_dtype,
                                void* out, int32_t out_dtype, float* lse,
                                const int32_t* cu_q_lens, const int32_t* ctx_before,
                                const int32_t* block_tables, int32_t bt_stride, int32_t num_reqs,
                                int32_t num_q_tokens, int32_t num_q_heads, int32_t max_chunk_len,
                                int32_t max_total_len, float sm_scale, int32_t split_tokens,
                                void* workspace, size_t workspace_bytes_in, pkv::AttnArgs* a,
                                size_t* need_out = nullptr) {
  pkv_status st = prepare_prefill(cache, q_dtype, out_dtype, num_reqs, num_q_tokens, num_q_heads,
                                  max_chunk_len, max_total_len, split_tokens, a);
  if (st != PKV_OK) return st;
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f))
    return fail(PKV_ERR_INVALID_ARG, "sm_scale must be finite and positive");
  if (need_out) *need_out = 0;
  if (num_q_tokens == 0 || num_reqs == 0) return PKV_OK;
  if (!q || !out || !cu_q_lens || !ctx_before || !block_tables)
    return fail(PKV_ERR_INVALID_ARG, "prefill pointers must not be NULL");
  if (bt_stride <= 0) return fail(PKV_ERR_INVALID_ARG, "bt_stride %d", bt_stride);
  if ((int64_t)bt_stride * cache->page_size < max_total_len)
    return fail(PKV_ERR_INVALID_ARG, "max_total_len %d exceeds bt_stride*page_size %lld",
                max_total_len, (long long)bt_stride * cache->page_size);
  const size_t need = prefill_ws_bytes(cache, num_q_tokens, num_q_heads, a->max_splits);
  if (need > 0 && (!workspace || workspace_bytes_in < need))
    return fail(PKV_ERR_INVALID_ARG, "workspace of %zu bytes needed, %zu given", need,
                workspace_bytes_in);
  a->q = q;
  a->out = out;
  a->lse = lse;
  a->bt = block_tables;
  a->bt_stride = bt_stride;
  a->cu_q = cu_q_lens;
  a->ctx_before = ctx_before;
  a->sm_scale = sm_scale;
  if (need > 0) {
    char* w = static_cast<char*>(workspace);
    const size_t n = (size_t)num_q_tokens * num_q_heads * a->max_splits;
    a->ws_acc = reinterpret_cast<float*>(w);
    a->ws_ml = reinterpret_cast<float*>(w + (n * cache->head_dim * 4 + 255) / 256 * 256);
  }
  if (need_out) *need_out = need;
  return PKV_OK;
}

pkv_status launch_prefill_call(const pkv::AttnArgs& a, hipStream_t s) {
  if (a.num_rows == 0 || a.num_tokens == 0) return PKV_OK;
  pkv_status st;
  if ((st = hip_status(pkv::launch_prefill(a, s), "paged_attn_chunked_prefill")) != PKV_OK)
    return st;
  return hip_status(pkv::launch_lse_merge(a, s), "paged_attn_chunked_prefill (merge)");
}

pkv_status launch_decode_call(const pkv::AttnArgs& a, hipStream_t s) {
  pkv_status st;
  if ((st = hip_status(pkv::launch_decode_partial(a, s), "paged_attn_decode (partial)")) != PKV_OK)
    return st;
  return hip_status(pkv::launch_lse_merge(a, s), "paged_attn_decode (merge)");
}

// Fork / join events of pkv_mixed_step, one pair per host thread and device
// (a thread issues one call at a time, so its pair is never shared).  They
// live until the process ends.
pkv_status step_events(hipEvent_t* fork, hipEvent_t* join) {
  struct Pair { int dev; hipEvent_t f, j; };
  thread_local std::vector<Pair> pairs;
  int dev = 0;
  pkv_status st;
  if ((st = hip_status(hipGetDevice(&dev), "mixed_step: current device")) != PKV_OK) return st;
  for (const Pair& p : pairs)
    if (p.dev == dev) { *fork = p.f; *join = p.j; return PKV_OK; }
  Pair p{dev, nullptr, nullptr};
  if ((st = hip_status(hipEventCreateWithFlags(&p.f, hipEventDisableTiming),
                       "mixed_step: create event")) != PKV_OK)
    return st;
  if ((st = hip_status(hipEventCreateWithFlags(&p.j, hipEventDisableTiming),
                       "mixed_step: create event")) != PKV_OK) {
    (void)hipEventDestroy(p.f);
    return st;
  }
  pairs.push_back(p);
  *fork = p.f;
  *join = p.j;
  return PKV_OK;
}

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

}  // namespace

namespace pkv_detail {
void set_error(const std::string& s) { g_err = s; }
}  // namespace pkv_detail

extern "C" {

const char* pkv_version(void) { return "0.1.0"; }

const char* pkv_last_error(void) { return g_err.c_str(); }

pkv_status pkv_kv_cache_append(const pkv_cache_desc* cache, const void* k_new, const void* v_new,
                               int32_t in_dtype, const int32_t* cu_new_tokens,
                               const int32_t* start_pos, const int32_t* block_tables,
                               int32_t bt_stride, int32_t num_rows, int32_t num_new_tokens,
                               void* stream) {
  pkv::AppendArgs a;
  pkv_status st = prepare_append(cache, k_new, v_new, in_dtype, cu_new_tokens, start_pos,
                                 block_tables, bt_stride, num_rows, num_new_tokens, &a);
  if (st != PKV_OK) return st;
  return hip_status(pkv::launch_append(a, static_cast<hipStream_t>(stream)), "kv_cache_append");
}

int32_t pkv_decode_split_tokens(const pkv_cache_desc* cache, int32_t num_seqs, int32_t num_q_heads,
                                int32_t max_context_len) {
  if (check_cache(cache) != PKV_OK || check_heads(cache, num_q_heads) != PKV_OK) return 0;
  if (num_seqs < 0 || max_context_len < 0) return 0;
  return default_split(cache, num_seqs, num_q_heads, max_context_len);
}

size_t pkv_decode_workspace_bytes(const pkv_cache_desc* cache, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t max_context_len,
                                  int32_t split_tokens) {
  if (check_cache(cache) != PKV_OK || check_heads(cache, num_q_heads) != PKV_OK) return 0;
  int32_t split;
  if (resolve_split(cache, num_seqs, num_q_heads, max_context_len, split_tokens, &split) != PKV_OK)
    return 0;
  return workspace_bytes(cache, num_seqs, num_q_heads, max_context_len, split);
}

pkv_status pkv_paged_attn_decode_partial(const pkv_cache_desc* cache, const void* q,
                                         int32_t q_dtype, void* out, int32_t out_dtype, float* lse,
                                         const int32_t* block_tables, int32_t bt_stride,
                                         const int32_t* context_lens, int32_t num_seqs,
                                         int32_t num_q_heads, int32_t max_context_len,
                                         float sm_scale, int32_t split_tokens, void* workspace,
                                         size_t workspace_bytes_in, void* stream) {
  pkv::AttnArgs a;
  pkv_status st = prepare_decode(cache, q, q_dtype, out, out_dtype, lse, block_tables, bt_stride,
                                 context_lens, num_seqs, num_q_heads, max_context_len, sm_scale,
                                 split_tokens, workspace, workspace_bytes_in, true, &a);
  if (st != PKV_OK) return st;
  return hip_status(pkv::launch_decode_partial(a, static_cast<hipStream_t>(stream)),
                    "paged_attn_decode (partial)");
}

pkv_status pkv_decode_work_list(const pkv_cache_desc* cache, const int32_t* context_lens,
                                int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                                int32_t split_tokens, void* workspace, size_t workspace_bytes_in,
                                void* stream) {
  pkv::AttnArgs a;
  // Only the shape arguments matter here: the shared checks get dtypes the
  // cache supports and a stand-in output pointer, which nothing writes.
  const int32_t qo = cache && cache->kv_dtype == PKV_F32 ? PKV_F32 : PKV_BF16;
  pkv_status st = prepare_decode(cache, nullptr, qo, const_cast<int32_t*>(context_lens), qo,
                                 nullptr, nullptr, 0, context_lens, num_seqs, num_q_heads,
                                 max_context_len, 1.0f, split_tokens, workspace,
                                 workspace_bytes_in, false, &a);
  if (st != PKV_OK) return st;
  if (!a.ws_acc || !pkv::decode_plan_useful(a)) return PKV_OK;   // the call walks its grid
  const pkv::DecodeListArgs l{context_lens, a.num_rows, a.split_tokens, a.max_splits,
                              decode_list_area(a)};
  return hip_status(pkv::launch_decode_list(l, static_cast<hipStream_t>(stream)),
                    "decode_work_list");
}

pkv_status pkv_paged_attn_decode_partial_listed(const pkv_cache_desc* cache, const void* q,
                                                int32_t q_dtype, void* out, int32_t out_dtype,
                                                float* lse, const int32_t* block_tables,
                                                int32_t bt_stride, const int32_t* context_lens,
                                                int32_t num_seqs, int32_t num_q_heads,
                                                int32_t max_context_len, float sm_scale,
                                                int32_t split_tokens, void* workspace,
                                                size_t workspace_bytes_in, void* stream) {
  pkv::AttnArgs a;
  pkv_status st = prepare_decode(cache, q, q_dtype, out, out_dtype, lse, block_tables, bt_stride,
                                 context_lens, num_seqs, num_q_heads, max_context_len, sm_scale,
                                 split_tokens, workspace, workspace_bytes_in, true, &a);
  if (st != PKV_OK) return st;
  if (a.ws_acc && pkv::decode_plan_useful(a)) a.plan = decode_list_area(a);
  return hip_status(pkv::launch_decode_partial(a, static_cast<hipStream_t>(stream)),
                    "paged_attn_decode (partial, listed)");
}

pkv_status pkv_lse_merge(const pkv_cache_desc* cache, void* out, int32_t out_dtype, float* lse,
                         const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                         int32_t max_context_len, int32_t split_tokens, const void* workspace,
                         size_t workspace_bytes_in, void* stream) {
  pkv::AttnArgs a;
  const int32_t q_dtype = cache && cache->kv_dtype == PKV_F32 ? PKV_F32 : PKV_BF16;
  pkv_status st = prepare_decode(cache, nullptr, q_dtype, out, out_dtype, lse, nullptr, 0,
                                 context_lens, num_seqs, num_q_heads, max_context_len, 1.0f,
                                 split_tokens, workspace, workspace_bytes_in, false, &a);
  if (st != PKV_OK) return st;
  return hip_status(pkv::launch_lse_merge(a, static_cast<hipStream_t>(stream)), "lse_merge");
}

pkv_status pkv_paged_attn_decode(const pkv_cache_desc* cache, const void* q, int32_t q_dtype,
                                 void* out, int32_t out_dtype, float* lse,
                                 const int32_t* block_tables, int32_t bt_stride,
                                 const int32_t* context_lens, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t max_context_len, float sm_scale,
                                 int32_t split_tokens, void* workspace, size_t workspace_bytes_in,
                                 void* stream) {
  pkv::AttnArgs a;
  pkv_status st = prepare_decode(cache, q, q_dtype, out, out_dtype, lse, block_tables, bt_stride,
                                 context_lens, num_seqs, num_q_heads, max_context_len, sm_scale,
                                 split_tokens, workspace, workspace_bytes_in, true, &a);
  if (st != PKV_OK) return st;
  return launch_decode_call(a, static_cast<hipStream_t>(stream));
}

pkv_status pkv_decode_step(const pkv_cache_desc* cache, const void* k_new, const void* v_new,
                           int32_t in_dtype, const void* q, int32_t q_dtype, void* out,
                           int32_t out_dtype, float* lse, const int32_t* block_tables,
                           int32_t bt_stride, const int32_t* context_lens, int32_t num_seqs,
                           int32_t num_q_heads, int32_t max_context_len, float sm_scale,
                           int32_t split_tokens, void* workspace, size_t workspace_bytes_in,
                           void* stream) {
  pkv::AttnArgs a;
  pkv_status st = prepare_decode(cache, q, q_dtype, out, out_dtype, lse, block_tables, bt_stride,
                                 context_lens, num_seqs, num_q_heads, max_context_len, sm_scale,
                                 split_tokens, workspace, workspace_bytes_in, true, &a);
  if (st != PKV_OK) return st;
  if ((st = check_append_input(cache, in_dtype)) != PKV_OK) return st;
  if (num_seqs > 0 && (!k_new || !v_new))
    return fail(PKV_ERR_INVALID_ARG, "k_new / v_new must not be NULL");
  a.new_k = k_new;
  a.new_v = v_new;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // A call with enough work items takes them longest first from a work list
  // (one single-workgroup launch before the attention, as
  // pkv_decode_work_list); smaller calls stay one attention launch.
  if (a.ws_acc && pkv::decode_plan_useful(a)) {
    a.plan = decode_list_area(a);
    const pkv::DecodeListArgs l{context_lens, a.num_rows, a.split_tokens, a.max_splits, a.plan};
    if ((st = hip_status(pkv::launch_decode_list(l, s), "decode_step (work list)")) != PKV_OK)
      return st;
  }
  return launch_decode_call(a, s);
}

pkv_status pkv_paged_attn_chunked_prefill(const pkv_cache_desc* cache, const void* q,
                                          int32_t q_dtype, void* out, int32_t out_dtype,
                                          float* lse, const int32_t* cu_q_lens,
                                          const int32_t* ctx_before, const int32_t* block_tables,
                                          int32_t bt_stride, int32_t num_reqs,
                                          int32_t num_q_tokens, int32_t num_q_heads,
                                          int32_t max_chunk_len, int32_t max_total_len,
                                          float sm_scale, int32_t split_tokens, void* workspace,
                                          size_t workspace_bytes_in, void* stream) {
  pkv::AttnArgs a;
  pkv_status st = prepare_prefill_call(cache, q, q_dtype, out, out_dtype, lse, cu_q_lens,
                                       ctx_before, block_tables, bt_stride, num_reqs,
                                       num_q_tokens, num_q_heads, max_chunk_len, max_total_len,
                                       sm_scale, split_tokens, workspace, workspace_bytes_in, &a);
  if (st != PKV_OK) return st;
  return launch_prefill_call(a, static_cast<hipStream_t>(stream));
}

int32_t pkv_prefill_split_tokens(const pkv_cache_desc* cache, int32_t num_reqs,
                                 int32_t num_q_heads, int32_t max_chunk_len,
                                 int32_t max_total_len) {
  if (check_cache(cache) != PKV_OK || check_heads(cache, num_q_heads) != PKV_OK) return 0;
  if (num_reqs < 0 || max_chunk_len < 0 || max_total_len < max_chunk_len) return 0;
  return default_prefill_split(cache, num_q_heads, max_chunk_len, max_total_len);
}

size_t pkv_prefill_workspace_bytes(const pkv_cache_desc* cache, int32_t num_reqs,
                                   int32_t num_q_tokens, int32_t num_q_heads,
                                   int32_t max_chunk_len, int32_t max_total_len,
                                   int32_t split_tokens) {
  pkv::AttnArgs a;
  const int32_t dt = cache && cache->kv_dtype == PKV_F32 ? PKV_F32 : PKV_BF16;
  if (prepare_prefill(cache, dt, dt, num_reqs, num_q_tokens, num_q_heads, max_chunk_len,
                      max_total_len, split_tokens, &a) != PKV_OK)
    return 0;
  return prefill_ws_bytes(cache, num_q_tokens, num_q_heads, a.max_splits);
}

pkv_status pkv_mixed_step(const pkv_cache_desc* cache, const pkv_append_batch* ap,
                          const pkv_decode_batch* dp, const pkv_prefill_batch* pp,
                          float sm_scale, void* stream, void* side_stream) {
  pkv::AppendArgs aa;
  pkv::AttnArgs da, pa;
  pkv_status st;
  if (ap && (st = prepare_append(cache, ap->k_new, ap->v_new, ap->in_dtype, ap->cu_new_tokens,
                                 ap->start_pos, ap->block_tables, ap->bt_stride, ap->num_rows,
                                 ap->num_new_tokens, &aa)) != PKV_OK)
    return st;
  size_t dneed = 0, pneed = 0;
  if (dp) {
    if ((st = prepare_decode(cache, dp->q, dp->q_dtype, dp->out, dp->out_dtype, dp->lse,
                             dp->block_tables, dp->bt_stride, dp->context_lens, dp->num_seqs,
                             dp->num_q_heads, dp->max_context_len, sm_scale, dp->split_tokens,
                             dp->workspace, dp->workspace_bytes, true, &da)) != PKV_OK)
      return st;
    dneed = workspace_bytes(cache, dp->num_seqs, dp->num_q_heads, dp->max_context_len,
                            da.split_tokens);
  }
  if (pp && (st = prepare_prefill_call(cache, pp->q, pp->q_dtype, pp->out, pp->out_dtype,
                                       pp->lse, pp->cu_q_lens, pp->ctx_before, pp->block_tables,
                                       pp->bt_stride, pp->num_reqs, pp->num_q_tokens,
                                       pp->num_q_heads, pp->max_chunk_len, pp->max_total_len,
                                       sm_scale, pp->split_tokens, pp->workspace,
                                       pp->workspace_bytes, &pa, &pneed)) != PKV_OK)
    return st;
  if (dp && pp && side_stream && ranges_overlap(dp->workspace, dneed, pp->workspace, pneed))
    return fail(PKV_ERR_INVALID_ARG, "decode and prefill workspaces overlap (they run concurrently)");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipStream_t side = static_cast<hipStream_t>(side_stream);
  const bool fork = dp && pp && side && side != s;
  // A decode with enough work items that has the GPU to itself gets a work
  // list (longest ranges first), written by one extra workgroup of the
  // append launch, which precedes the decode on `stream`: no further launch
  // and no cross-stream wait.  Beside a concurrent prefill the plain grid
  // order is kept: its long items first hold slots the prefill needs
  // (measured 141 against 130 us on the 8B mixed step).
  if (ap && dp && !fork && da.ws_acc && pkv::decode_plan_useful(da)) {
    da.plan = decode_list_area(da);
    aa.list = pkv::DecodeListArgs{dp->context_lens, da.num_rows, da.split_tokens, da.max_splits,
                                  da.plan};
  }
  if (ap && (st = hip_status(pkv::launch_append(aa, s), "mixed_step: append")) != PKV_OK) return st;
  if (!fork) {
    // The decode (partial + merge) completes before the prefill starts: its
    // work list and partials are consumed before the prefill writes its own,
    // so the two parts may share one workspace here.
    if (dp && (st = launch_decode_call(da, s)) != PKV_OK) return st;
    if (pp && (st = launch_prefill_call(pa, s)) != PKV_OK) return st;
    return PKV_OK;
  }
  hipEvent_t ev_fork, ev_join;
  if ((st = step_events(&ev_fork, &ev_join)) != PKV_OK) return st;
  if ((st = hip_status(hipEventRecord(ev_fork, s), "mixed_step: fork")) != PKV_OK) return st;
  if ((st = hip_status(hipStreamWaitEvent(side, ev_fork, 0), "mixed_step: fork")) != PKV_OK) return st;
  // Decode first: with the direct-to-LDS prefill this packs as well as the
  // prefill-first order on a warm cache and 4% better from HBM (8B mixed
  // step: 156 against 163 us with the caches flushed).
  if ((st = launch_decode_call(da, s)) != PKV_OK) return st;
  if ((st = launch_prefill_call(pa, side)) != PKV_OK) return st;
  if ((st = hip_status(hipEventRecord(ev_join, side), "mixed_step: join")) != PKV_OK) return st;
  return hip_status(hipStreamWaitEvent(s, ev_join, 0), "mixed_step: join");
}

pkv_status pkv_context_fmha(const void* q, const void* k, const void* v, int32_t dtype, void* out,
                            float* lse, const int32_t* cu_seqlens, int32_t num_seqs,
                            int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t max_seqlen, float sm_scale,
                            int32_t split_tokens, void* workspace, size_t workspace_bytes_in,
                            void* stream) {
  pkv::AttnArgs a;
  size_t need = 0;
  pkv_status st = prepare_context(q, k, v, dtype, out, lse, cu_seqlens, num_seqs, num_tokens,
                                  num_q_heads, num_kv_heads, head_dim, max_seqlen, sm_scale,
                                  split_tokens, true, &a, &need);
  if (st != PKV_OK) return st;
  if (num_seqs == 0 || num_tokens == 0) return PKV_OK;
  if (need > 0 && (!workspace || workspace_bytes_in < need))
    return fail(PKV_ERR_INVALID_ARG, "workspace of %zu bytes needed, %zu given", need,
                workspace_bytes_in);
  if (need > 0) {
    char* w = static_cast<char*>(workspace);
    const size_t n = (size_t)num_tokens * num_q_heads * a.max_splits;
    a.ws_acc = reinterpret_cast<float*>(w);
    a.ws_ml = reinterpret_cast<float*>(w + (n * head_dim * 4 + 255) / 256 * 256);
  }
  return launch_prefill_call(a, static_cast<hipStream_t>(stream));
}

size_t pkv_context_fmha_workspace_bytes(int32_t num_seqs, int32_t num_tokens,
                                        int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t max_seqlen,
                                        int32_t split_tokens) {
  pkv::AttnArgs a;
  size_t need = 0;
  if (prepare_context(nullptr, nullptr, nullptr, PKV_BF16, nullptr, nullptr, nullptr, num_seqs,
                      num_tokens, num_q_heads, num_kv_heads, head_dim, max_seqlen, 1.0f,
                      split_tokens, false, &a, &need) != PKV_OK)
    return 0;
  return need;
}

pkv_status pkv_validate_block_tables(const pkv_cache_desc* cache, const int32_t* block_tables,
                                     int32_t bt_stride, const int32_t* lens, int32_t num_seqs,
                                     void* stream) {
  pkv_status st;
  if ((st = check_cache(cache)) != PKV_OK) return st;
  if (num_seqs < 0 || bt_stride <= 0) return fail(PKV_ERR_INVALID_ARG, "num_seqs/bt_stride");
  if (num_seqs == 0) return PKV_OK;
  if (!block_tables || !lens) return fail(PKV_ERR_INVALID_ARG, "NULL block_tables/lens");
  std::vector<int32_t> bt((size_t)num_seqs * bt_stride), ln(num_seqs);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = hip_status(hipMemcpyAsync(bt.data(), block_tables, bt.size() * 4, hipMemcpyDeviceToHost, s),
                       "validate: copy block tables")) != PKV_OK)
    return st;
  if ((st = hip_status(hipMemcpyAsync(ln.data(), lens, ln.size() * 4, hipMemcpyDeviceToHost, s),
                       "validate: copy lengths")) != PKV_OK)
    return st;
  if ((st = hip_status(hipStreamSynchronize(s), "validate: synchronize")) != PKV_OK) return st;
  const int64_t cap = (int64_t)bt_stride * cache->page_size;
  for (int32_t r = 0; r < num_seqs; ++r) {
    if (ln[r] < 0 || ln[r] > cap)
      return fail(PKV_ERR_BAD_BLOCK_TABLE, "row %d: length %d outside [0, %lld]", r, ln[r],
                  (long long)cap);
    const int32_t used = ceil_div(ln[r], cache->page_size);
    for (int32_t i = 0; i < used; ++i) {
      const int32_t id = bt[(size_t)r * bt_stride + i];
      if (id < 0 || id >= cache->num_pages)
        return fail(PKV_ERR_BAD_BLOCK_TABLE, "row %d: entry %d = %d outside [0, %d)", r, i, id,
                    cache->num_pages);
    }
  }
  return PKV_OK;
}

pkv_status pkv_fp8_e4m3fn_to_f32(const uint8_t* codes, float* out, int64_t n, void* stream) {
  if (n < 0) return fail(PKV_ERR_INVALID_ARG, "n negative");
  if (n > 0 && (!codes || !out)) return fail(PKV_ERR_INVALID_ARG, "NULL pointer");
  if (n > 0 && (reinterpret_cast<uintptr_t>(codes) & 3))
    return fail(PKV_ERR_INVALID_ARG, "codes must be 4-byte aligned");
  return hip_status(pkv::launch_fp8_to_f32(codes, out, n, static_cast<hipStream_t>(stream)),
                    "fp8_e4m3fn_to_f32");
}

}  // extern "C"
