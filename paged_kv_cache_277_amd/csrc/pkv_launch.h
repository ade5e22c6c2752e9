// Internal launch interface between the C ABI front end (api.cpp) and the
// HIP kernels.  Host-side checks are done before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

struct CacheView {
  const void* k_pool;
  const void* v_pool;
  void* k_pool_w;
  void* v_pool_w;
  const float* k_scale;
  const float* v_scale;
  int32_t num_pages, num_kv_heads, page_size, head_dim, kv_dtype;
};

// Inputs of a decode work list (see decode_list.h): built by one extra
// workgroup of the append launch that precedes the decode in a mixed step.
struct DecodeListArgs {
  const int32_t* context_lens;
  int32_t num_rows, split_tokens, max_splits;
  int32_t* list;                 // {count, 0, (row, range) x count}; null: no list
};

struct AppendArgs {
  CacheView c;
  const void* k_new;
  const void* v_new;
  int32_t in_dtype;
  const int32_t* cu;
  const int32_t* start_pos;
  const int32_t* bt;
  int32_t bt_stride, num_rows, num_tokens;
  DecodeListArgs list;           // list.list null unless a decode list is wanted
};

// Rows of an attention launch are either decode sequences (one query each)
// or prefill chunk rows (query i of request r).
struct AttnArgs {
  CacheView c;
  const void* q;
  void* out;
  float* lse;
  const int32_t* bt;
  int32_t bt_stride;
  const int32_t* context_lens;   // decode
  const int32_t* cu_q;           // prefill
  const int32_t* ctx_before;     // prefill
  int32_t num_rows;              // decode: sequences; prefill: requests
  int32_t num_tokens;            // prefill: packed query tokens (rows of out / workspace)
  int32_t max_chunk;             // prefill: longest chunk
  int32_t num_q_heads;
  int32_t split_tokens;
  int32_t max_splits;
  float sm_scale;
  float* ws_acc;                 // [rows][Hq][max_splits][D]   (prefill rows: tokens)
  float* ws_ml;                  // [rows][Hq][max_splits][2]
  // decode: work list {count, 0, (row, range) x count}, longest ranges
  // first (decode_list.h); null: the grid walks (row, range) itself
  int32_t* plan;
  int32_t prefill;
  int32_t contiguous;            // prefill over contiguous K/V [tokens][Hkv][D] (no pages)
  int32_t page_shift;            // log2(page_size)
  // fused decode step: each sequence's new token (position L - 1), packed
  // [num_seqs][Hkv][D], written by the decode launch itself; null otherwise
  const void* new_k;
  const void* new_v;
};

hipError_t launch_append(const AppendArgs& a, hipStream_t s);
hipError_t launch_decode_partial(const AttnArgs& a, hipStream_t s);
hipError_t launch_lse_merge(const AttnArgs& a, hipStream_t s);
// Decode work list: whether a call is worth one, and the grid of a decode
// launch that reads it, (KV heads, y, z) with y * z >= rows * max_splits.
bool decode_plan_useful(const AttnArgs& a);
dim3 decode_plan_grid(const AttnArgs& a);
hipError_t launch_decode_list(const DecodeListArgs& a, hipStream_t s);   // one workgroup
hipError_t launch_prefill(const AttnArgs& a, hipStream_t s);
// Grouped-query decode on the matrix cores (G >= 3, bf16 or fp8 KV).
bool decode_mfma_supported(const AttnArgs& a);
hipError_t launch_decode_partial_mfma(const AttnArgs& a, hipStream_t s);
// Chunked prefill on the matrix cores (bf16 queries, bf16 or fp8 KV).
bool prefill_mfma_supported(const AttnArgs& a);
long long prefill_mfma_grid(const AttnArgs& a);    // workgroups of one launch
hipError_t launch_prefill_mfma(const AttnArgs& a, hipStream_t s);
hipError_t launch_fp8_to_f32(const uint8_t* codes, float* out, int64_t n, hipStream_t s);

}  // namespace pkv
