/* A plain C client of libpagedkv (no Python, no PyTorch in the process).
 *
 * Reads raw input files from a directory, places the given pool contents in
 * device memory, appends one decode step's new tokens with
 * pkv_kv_cache_append, runs pkv_paged_attn_decode on the default stream and
 * writes the pools and the outputs back as raw files:
 *
 *   meta.txt   num_pages num_kv_heads page_size head_dim kv_dtype
 *              num_seqs num_q_heads bt_stride max_context_len sm_scale
 *              step_rows step_tokens step_bt_stride in_dtype
 *   kpool.bin vpool.bin           pools before the step (storage format)
 *   kscale.bin vscale.bin         float[num_kv_heads] (8-bit caches only)
 *   knew.bin vnew.bin             [step_tokens][num_kv_heads][head_dim], in_dtype
 *   cu.bin start.bin stepbt.bin   int32 step metadata
 *   q.bin bt.bin lens.bin         decode query (bf16), block tables, lengths
 * Outputs: kpool_out.bin vpool_out.bin out.bin (bf16) lse.bin (float).
 *
 * With a file fused.txt beside them, knew.bin / vnew.bin hold one row per
 * sequence ([num_seqs][num_kv_heads][head_dim], the token at position
 * L - 1) and one pkv_decode_step call replaces the append and the decode.
 *
 * With a file pfmeta.txt (num_reqs num_q_tokens max_chunk_len max_total_len
 * pf_bt_stride) and pfq.bin pfcu.bin pfctx.bin pfbt.bin beside them, the
 * three parts (append, decode, chunked prefill) run instead as one
 * pkv_mixed_step call with the prefill on a second stream, filled in the
 * library's structs; pfout.bin (bf16) and pflse.bin (float) are written too.
 *
 * Exit status 0 on success; every library status and runtime error is checked
 * and reported with pkv_last_error(). */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pagedkv.h"

static const char* g_dir;

static void die(const char* what, const char* detail) {
  fprintf(stderr, "decode_client: %s: %s\n", what, detail ? detail : "");
  exit(1);
}

static void hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) die(what, hipGetErrorString(e));
}

static void pkv_check(pkv_status s, const char* what) {
  if (s != PKV_OK) die(what, pkv_last_error());
}

static int exists(const char* name) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", g_dir, name);
  FILE* f = fopen(path, "rb");
  if (f) fclose(f);
  return f != NULL;
}

static void* read_file(const char* name, size_t* size) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", g_dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) die("open", path);
  fseek(f, 0, SEEK_END);
  const long n = ftell(f);
  fseek(f, 0, SEEK_SET);
  void* buf = malloc(n > 0 ? (size_t)n : 1);
  if (!buf || (n > 0 && fread(buf, 1, (size_t)n, f) != (size_t)n)) die("read", path);
  fclose(f);
  *size = (size_t)n;
  return buf;
}

static void write_file(const char* name, const void* data, size_t n) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", g_dir, name);
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(data, 1, n, f) != n) die("write", path);
  fclose(f);
}

/* Copies a file to new device memory; returns the pointer, size in *n. */
static void* to_device(const char* name, size_t* n) {
  size_t size;
  void* host = read_file(name, &size);
  void* dev = NULL;
  if (size > 0) {
    hip_check(hipMalloc(&dev, size), "hipMalloc");
    hip_check(hipMemcpy(dev, host, size, hipMemcpyHostToDevice), "hipMemcpy H2D");
  }
  free(host);
  if (n) *n = size;
  return dev;
}

static void from_device(const char* name, const void* dev, size_t n) {
  void* host = malloc(n > 0 ? n : 1);
  if (!host) die("malloc", name);
  hip_check(hipMemcpy(host, dev, n, hipMemcpyDeviceToHost), "hipMemcpy D2H");
  write_file(name, host, n);
  free(host);
}

int main(int argc, char** argv) {
  if (argc != 2) die("usage", "decode_client DIR");
  g_dir = argv[1];
  size_t n;
  char* meta = (char*)read_file("meta.txt", &n);
  meta = (char*)realloc(meta, n + 1);
  meta[n] = 0;
  int num_pages, hkv, page, hd, kv_dtype, seqs, hq, bt_stride, max_len, step_rows, step_tokens,
      step_stride, in_dtype;
  float sm_scale;
  if (sscanf(meta, "%d %d %d %d %d %d %d %d %d %f %d %d %d %d", &num_pages, &hkv, &page, &hd,
             &kv_dtype, &seqs, &hq, &bt_stride, &max_len, &sm_scale, &step_rows, &step_tokens,
             &step_stride, &in_dtype) != 14)
    die("meta.txt", "14 fields expected");
  free(meta);
  printf("decode_client: %s (%d seqs, %d/%d heads, head_dim %d, page %d, kv dtype %d)\n",
         pkv_version(), seqs, hq, hkv, hd, page, kv_dtype);

  size_t pool_bytes;
  pkv_cache_desc cache;
  memset(&cache, 0, sizeof cache);
  cache.k_pool = to_device("kpool.bin", &pool_bytes);
  cache.v_pool = to_device("vpool.bin", NULL);
  if (kv_dtype == PKV_FP8_E4M3FN || kv_dtype == PKV_INT8) {
    cache.k_scale = (const float*)to_device("kscale.bin", NULL);
    cache.v_scale = (const float*)to_device("vscale.bin", NULL);
  }
  cache.num_pages = num_pages;
  cache.num_kv_heads = hkv;
  cache.page_size = page;
  cache.head_dim = hd;
  cache.kv_dtype = kv_dtype;

  /* the step's appends */
  void* knew = to_device("knew.bin", NULL);
  void* vnew = to_device("vnew.bin", NULL);
  const int32_t* cu = (const int32_t*)to_device("cu.bin", NULL);
  const int32_t* start = (const int32_t*)to_device("start.bin", NULL);
  const int32_t* stepbt = (const int32_t*)to_device("stepbt.bin", NULL);

  /* decode operands */
  size_t q_bytes;
  const void* q = to_device("q.bin", &q_bytes);
  const int32_t* bt = (const int32_t*)to_device("bt.bin", NULL);
  const int32_t* lens = (const int32_t*)to_device("lens.bin", NULL);
  void* out = NULL;
  float* lse = NULL;
  hip_check(hipMalloc(&out, q_bytes), "hipMalloc out");
  hip_check(hipMalloc((void**)&lse, (size_t)seqs * hq * sizeof(float)), "hipMalloc lse");
  const size_t ws_bytes = pkv_decode_workspace_bytes(&cache, seqs, hq, max_len, 0);
  void* ws = NULL;
  if (ws_bytes > 0) hip_check(hipMalloc(&ws, ws_bytes), "hipMalloc workspace");

  const int mixed = exists("pfmeta.txt");
  const int fused = exists("fused.txt");
  void* pfout = NULL;
  float* pflse = NULL;
  size_t pfq_bytes = 0;
  int num_reqs = 0, pf_tokens = 0;
  if (fused) {
    pkv_check(pkv_decode_step(&cache, knew, vnew, in_dtype, q, PKV_BF16, out, PKV_BF16, lse, bt,
                              bt_stride, lens, seqs, hq, max_len, sm_scale, 0, ws, ws_bytes, NULL),
              "pkv_decode_step");
    printf("decode_client: fused decode step\n");
  } else if (!mixed) {
    pkv_check(pkv_kv_cache_append(&cache, knew, vnew, in_dtype, cu, start, stepbt, step_stride,
                                  step_rows, step_tokens, NULL),
              "pkv_kv_cache_append");
    pkv_check(pkv_paged_attn_decode(&cache, q, PKV_BF16, out, PKV_BF16, lse, bt, bt_stride, lens,
                                    seqs, hq, max_len, sm_scale, 0, ws, ws_bytes, NULL),
              "pkv_paged_attn_decode");
  } else {
    char* pm = (char*)read_file("pfmeta.txt", &n);
    pm = (char*)realloc(pm, n + 1);
    pm[n] = 0;
    int max_chunk, max_total, pf_stride;
    if (sscanf(pm, "%d %d %d %d %d", &num_reqs, &pf_tokens, &max_chunk, &max_total, &pf_stride) != 5)
      die("pfmeta.txt", "5 fields expected");
    free(pm);
    const void* pfq = to_device("pfq.bin", &pfq_bytes);
    const int32_t* pfcu = (const int32_t*)to_device("pfcu.bin", NULL);
    const int32_t* pfctx = (const int32_t*)to_device("pfctx.bin", NULL);
    const int32_t* pfbt = (const int32_t*)to_device("pfbt.bin", NULL);
    hip_check(hipMalloc(&pfout, pfq_bytes), "hipMalloc pfout");
    hip_check(hipMalloc((void**)&pflse, (size_t)pf_tokens * hq * sizeof(float)), "hipMalloc pflse");
    const size_t pws_bytes =
        pkv_prefill_workspace_bytes(&cache, num_reqs, pf_tokens, hq, max_chunk, max_total, 0);
    void* pws = NULL;
    if (pws_bytes > 0) hip_check(hipMalloc(&pws, pws_bytes), "hipMalloc prefill workspace");

    pkv_append_batch ab;
    memset(&ab, 0, sizeof ab);
    ab.k_new = knew;
    ab.v_new = vnew;
    ab.in_dtype = in_dtype;
    ab.cu_new_tokens = cu;
    ab.start_pos = start;
    ab.block_tables = stepbt;
    ab.bt_stride = step_stride;
    ab.num_rows = step_rows;
    ab.num_new_tokens = step_tokens;
    pkv_decode_batch db;
    memset(&db, 0, sizeof db);
    db.q = q;
    db.q_dtype = PKV_BF16;
    db.out = out;
    db.out_dtype = PKV_BF16;
    db.lse = lse;
    db.block_tables = bt;
    db.bt_stride = bt_stride;
    db.context_lens = lens;
    db.num_seqs = seqs;
    db.num_q_heads = hq;
    db.max_context_len = max_len;
    db.split_tokens = 0;
    db.workspace = ws;
    db.workspace_bytes = ws_bytes;
    pkv_prefill_batch pb;
    memset(&pb, 0, sizeof pb);
    pb.q = pfq;
    pb.q_dtype = PKV_BF16;
    pb.out = pfout;
    pb.out_dtype = PKV_BF16;
    pb.lse = pflse;
    pb.cu_q_lens = pfcu;
    pb.ctx_before = pfctx;
    pb.block_tables = pfbt;
    pb.bt_stride = pf_stride;
    pb.num_reqs = num_reqs;
    pb.num_q_tokens = pf_tokens;
    pb.num_q_heads = hq;
    pb.max_chunk_len = max_chunk;
    pb.max_total_len = max_total;
    pb.split_tokens = 0;
    pb.workspace = pws;
    pb.workspace_bytes = pws_bytes;
    hipStream_t main_stream, side;
    hip_check(hipStreamCreate(&main_stream), "hipStreamCreate");
    hip_check(hipStreamCreate(&side), "hipStreamCreate");
    pkv_check(pkv_mixed_step(&cache, &ab, &db, &pb, sm_scale, main_stream, side),
              "pkv_mixed_step");
    hip_check(hipStreamSynchronize(main_stream), "hipStreamSynchronize");
    printf("decode_client: mixed step, %d prefill requests, %d chunk rows, prefill workspace %zu bytes\n",
           num_reqs, pf_tokens, pws_bytes);
  }
  hip_check(hipDeviceSynchronize(), "hipDeviceSynchronize");

  from_device("kpool_out.bin", cache.k_pool, pool_bytes);
  from_device("vpool_out.bin", cache.v_pool, pool_bytes);
  from_device("out.bin", out, q_bytes);
  from_device("lse.bin", lse, (size_t)seqs * hq * sizeof(float));
  if (mixed) {
    from_device("pfout.bin", pfout, pfq_bytes);
    from_device("pflse.bin", pflse, (size_t)pf_tokens * hq * sizeof(float));
  }
  printf("decode_client: workspace %zu bytes, done\n", ws_bytes);
  return 0;
}
