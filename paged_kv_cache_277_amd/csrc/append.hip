// kv_cache_append: scatter new tokens' K/V rows into their page slots.
//
// A new token joins its request's cache at the next logical position; the
// position maps to a physical page through the request's block table
// ("TensorRT-LLM框架解析与高性能推理优化实践" §4.2; in-flight batching places each
// request's KV as it grows, "TensorRT-LLM内核融合与动态批处理", In-flight Batching).
// An fp8 cache stores x / scale[head] rounded to e4m3fn, an int8 cache its
// symmetric int8 code (first page, §7.2: one scale per head).
//
// Launch: one workgroup per new token; its threads cover the token's
// Hkv x head_dim row in 16-byte output pieces, so every page row is written
// with full 16-byte stores and the packed input is read contiguously.  The
// workgroup size is a multiple of 64 (the row lookup is wave-wide).
#include "decode_list.h"
#include "kv_write.h"
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

// Request owning packed token t: the largest r < n with cu[r] <= t
// (cu[0] = 0, non-decreasing, n >= 1, t < cu[n]), which is the number of
// rows 1 .. n-1 that start at or before t.  The wave's lanes test 64 offsets
// per load and a ballot counts them, so the lookup costs one load latency per
// 64 rows instead of one per step of a binary search.  Every lane of the
// wave must be active; the result is wave-uniform.
__device__ __forceinline__ int owner_row(const int32_t* cu, int n, int t) {
  const int lane = threadIdx.x & 63;
  int r = 0;
  for (int base = 1; base < n; base += 64) {
    const int i = base + lane;
    r += __popcll(__ballot(i < n && cu[i] <= t));
  }
  return r;
}

template <int KVT>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  constexpr int EPL = 16 / KvBytes<KVT>::value;  // cache elements per 16-byte piece
  if (a.list.list && blockIdx.x == a.num_tokens) {   // the extra workgroup: decode work list
    build_decode_list(a.list);
    return;
  }
  const int t = blockIdx.x;
  const int D = a.c.head_dim, Hkv = a.c.num_kv_heads;
  const int pieces = D / EPL;                    // per head
  const int total = Hkv * pieces;
  // The input does not depend on where the token goes: the first piece's
  // loads are issued before the lookups of its row, position and page.
  const int c0 = threadIdx.x, j0 = c0 / pieces, pc0 = c0 % pieces;
  KvInput<KVT> in0;
  if (c0 < total)
    in0 = load_kv_input<KVT>(a.c, a.k_new, a.v_new, ((size_t)t * Hkv + j0) * D + (size_t)pc0 * EPL,
                             j0);
  const int r = owner_row(a.cu, a.num_rows, t);
  const int pos = a.start_pos[r] + (t - a.cu[r]);
  const int P = a.c.page_size;
  const int page = a.bt[(size_t)r * a.bt_stride + pos / P];
  const int slot = pos % P;
  if (c0 < total) store_kv_input<KVT>(a.c, in0, kv_piece_offset<KVT>(a.c, page, j0, slot, pc0));
  for (int c = c0 + blockDim.x; c < total; c += blockDim.x) {
    const int j = c / pieces, pc = c % pieces;
    const size_t src_e = ((size_t)t * Hkv + j) * D + (size_t)pc * EPL;   // input element
    write_kv_piece<KVT>(a.c, a.k_new, a.v_new, src_e, kv_piece_offset<KVT>(a.c, page, j, slot, pc), j);
  }
}

// Decodes through the fp8 -> bf16 conversion of the matrix-core attention
// path (the bf16 result widens to float exactly).
__global__ __launch_bounds__(256) void fp8_to_f32_kernel(const uint8_t* codes, float* out, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  uint32_t w = 0;
  if (i + 4 <= n) {
    w = *reinterpret_cast<const uint32_t*>(codes + i);
  } else {
    for (int64_t k = i; k < n; ++k) w |= uint32_t(codes[k]) << (8 * (k - i));
  }
  const uint32_t lo = fp8x2_to_bf16x2<false>(w), hi = fp8x2_to_bf16x2<true>(w);
  const float o[4] = {bf16_lo(lo), bf16_hi(lo), bf16_lo(hi), bf16_hi(hi)};
  for (int k = 0; k < 4 && i + k < n; ++k) out[i + k] = o[k];
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  if (a.num_tokens == 0 && !a.list.list) return hipSuccess;
  const dim3 grid(a.num_tokens + (a.list.list ? 1 : 0));
  const dim3 block(a.c.num_kv_heads * a.c.head_dim >= 2048 ? 256 : 128);
  switch (a.c.kv_dtype) {
    case KV_F32: hipLaunchKernelGGL(append_kernel<KV_F32>, grid, block, 0, s, a); break;
    case KV_BF16: hipLaunchKernelGGL(append_kernel<KV_BF16>, grid, block, 0, s, a); break;
    case KV_FP8: hipLaunchKernelGGL(append_kernel<KV_FP8>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(append_kernel<KV_INT8>, grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_fp8_to_f32(const uint8_t* codes, float* out, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t groups = (n + 3) / 4;
  const dim3 grid((unsigned)((groups + 255) / 256)), block(256);
  hipLaunchKernelGGL(fp8_to_f32_kernel, grid, block, 0, s, codes, out, n);
  return hipGetLastError();
}

}  // namespace pkv
