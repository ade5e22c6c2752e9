// Log-sum-exp merge of per-range partials (decode ranges and prefill key
// ranges).
//
// Method: a row whose keys were split into ranges s carries, per range, the
// running max m_s (log2 units), the running sum l_s and the unnormalised
// accumulator acc_s of the one-pass softmax ("TensorRT-LLM框架解析与高性能推理优化实践"
// §6.1, running max / running sum); the ranges combine as
//   M = max_s m_s,  w_s = exp2(m_s - M),
//   out = sum_s w_s acc_s / sum_s w_s l_s,
//   lse = (M + log2 sum_s w_s l_s) ln 2.
//
// Work decomposition (MI355X): every thread owns one 16-byte chunk (four
// floats) of one query head's output; a workgroup of 256 threads covers
// 256 / (D/4) heads of one row (8 at D = 128).  The grid is (row, head
// group) for decode and (chunk row, head group, request) for prefill, so a
// prefill workgroup reads its request's offsets directly; rows with one
// range were written by the attention kernel and exit at once.  A thread
// reads its head's (m, l) pairs (the same 8-byte words for the whole head,
// served from cache) and that head's accumulators, contiguous [ranges][D].
// Rows of up to four ranges issue all of those loads in one round; longer
// rows take the maximum first, then stream the accumulators four ranges at
// a time.  No LDS and no barrier.
#include <math.h>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

template <int D>
__device__ __forceinline__ void store4(float* o, size_t i, f32x4 v) {
  *reinterpret_cast<f32x4*>(o + i) = v;
}
template <int D>
__device__ __forceinline__ void store4(uint16_t* o, size_t i, f32x4 v) {
  *reinterpret_cast<u32x2*>(o + i) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

template <typename OT, int D>
__global__ __launch_bounds__(256) void lse_merge_kernel(AttnArgs a) {
  constexpr int C4 = D / 4;                      // 16-byte chunks per head
  constexpr int HPW = 256 / C4;                  // heads per workgroup
  const int h = blockIdx.y * HPW + threadIdx.x / C4;
  const int d = 4 * (threadIdx.x % C4);
  const int Hq = a.num_q_heads, ms = a.max_splits;
  if (h >= Hq) return;
  int z, L;
  if (a.prefill) {
    // Chunk row i of request r is packed row cu_q[r] + i, at absolute
    // position ctx_before[r] + i: it attends that many keys plus itself.
    const int r = blockIdx.z, i = blockIdx.x;
    const int c0 = a.cu_q[r], c1 = a.cu_q[r + 1], pr = a.ctx_before ? a.ctx_before[r] : 0;
    if (i >= c1 - c0) return;
    z = c0 + i;
    L = pr + i + 1;
  } else {
    z = blockIdx.x;
    L = a.context_lens[z];
  }
  const int n = min((L + a.split_tokens - 1) / a.split_tokens, ms);
  if (n <= 1) return;
  const size_t slot0 = ((size_t)z * Hq + h) * ms;
  const f32x2* ml = reinterpret_cast<const f32x2*>(a.ws_ml) + slot0;
  const float* acc = a.ws_acc + slot0 * D + d;
  f32x4 o = {0.0f, 0.0f, 0.0f, 0.0f};
  float den = 0.0f;
  float M = -INFINITY;
  // Four ranges per batch of independent loads; indices past the last range
  // repeat it and get weight 0.
  auto batch = [&](int s0) {
    f32x4 v[4];
    f32x2 mlv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ss = min(s0 + u, n - 1);
      v[u] = *reinterpret_cast<const f32x4*>(acc + (size_t)ss * D);
      mlv[u] = ml[ss];
    }
    if (s0 == 0 && n <= 4) {                     // the whole row in this batch
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (u < n) M = fmaxf(M, mlv[u][0]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float wgt = s0 + u < n ? __builtin_amdgcn_exp2f(mlv[u][0] - M) : 0.0f;
      den = fmaf(mlv[u][1], wgt, den);
      o += v[u] * wgt;
    }
  };
  if (n <= 4) {
    batch(0);
  } else {
    for (int s = 0; s < n; ++s) M = fmaxf(M, ml[s][0]);
    for (int s0 = 0; s0 < n; s0 += 4) batch(s0);
  }
  store4<D>(static_cast<OT*>(a.out), ((size_t)z * Hq + h) * D + d, o * (1.0f / den));
  if (d == 0 && a.lse) a.lse[(size_t)z * Hq + h] = (M + __log2f(den)) * kLn2;
}

}  // namespace

hipError_t launch_lse_merge(const AttnArgs& a, hipStream_t s) {
  const int rows = a.prefill ? a.num_tokens : a.num_rows;
  if (a.num_rows == 0 || rows == 0 || a.max_splits <= 1) return hipSuccess;
  const bool f32 = a.c.kv_dtype == KV_F32;
  const int hpw = 256 / (a.c.head_dim / 4);
  const int groups = (a.num_q_heads + hpw - 1) / hpw;
  const dim3 grid = a.prefill ? dim3(a.max_chunk, groups, a.num_rows) : dim3(rows, groups);
  const dim3 block(256);
  if (a.c.head_dim == 64) {
    if (f32) hipLaunchKernelGGL((lse_merge_kernel<float, 64>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((lse_merge_kernel<uint16_t, 64>), grid, block, 0, s, a);
  } else {
    if (f32) hipLaunchKernelGGL((lse_merge_kernel<float, 128>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((lse_merge_kernel<uint16_t, 128>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace pkv
