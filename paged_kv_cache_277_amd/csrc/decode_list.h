// Decode work list: every (row, context range) item of a decode call, ordered
// longest first, so that the decode launch ends on its shortest items rather
// than on whichever ranges its grid order would put last.
//
// A counting sort of the items' token counts into kListClasses classes, full
// ranges in the first.  An empty row has one item, which writes its zero
// output.  Order within a class follows the atomic cursors; the decode's
// results do not depend on it, each item writing its own outputs.  Runs on
// one workgroup of at least 64 threads (every thread must call it).
#pragma once

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

constexpr int kListClasses = 64;                // <= 64: one wave scans them

__device__ __forceinline__ void build_decode_list(const DecodeListArgs& a) {
  __shared__ int cursor[kListClasses];
  if (threadIdx.x < kListClasses) cursor[threadIdx.x] = 0;
  const int S = a.split_tokens, ms = a.max_splits;
  // items of a row of L tokens: n ranges, the last one in class c
  auto items = [&](int L, int& n, int& c) {
    int last = 0;
    if (L <= 0) {
      n = 1;
    } else {
      n = min((L + S - 1) / S, ms);
      last = min(L, n * S) - (n - 1) * S;
    }
    c = (int)((int64_t)(S - last) * (kListClasses - 1) / S);
  };
  __syncthreads();
  for (int r = threadIdx.x; r < a.num_rows; r += blockDim.x) {
    int n, c;
    items(a.context_lens[r], n, c);
    if (n > 1) atomicAdd(&cursor[0], n - 1);
    atomicAdd(&cursor[c], 1);
  }
  __syncthreads();
  if (threadIdx.x < 64) {                        // exclusive scan of the class sizes
    const int v = threadIdx.x < kListClasses ? cursor[threadIdx.x] : 0;
    int incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(incl, d, 64);
      if ((int)threadIdx.x >= d) incl += t;
    }
    if (threadIdx.x < kListClasses) cursor[threadIdx.x] = incl - v;
    if (threadIdx.x == 63) {
      a.list[0] = incl;
      a.list[1] = 0;
    }
  }
  __syncthreads();
  int* out = a.list + 2;
  for (int r = threadIdx.x; r < a.num_rows; r += blockDim.x) {
    int n, c;
    items(a.context_lens[r], n, c);
    if (n > 1) {
      const int p = atomicAdd(&cursor[0], n - 1);
      for (int k = 0; k < n - 1; ++k) {
        out[2 * (p + k)] = r;
        out[2 * (p + k) + 1] = k;
      }
    }
    const int p = atomicAdd(&cursor[c], 1);
    out[2 * p] = r;
    out[2 * p + 1] = n - 1;
  }
}

}  // namespace pkv
