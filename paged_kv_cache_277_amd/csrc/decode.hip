// Paged decode attention: split-K partial pass (vector path), the decode
// work list and the launch dispatch (the range merge is in merge.hip).
//
// Method: the query attends every cached token of its sequence; the kernel
// reaches each token's K/V through the block table (page = bt[t / P], slot
// t % P) — "TensorRT-LLM框架解析与高性能推理优化实践" §6.2 — and keeps a running
// max and running sum so that one pass over the keys gives the softmax
// (§6.1).  The score is sm_scale * <q, k> (scaled dot-product attention,
// "TensorRT-LLM性能调优：提升LLM推理效率", fused-MHA row of the layer-fusion table).
//
// Work decomposition (MI355X): one workgroup of 4 waves per
// (row, KV head, context range of split_tokens tokens).  The G query heads
// that share a KV head are processed together, so each K/V byte is read
// once per group.  Within a wave, R = head_dim*bytes/16 consecutive lanes
// read one token row with 16-byte loads (a wave reads 64/R whole rows per
// instruction, contiguous inside the page), each lane dots its 16-byte piece
// with the matching query slice and the R-lane group sums the pieces.
// Every row-group of a wave runs its own online softmax; the states merge
// across lanes and waves at the end.  Ranges are aligned to 16 tokens and
// page sizes are multiples of 16, so every 16-token tile sits in one page
// and costs one block-table read.
//
// Output of a work item: if the row needs one range, the final output and
// log-sum-exp; otherwise (m, l, acc) into the workspace for the merge.
// m is kept in the log2 domain (scores are pre-multiplied by log2(e)).
//
// Both decode kernels (this one and decode_mfma.hip) also come in a fused
// step form (STEP = true, pkv_decode_step): the range that ends at a
// sequence's new token first stores that token's K/V row (kv_write.h), one
// 16-byte piece from each lane that later loads it.
#include <math.h>

#include <algorithm>

#include <type_traits>

#include "decode_list.h"
#include "kv_write.h"
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;

template <int KVT, int D>
struct VecShape {
  static constexpr int KVB = KvBytes<KVT>::value;
  static constexpr int EPL = 16 / KVB;                 // elements per lane load
  static constexpr int R = D / EPL;                    // lanes per token row
  static constexpr int RW = 64 / R;                    // rows per wave load
  static constexpr int U = (16 / RW) < 4 ? (16 / RW) : 4;  // loads per lane per tile
  static constexpr int TOK = U * RW;                   // tokens per wave tile
  static_assert(R >= 1 && R <= 64 && U >= 1, "shape");
};

// Convert one 16-byte piece to floats.
template <int KVT>
__device__ __forceinline__ void piece_to_f32(const u32x4& x, float* o) {
  if constexpr (KVT == KV_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(x[i]);
  } else if constexpr (KVT == KV_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { o[2 * i] = bf16_lo(x[i]); o[2 * i + 1] = bf16_hi(x[i]); }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) code4_to_f32<KVT>(x[i], o + 4 * i);
  }
}

template <typename T> __device__ __forceinline__ float load_q(const void* q, size_t i);
template <> __device__ __forceinline__ float load_q<float>(const void* q, size_t i) {
  return static_cast<const float*>(q)[i];
}
template <> __device__ __forceinline__ float load_q<uint16_t>(const void* q, size_t i) {
  return bf16_to_f32(static_cast<const uint16_t*>(q)[i]);
}

template <typename T> __device__ __forceinline__ void store_o(void* o, size_t i, float v);
template <> __device__ __forceinline__ void store_o<float>(void* o, size_t i, float v) {
  static_cast<float*>(o)[i] = v;
}
template <> __device__ __forceinline__ void store_o<uint16_t>(void* o, size_t i, float v) {
  static_cast<uint16_t*>(o)[i] = f32_to_bf16_rne(v);
}

// Resolve which query row, context length and block-table row a launch row
// (blockIdx.y) stands for.  Returns false if the row is empty padding.
__device__ __forceinline__ bool resolve_row(const AttnArgs& a, int z, int& L, int& btr,
                                            size_t& qrow) {
  if (a.prefill) {
    const int r = z / a.max_chunk, i = z - r * a.max_chunk;
    const int c0 = a.cu_q[r], c1 = a.cu_q[r + 1];
    if (i >= c1 - c0) return false;
    L = a.ctx_before[r] + i + 1;
    btr = r;
    qrow = (size_t)c0 + i;
  } else {
    L = a.context_lens[z];
    btr = z;
    qrow = (size_t)z;
  }
  return true;
}

// Load EPL query elements of one head at `idx` (16-byte loads), scaled.
template <typename QT, int EPL>
__device__ __forceinline__ void load_q_slice(const void* q, size_t idx, float mul, float* out) {
  if constexpr (sizeof(QT) == 4) {
    static_assert(EPL % 4 == 0, "");
#pragma unroll
    for (int c = 0; c < EPL / 4; ++c) {
      const u32x4 x = ld16(static_cast<const float*>(q) + idx + 4 * c);
#pragma unroll
      for (int i = 0; i < 4; ++i) out[4 * c + i] = __uint_as_float(x[i]) * mul;
    }
  } else {
    static_assert(EPL % 8 == 0, "");
#pragma unroll
    for (int c = 0; c < EPL / 8; ++c) {
      const u32x4 x = ld16(static_cast<const uint16_t*>(q) + idx + 8 * c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        out[8 * c + 2 * i] = bf16_lo(x[i]) * mul;
        out[8 * c + 2 * i + 1] = bf16_hi(x[i]) * mul;
      }
    }
  }
}

template <int KVT, int D, int GMAX, bool STEP>
__global__ __launch_bounds__(256) void decode_partial_vec(AttnArgs a) {
  using S = VecShape<KVT, D>;
  using QT = typename std::conditional<KVT == KV_F32, float, uint16_t>::type;
  constexpr int EPL = S::EPL, R = S::R, RW = S::RW, U = S::U, TOK = S::TOK;
  constexpr int ROWB = D * S::KVB;                 // bytes of one token row of one head

  // KV heads are the fastest grid dimension: workgroups dispatched together
  // read the head slabs of the same physical pages, which sit side by side.
  // The slowest dimension counts ranges back from each row's last: the last
  // (partial, on average half-size) range of every row is dispatched last,
  // so the launch ends on short work items instead of full ones.
  // With a work list (decode only) blockIdx.y + gridDim.y * blockIdx.z
  // indexes it instead (longest ranges first); workgroups past its end have
  // nothing to do.
  const int j = blockIdx.x;
  int z = blockIdx.y, item_range = 0;
  if (a.plan) {
    const int idx = blockIdx.y + gridDim.y * blockIdx.z;
    if (idx >= a.plan[0]) return;
    z = a.plan[2 + 2 * idx];
    item_range = a.plan[3 + 2 * idx];
    // (entries of a list written for another call, or overwritten, are
    // skipped: nothing outside this call's rows and ranges is accessed)
    if (z < 0 || z >= a.num_rows || item_range < 0 || item_range >= a.max_splits) return;
  }
  int L, btr;
  size_t qrow;
  if (!resolve_row(a, z, L, btr, qrow)) return;
  const int Hq = a.num_q_heads, Hkv = a.c.num_kv_heads;
  const int pshift = a.page_shift, pmask = (1 << pshift) - 1;
  const int G = Hq / Hkv;
  if (L <= 0) {
    if (a.plan || blockIdx.z == a.max_splits - 1) {  // empty context: output 0, lse = -inf
      for (int i = threadIdx.x; i < G * D; i += blockDim.x)
        store_o<QT>(a.out, (qrow * Hq + (size_t)j * G) * D + i, 0.0f);
      if (a.lse && threadIdx.x < G) a.lse[qrow * Hq + (size_t)j * G + threadIdx.x] = -INFINITY;
    }
    return;
  }
  // (a length beyond max_splits ranges breaks the call's precondition: the
  // clamp keeps every write inside the workspace)
  const int n_split = min((L + a.split_tokens - 1) / a.split_tokens, a.max_splits);
  const int split = a.plan ? item_range : n_split - a.max_splits + (int)blockIdx.z;
  if (split < 0) return;
  const int t_begin = split * a.split_tokens;
  const int t_end = min(L, t_begin + a.split_tokens);

  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int rg = lane / R, col = lane % R;
  // Fused decode step: the range that ends at the new token (position
  // L - 1) stores it.  Its tile (TOK tokens) belongs to wave
  // (o / TOK) % kWaves, which loads row o % TOK of the tile with the lanes
  // of row group (o % TOK) % RW, lane col taking piece col; those lanes
  // store exactly the pieces they load later.
  [[maybe_unused]] bool step_lane = false;
  [[maybe_unused]] StepPiece<KVT> step_piece;
  if constexpr (STEP) {
    const int o = L - 1 - t_begin;
    step_lane = t_end == L && w == (o / TOK) % kWaves && rg == (o % TOK) % RW;
    if (step_lane) step_piece.load(a, z, j, L - 1, col);
  }

  float kscale = 1.0f, vscale = 1.0f;
  if constexpr (KvCoded<KVT>::value) { kscale = a.c.k_scale[j]; vscale = a.c.v_scale[j]; }
  const float qmul = a.sm_scale * kLog2e * kscale;

  float qf[GMAX][EPL];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    if (g < G) {
      load_q_slice<QT, EPL>(a.q, (qrow * Hq + (size_t)j * G + g) * D + col * EPL, qmul, qf[g]);
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[g][e] = 0.0f;
    }
  }

  float m[GMAX], l[GMAX], acc[GMAX][EPL];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.0f;
  }

  const int32_t* btrow = a.bt + (size_t)btr * a.bt_stride;
  const uint8_t* kp = static_cast<const uint8_t*>(a.c.k_pool);
  const uint8_t* vp = static_cast<const uint8_t*>(a.c.v_pool);
  // Byte offset of this lane's piece inside a 16-token tile of page `page`.
  const size_t lane_off = (size_t)rg * ROWB + (size_t)col * 16;
  auto tile_base = [&](int page, int t) -> size_t {
    return (((size_t)page * Hkv + j) << pshift | (size_t)(t & pmask)) * ROWB + lane_off;
  };
  constexpr int STRIDE = kWaves * TOK;

  // Software pipeline.  This wave's tiles start at tw0 + k*STRIDE, k < nt.
  // Two register images alternate: while one tile is scored the next one's
  // K/V loads are in flight.  Page ids are read from the block table two
  // tiles ahead, each before the K/V loads of the tile after the current one,
  // so that every wait (vector loads retire in order) covers only what the
  // next step needs.  The main loop runs only while two more tiles exist, so
  // its loads are unconditional (page lookups past the range are clamped to
  // its last token) and no wait has to cover a branch; the last tiles are
  // peeled.
  const int tw0 = t_begin + w * TOK;
  const int nt = tw0 < t_end ? (t_end - tw0 + STRIDE - 1) / STRIDE : 0;
  auto page_of = [&](int k) { return btrow[min(tw0 + k * STRIDE, t_end - 1) >> pshift]; };
  auto load = [&](u32x4 (&kd)[U], u32x4 (&vd)[U], int page, int t) {
    const size_t base = tile_base(page, t);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      kd[u] = ld16_stream(kp + base + (size_t)u * RW * ROWB);
      vd[u] = ld16_stream(vp + base + (size_t)u * RW * ROWB);
    }
  };
  auto compute = [&](const u32x4 (&kc)[U], const u32x4 (&vc_in)[U], const int t0) {
    const bool full = t0 + TOK <= t_end;
    u32x4 vc[U];
    float sc[GMAX][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool valid = full || (t0 + u * RW + rg < t_end);
      float kf[EPL];
      piece_to_f32<KVT>(kc[u], kf);
#pragma unroll
      for (int g = 0; g < GMAX; ++g) {
        float s = 0.0f;
        if (g < G) {
#pragma unroll
          for (int e = 0; e < EPL; ++e) s = fmaf(qf[g][e], kf[e], s);
        }
        s = group_sum<R>(s);
        sc[g][u] = valid ? s : -INFINITY;
      }
      vc[u] = valid ? vc_in[u] : u32x4{0, 0, 0, 0};   // rows past the end may hold NaN
    }
    float p[GMAX][U];
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      float mx = sc[g][0];
#pragma unroll
      for (int u = 1; u < U; ++u) mx = fmaxf(mx, sc[g][u]);
      const float mn = fmaxf(m[g], mx);
      // mn is finite for every lane with a valid row so far; lanes with none
      // keep m = -inf and p = 0 (exp2 of -inf is 0, and -inf - -inf is avoided).
      const float alpha = (mn == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m[g] - mn);
      l[g] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
      m[g] = mn;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        p[g][u] = (mn == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(sc[g][u] - mn);
        l[g] += p[g][u];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[EPL];
      piece_to_f32<KVT>(vc[u], vf);
#pragma unroll
      for (int g = 0; g < GMAX; ++g) {
        if (g < G) {
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(p[g][u], vf[e], acc[g][e]);
        }
      }
    }
  };

  // Prologue: a wave without tiles (nt == 0) loads the range's last tile
  // instead and never uses it (in bounds, and no branch around the loads).
  u32x4 kA[U], vA[U], kB[U], vB[U];
  const int ta = tw0 < t_end ? tw0 : ((t_end - 1) & ~(TOK - 1));
  const int pg0 = btrow[ta >> pshift];
  int pg_next = page_of(1);
  // The new token lies in the owner wave's last tile: with more than one
  // tile that one is loaded in the loop, so the store can follow this first
  // load (whose wait then does not cover it); with one tile it must precede it.
  if constexpr (STEP) {
    if (step_lane && nt == 1) step_piece.store(a);
  }
  load(kA, vA, pg0, ta);
  if constexpr (STEP) {
    if (step_lane && nt > 1) step_piece.store(a);
  }
  // step(k): page id of tile k+2, loads of tile k+1 into nxt, score tile k.
  auto step = [&](int k, const u32x4 (&kc)[U], const u32x4 (&vc)[U], u32x4 (&kn)[U],
                  u32x4 (&vn)[U]) {
    const int pg = pg_next;
    pg_next = page_of(k + 2);
    load(kn, vn, pg, tw0 + (k + 1) * STRIDE);
    compute(kc, vc, tw0 + k * STRIDE);
  };
  int k = 0;
  for (; k + 2 < nt; k += 2) {
    step(k, kA, vA, kB, vB);
    step(k + 1, kB, vB, kA, vA);
  }
  if (k + 1 < nt) {                              // two tiles left: A holds tile k
    step(k, kA, vA, kB, vB);
    compute(kB, vB, tw0 + (k + 1) * STRIDE);
  } else if (k < nt) {                           // one tile left
    compute(kA, vA, tw0 + k * STRIDE);
  }

  // Merge the row-groups of this wave (lanes that share `col`).
#pragma unroll
  for (int mask = R; mask < 64; mask <<= 1) {
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      if (g >= G) continue;
      const float mo = __shfl_xor(m[g], mask, 64);
      const float lo = __shfl_xor(l[g], mask, 64);
      const float mn = fmaxf(m[g], mo);
      const float fa = (m[g] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m[g] - mn);
      const float fb = (mo == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mo - mn);
      l[g] = l[g] * fa + lo * fb;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float ao = __shfl_xor(acc[g][e], mask, 64);
        acc[g][e] = acc[g][e] * fa + ao * fb;
      }
      m[g] = mn;
    }
  }

  // Merge the waves through LDS.
  __shared__ float sm_acc[kWaves][GMAX][D];
  __shared__ float sm_m[kWaves][GMAX], sm_l[kWaves][GMAX];
  if (rg == 0) {
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      if (g >= G) continue;
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_acc[w][g][col * EPL + e] = acc[g][e];
      if (col == 0) { sm_m[w][g] = m[g]; sm_l[w][g] = l[g]; }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
    const int g = i / D, d = i - g * D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm_m[ww][g]);
    float lt = 0.0f, at = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float mw = sm_m[ww][g];
      const float f = (mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
      lt = fmaf(sm_l[ww][g], f, lt);
      at = fmaf(sm_acc[ww][g][d], f, at);
    }
    const int h = j * G + g;
    if (n_split == 1) {
      store_o<QT>(a.out, (qrow * Hq + h) * D + d, at * vscale / lt);
      if (d == 0 && a.lse) a.lse[qrow * Hq + h] = (M + __log2f(lt)) * kLn2;
    } else {
      const size_t slot = ((size_t)z * Hq + h) * a.max_splits + split;
      a.ws_acc[slot * D + d] = at * vscale;
      if (d == 0) { a.ws_ml[slot * 2] = M; a.ws_ml[slot * 2 + 1] = lt; }
    }
  }
}

// The work list on its own (separate calls): one workgroup.
__global__ __launch_bounds__(256) void decode_list_kernel(DecodeListArgs a) {
  build_decode_list(a);
}

template <int KVT, int D, bool STEP>
hipError_t launch_vec_d(const AttnArgs& a, dim3 grid, hipStream_t s) {
  const int G = a.num_q_heads / a.c.num_kv_heads;
  const dim3 block(256);
  if (G <= 1) hipLaunchKernelGGL((decode_partial_vec<KVT, D, 1, STEP>), grid, block, 0, s, a);
  else if (G <= 2) hipLaunchKernelGGL((decode_partial_vec<KVT, D, 2, STEP>), grid, block, 0, s, a);
  else if (G <= 4) hipLaunchKernelGGL((decode_partial_vec<KVT, D, 4, STEP>), grid, block, 0, s, a);
  else if (G <= 8) hipLaunchKernelGGL((decode_partial_vec<KVT, D, 8, STEP>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((decode_partial_vec<KVT, D, 16, STEP>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int KVT>
hipError_t launch_vec(const AttnArgs& a, dim3 grid, hipStream_t s) {
  if (a.new_k)
    return a.c.head_dim == 64 ? launch_vec_d<KVT, 64, true>(a, grid, s)
                              : launch_vec_d<KVT, 128, true>(a, grid, s);
  return a.c.head_dim == 64 ? launch_vec_d<KVT, 64, false>(a, grid, s)
                            : launch_vec_d<KVT, 128, false>(a, grid, s);
}

hipError_t launch_vec_any(const AttnArgs& a, dim3 grid, hipStream_t s) {
  switch (a.c.kv_dtype) {
    case KV_F32: return launch_vec<KV_F32>(a, grid, s);
    case KV_BF16: return launch_vec<KV_BF16>(a, grid, s);
    case KV_FP8: return launch_vec<KV_FP8>(a, grid, s);
    default: return launch_vec<KV_INT8>(a, grid, s);
  }
}

}  // namespace

// A work list is worth building when the call has enough workgroups for
// their order to matter.
bool decode_plan_useful(const AttnArgs& a) {
  return !a.prefill && a.max_splits > 1 && a.num_rows > 0 &&
         (int64_t)a.num_rows * a.max_splits * a.c.num_kv_heads >= 1024;
}

hipError_t launch_decode_list(const DecodeListArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(decode_list_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

dim3 decode_plan_grid(const AttnArgs& a) {
  const int64_t n = (int64_t)a.num_rows * a.max_splits;
  const int y = (int)std::min<int64_t>(n, 65535);
  return dim3(a.c.num_kv_heads, y, (unsigned)((n + y - 1) / y));
}

hipError_t launch_decode_partial(const AttnArgs& a, hipStream_t s) {
  if (a.num_rows == 0) return hipSuccess;
  if (decode_mfma_supported(a)) return launch_decode_partial_mfma(a, s);
  const dim3 grid = a.plan ? decode_plan_grid(a) : dim3(a.c.num_kv_heads, a.num_rows, a.max_splits);
  return launch_vec_any(a, grid, s);
}

// Chunked prefill.  bf16 queries go to the matrix-core kernel; the generic
// path (fp32) treats every chunk row as a decode query over its causal prefix
// (keys 0 .. ctx_before + i), one context range per row.
hipError_t launch_prefill(const AttnArgs& a, hipStream_t s) {
  if (a.num_rows == 0 || a.max_chunk == 0) return hipSuccess;
  if (prefill_mfma_supported(a)) return launch_prefill_mfma(a, s);
  const dim3 grid(a.c.num_kv_heads, a.num_rows * a.max_chunk, 1);
  return launch_vec_any(a, grid, s);
}

}  // namespace pkv
