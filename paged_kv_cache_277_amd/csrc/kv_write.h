// Writing new tokens' K/V rows into the paged pools.
//
// A token at logical position t of a request lands in page bt[t / P], slot
// t % P of that page ("TensorRT-LLM框架解析与高性能推理优化实践" §4.2 and §6.2: the
// block table maps logical blocks to physical pages).  F32 and BF16 caches
// store the input bits; an fp8 cache stores e4m3fn(x / scale[head]) and an
// int8 cache the symmetric int8 code of x / scale[head] (first page, §7.2:
// one scale per head).  The standalone append and the fused decode step both
// write through these helpers, so the two store the same bytes.
#pragma once

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

// Byte offset, in either pool, of 16-byte piece `pc` of KV head j's row at
// slot `slot` of page `page` (pool layout [page][Hkv][P][D]).
template <int KVT>
__device__ __forceinline__ size_t kv_piece_offset(const CacheView& c, int page, int j, int slot,
                                                  int pc) {
  constexpr int KVB = KvBytes<KVT>::value;
  constexpr int EPL = 16 / KVB;
  return ((((size_t)page * c.num_kv_heads + j) * c.page_size + slot) * c.head_dim +
          (size_t)pc * EPL) * KVB;
}

// Input of one 16-byte cache piece of a token's K row and V row of one KV
// head: 16 bytes each for F32/BF16 caches (a copy), 16 floats each plus the
// head's scales for 8-bit caches (encoded on the way out).
template <int KVT>
struct KvInput {
  static constexpr int N = KvCoded<KVT>::value ? 4 : 1;
  u32x4 k[N], v[N];
  float ks, vs;
};

// src_e: index of the piece's first element in the packed input rows (the
// cache's own dtype for F32/BF16, float32 for 8-bit caches).
template <int KVT>
__device__ __forceinline__ KvInput<KVT> load_kv_input(const CacheView& c, const void* k_new,
                                                      const void* v_new, size_t src_e, int j) {
  constexpr int KVB = KvBytes<KVT>::value;
  KvInput<KVT> in;
  if constexpr (KvCoded<KVT>::value) {
    const u32x4* ksrc = reinterpret_cast<const u32x4*>(static_cast<const float*>(k_new) + src_e);
    const u32x4* vsrc = reinterpret_cast<const u32x4*>(static_cast<const float*>(v_new) + src_e);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      in.k[q4] = ksrc[q4];
      in.v[q4] = vsrc[q4];
    }
    in.ks = c.k_scale[j];
    in.vs = c.v_scale[j];
  } else {
    in.k[0] = ld16(static_cast<const uint8_t*>(k_new) + src_e * KVB);
    in.v[0] = ld16(static_cast<const uint8_t*>(v_new) + src_e * KVB);
  }
  return in;
}

// Encode (8-bit caches: 16 floats -> 16 codes of x / scale) and store the
// piece at byte offset dst of both pools.
template <int KVT>
__device__ __forceinline__ void store_kv_input(const CacheView& c, const KvInput<KVT>& in,
                                               size_t dst) {
  uint8_t* kdst = static_cast<uint8_t*>(c.k_pool_w);
  uint8_t* vdst = static_cast<uint8_t*>(c.v_pool_w);
  if constexpr (KvCoded<KVT>::value) {
    u32x4 ko, vo;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      uint32_t kw = 0, vw = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kw |= f32_to_code<KVT>(__uint_as_float(in.k[q4][e]) / in.ks) << (8 * e);
        vw |= f32_to_code<KVT>(__uint_as_float(in.v[q4][e]) / in.vs) << (8 * e);
      }
      ko[q4] = kw;
      vo[q4] = vw;
    }
    *reinterpret_cast<u32x4*>(kdst + dst) = ko;
    *reinterpret_cast<u32x4*>(vdst + dst) = vo;
  } else {
    *reinterpret_cast<u32x4*>(kdst + dst) = in.k[0];
    *reinterpret_cast<u32x4*>(vdst + dst) = in.v[0];
  }
}

template <int KVT>
__device__ __forceinline__ void write_kv_piece(const CacheView& c, const void* k_new,
                                               const void* v_new, size_t src_e, size_t dst,
                                               int j) {
  store_kv_input<KVT>(c, load_kv_input<KVT>(c, k_new, v_new, src_e, j), dst);
}

// Fused decode step: piece `pc` of the new token's K and V rows of KV head
// j (position pos of sequence z; input row z of new_k / new_v,
// [num_seqs][Hkv][D]).  The attention kernels load it early and store it
// from the lane that later loads that same piece from the pool, right after
// that wave's first K/V load (or just before it, when the first tile is the
// one holding the token): the store precedes the load of the token's row in
// that thread's program order, so no barrier is needed, and the inputs have
// arrived by then.  Vector memory waits retire in order, so a store issued
// before a wait's target loads would hold that wait up until it completed.
template <int KVT>
struct StepPiece {
  KvInput<KVT> in;
  size_t dst;

  __device__ __forceinline__ void load(const AttnArgs& a, int z, int j, int pos, int pc) {
    constexpr int EPL = 16 / KvBytes<KVT>::value;
    const int page = a.bt[(size_t)z * a.bt_stride + (pos >> a.page_shift)];
    const int slot = pos & ((1 << a.page_shift) - 1);
    in = load_kv_input<KVT>(a.c, a.new_k, a.new_v,
                            ((size_t)z * a.c.num_kv_heads + j) * a.c.head_dim + (size_t)pc * EPL,
                            j);
    dst = kv_piece_offset<KVT>(a.c, page, j, slot, pc);
  }
  __device__ __forceinline__ void store(const AttnArgs& a) const { store_kv_input<KVT>(a.c, in, dst); }
};

}  // namespace pkv
