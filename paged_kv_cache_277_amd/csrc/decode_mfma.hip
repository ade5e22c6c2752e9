// Paged decode attention for grouped query heads on the matrix cores (MFMA).
//
// Same method as the vector path (block-table walk, running max / running
// sum: "TensorRT-LLM框架解析与高性能推理优化实践" §6.1-§6.2; scaled dot-product
// attention; per-head fp8 KV scales dequantised in the kernel, §7.2), for
// query groups G = Hq/Hkv >= 3, where the G heads that share a KV head turn
// decode into a small dense contraction per 32-token tile:
//
//   S^T[t][h] = sum_d K[t][d] Q[h][d]        v_mfma_f32_16x16x32_bf16, M = 16 tokens,
//                                            N = 16 head slots (G used), K = 32 of d
//   O^T[d][h] += sum_t V[t][d] P^T[t][h]     M = 16 of d, N = 16 head slots, K = 32 tokens
//
// Lane layouts of the 16x16x32 bf16 MFMA (wave64): A[i][k] in lane i%16 +
// 16*(k/8), element k%8; B[k][j] in lane j + 16*(k/8); C[i][j] in lane
// j + 16*(i/4), element i%4.  Consequences used below:
//   * K and V rows are loaded whole (each load instruction reads contiguous
//     row bytes, with the streaming hint) and K is written, in its storage
//     format, to the wave's padded LDS slice.  The A operand of step kk is
//     read back per lane: token l%16, 16-byte piece 4*(kk/SPP) + g (g = l/16,
//     SPP = MFMA steps per piece).  For bf16, step kk uses d = 32kk + 8g + e;
//     for 8-bit codes (16 per piece, widened in registers) d = 64(kk/2) + 16g
//     + 8(kk%2) + e.  Q^T (B operand) is loaded in the same d order.
//   * The S^T result leaves, in lane l, head h = l%16 for tokens 4g+r of each
//     16-token block; over the two blocks of a tile that is 8 tokens of one
//     head — exactly a B operand row of P^T if the tile's tokens are taken in
//     the order (4g..4g+3, 16+4g..16+4g+3).  No lane shuffle is needed.
//   * O^T accumulates in lane l for head h = l%16, so the online-softmax
//     rescale of a head touches only that lane's registers.
//   * V^T (A operand of the second product) needs 8 tokens of one d per lane:
//     the tile's V rows are written row-major to this wave's LDS slice with
//     16-byte stores and read back with gfx950's transpose read
//     (ds_read_b64_tr_b16: inside each 16-lane group, lane i receives element
//     i%4 of the 4-element reads of lanes 4r + i/4, r = 0..3).  Two such reads
//     give one A operand.
//
// Work decomposition: like the vector path, one workgroup of 4 waves per
// (row, KV head, context range); each wave walks 32-token tiles of the range
// with its own softmax state, the next tile's K/V loads in flight while the
// current tile is computed.  Scores are kept in the log2 domain.  The
// fused step form (STEP = true) is described in decode.hip.
#include <math.h>

#include <type_traits>

#include "kv_write.h"
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;
constexpr int kTile = 32;                      // tokens per wave tile
constexpr int kMaxRangePages = 512;            // block-table entries staged per work item
// A head's running max moves only when a score exceeds it by more than this
// (log2 units); the final (m, l, acc) describes the same softmax whichever
// shift was used.
constexpr float kSlack = 8.0f;

typedef __bf16 bf16x8_t __attribute__((__vector_size__(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}



// Per-lane register image of one 32-token tile, K and V alike: lane l holds
// the 16-byte pieces l%R of rows (l/R) + (64/R)*i of each 16-token block, so
// every load instruction reads whole rows (64*16 contiguous bytes per block
// row group) and can carry the streaming hint.
template <int KVT, int D>
struct TileRegs {
  static constexpr int KVB = KvBytes<KVT>::value;
  static constexpr int VROWB = D * KVB;                // bytes per K/V row in the pool
  static constexpr int VLOADS = (kTile * VROWB) / (64 * 16);  // 16-byte loads per lane, each of K and V
  u32x4 k[VLOADS];
  u32x4 v[VLOADS];
};

// Page ids of the two 16-token blocks of the tile at t0 < t_end.  A block
// past the end looks up the page of token t_end - 1, which is block 0's page
// (16-token blocks never straddle a page): in bounds, and masked later.
// `pages` holds the block-table entries of this work item's range, from
// entry `first`.
__device__ __forceinline__ void tile_pages(const int32_t* pages,
                                           int first, int t0, int t_end,
                                           int pshift, int& p0, int& p1) {
  p0 = pages[(t0 >> pshift) - first];
  p1 = pages[(min(t0 + 16, t_end - 1) >> pshift) - first];
}

// First of the 8 consecutive d values that MFMA step kk takes for lane group g:
// K load i of a lane holds 16-byte piece 4i + g of its token row, i.e. 8 bf16
// (step kk = i) or 16 8-bit codes (steps 2i and 2i + 1).
template <int KVT>
__device__ __forceinline__ int k_elem_offset(int kk, int g) {
  if constexpr (KvCoded<KVT>::value) return 64 * (kk >> 1) + 16 * g + 8 * (kk & 1);
  else return 32 * kk + 8 * g;
}

// Loads of one tile.  The row of a block is the same for the whole wave (page
// ids are wave-uniform), so the block's base addresses stay in scalar
// registers and every lane adds only its fixed offset `loff` = byte offset of
// its first piece in the block (row l/R, piece l%R); the load i of a block is
// a further i*RPI rows.
template <int KVT, int D>
__device__ __forceinline__ void load_tile(TileRegs<KVT, D>& r, const uint8_t* kp, const uint8_t* vp,
                                          int p0, int p1, int t0, int t_end, int Hkv, int j,
                                          int pshift, uint32_t loff) {
  using TR = TileRegs<KVT, D>;
  constexpr int ROWB = TR::VROWB;
  constexpr int R = ROWB / 16, RPI = 64 / R, LPB = TR::VLOADS / 2;
  const int pmask = (1 << pshift) - 1;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const int tb = (blk == 1 && t0 + 16 >= t_end) ? t0 : t0 + 16 * blk;
    const int page = blk == 0 ? p0 : p1;
    const size_t row = (((size_t)page * Hkv + j) << pshift | (size_t)(tb & pmask));
    const uint8_t* kb = kp + row * ROWB;
    const uint8_t* vb = vp + row * ROWB;
#pragma unroll
    for (int i = 0; i < LPB; ++i) {
      r.k[blk * LPB + i] = ld16_stream(kb + loff + i * RPI * ROWB);
      r.v[blk * LPB + i] = ld16_stream(vb + loff + i * RPI * ROWB);
    }
  }
}

template <int KVT, int D, bool STEP>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(KvBytes<KVT>::value == 1 || D == 64 ? 3 : 2)))
void decode_partial_mfma(AttnArgs a) {
  using TR = TileRegs<KVT, D>;
  constexpr int KK = D / 32;                    // MFMA steps over d
  constexpr int DT = D / 16;                    // 16-wide d tiles of the output
  constexpr int ROWB = TR::VROWB;
  constexpr int R = ROWB / 16, RPI = 64 / R, LPB = TR::VLOADS / 2;
  constexpr int LDS_ROW = D * 2 + 32;           // bf16 V rows in LDS, padded against bank conflicts
  constexpr int K_LDS_ROW = ROWB + 16;          // raw K rows in LDS (same slice, used before V)
  constexpr int STAGE_BYTES = kWaves * kTile * LDS_ROW;
  constexpr int OROW = D + 4;                   // padded rows of the merge image (floats)
  constexpr int MERGE_BYTES = (kWaves * 16 * OROW + kWaves * 32) * 4;
  __shared__ __attribute__((aligned(16)))
  uint8_t smem[STAGE_BYTES > MERGE_BYTES ? STAGE_BYTES : MERGE_BYTES];

  // Grid (KV head, row, range counted back from the row's last): the last,
  // partial range of every row is dispatched last (see decode.hip).
  // With a work list, blockIdx.y + gridDim.y * blockIdx.z indexes it instead
  // (longest ranges first); workgroups past its end have nothing to do.
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
  const int L = a.context_lens[z];
  const int Hq = a.num_q_heads, Hkv = a.c.num_kv_heads;
  const int G = Hq / Hkv;
  const size_t qrow = (size_t)z;
  if (L <= 0) {
    if (a.plan || blockIdx.z == a.max_splits - 1) {  // empty context: output 0, lse = -inf
      for (int i = threadIdx.x; i < G * D; i += blockDim.x)
        static_cast<uint16_t*>(a.out)[(qrow * Hq + (size_t)j * G) * D + i] = 0;
      if (a.lse && threadIdx.x < G) a.lse[qrow * Hq + (size_t)j * G + threadIdx.x] = -INFINITY;
    }
    return;
  }
  const int n_split = min((L + a.split_tokens - 1) / a.split_tokens, a.max_splits);
  const int split = a.plan ? item_range : n_split - a.max_splits + (int)blockIdx.z;
  if (split < 0) return;
  const int t_begin = split * a.split_tokens;
  const int t_end = min(L, t_begin + a.split_tokens);
  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int g4 = lane >> 4, h = lane & 15;       // lane group and head slot
  const int pshift = a.page_shift;

  float kscale = 1.0f, vscale = 1.0f;
  if constexpr (KvCoded<KVT>::value) { kscale = a.c.k_scale[j]; vscale = a.c.v_scale[j]; }
  const float smul = a.sm_scale * kLog2e * kscale;

  const int32_t* btrow = a.bt + (size_t)z * a.bt_stride;
  const uint8_t* kp = static_cast<const uint8_t*>(a.c.k_pool);
  const uint8_t* vp = static_cast<const uint8_t*>(a.c.v_pool);
  uint8_t* lds = smem + w * kTile * LDS_ROW;
  constexpr int STRIDE = kWaves * kTile;
  const uint32_t loff = (uint32_t)((lane / R) * ROWB + (lane % R) * 16);
  // Fused decode step: the range that ends at the new token (position
  // L - 1) stores it.  Its tile belongs to wave (o / kTile) % kWaves, which
  // loads row b = o % 16 of the token's 16-token block with the lanes
  // l / R = b % RPI, lane l taking piece l % R (load_tile); those lanes
  // store exactly the pieces they load later.
  [[maybe_unused]] bool step_lane = false;
  [[maybe_unused]] StepPiece<KVT> step_piece;
  if constexpr (STEP) {
    const int o = L - 1 - t_begin;
    step_lane = t_end == L && w == (o / kTile) % kWaves && lane / R == (o & 15) % RPI;
    if (step_lane) step_piece.load(a, z, j, L - 1, lane % R);
  }
  // This wave's tiles are t_begin + w*kTile + k*STRIDE, k = 0..nt-1.
  const int tw0 = t_begin + w * kTile;
  const int nt = tw0 < t_end ? (t_end - tw0 + STRIDE - 1) / STRIDE : 0;

  // Prologue, ordered so that its memory latencies overlap: the range's
  // block-table entries (for the LDS copy below; at most 2 per thread, the
  // host keeps ranges within kMaxRangePages pages), the page ids of this
  // wave's first two tiles straight from the table, then Q, then the first
  // tile's K/V loads, which wait only for their own two page ids.
  const int first = t_begin >> pshift;
  const int npg = ((t_end - 1) >> pshift) - first + 1;
  // (Indices are clamped rather than branched on, so that no wait has to
  // cover a branch: entries past the range repeat its last one, and the page
  // ids of tiles this wave does not have are those of the range's last token.)
  const int bte0 = btrow[first + min((int)threadIdx.x, npg - 1)];
  const int bte1 = btrow[first + min((int)threadIdx.x + 256, npg - 1)];
  // A wave without tiles (nt == 0) loads the range's last 16-aligned block
  // instead and never uses it.
  const int ta = tw0 < t_end ? tw0 : ((t_end - 1) & ~15);
  int pn0, pn1, pq0, pq1;                       // pages of tiles 0 and 1 of this wave
  tile_pages(btrow, 0, ta, t_end, pshift, pn0, pn1);
  tile_pages(btrow, 0, min(tw0 + STRIDE, t_end - 1), t_end, pshift, pq0, pq1);

  // Q^T as B operand: lane (g, h) holds Q[j*G + h][d] for the d's that MFMA
  // step kk takes from K (k_elem_offset); zero for h >= G.
  u32x4 qb[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) qb[kk] = u32x4{0, 0, 0, 0};
  if (h < G) {
    const uint16_t* q = static_cast<const uint16_t*>(a.q) + (qrow * Hq + (size_t)j * G + h) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qb[kk] = ld16(q + k_elem_offset<KVT>(kk, g4));
  }

  // Two register images alternate: while one tile is computed the next one's
  // loads are in flight, and the page ids of the tile after that are read
  // from LDS.  The main loop only runs while a next tile exists, so every
  // load in it is unconditional and the wait for the current tile's data
  // never has to cover the next tile's loads; the last tiles are peeled.
  // Only a range's last tile can hold tokens past its end, so every tile of
  // the main loop is computed without masks.
  TR buf0, buf1;
  // (Fused step: the new token lies in the owner wave's last tile, loaded
  // in the loop when the wave has more than one; see decode.hip.)
  if constexpr (STEP) {
    if (step_lane && nt == 1) step_piece.store(a);
  }
  load_tile<KVT, D>(buf0, kp, vp, pn0, pn1, ta, t_end, Hkv, j, pshift, loff);
  if constexpr (STEP) {
    if (step_lane && nt > 1) step_piece.store(a);
  }
  pn0 = pq0;                                    // pages of the next tile to load
  pn1 = pq1;

  // The range's block-table entries, staged in LDS once: later page lookups
  // then never wait behind the K/V loads in flight (vector-memory waits
  // retire in order).
  __shared__ int32_t pages[kMaxRangePages];
  pages[threadIdx.x] = bte0;
  pages[threadIdx.x + 256] = bte1;
  __syncthreads();
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) settle(qb[kk]);

  f32x4 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = f32x4{0, 0, 0, 0};
  // Running max m of head h (log2 domain; the same in the 4 lanes of h) and
  // this lane's share l of the head's running sum (its 8 tokens per tile).
  float m = -INFINITY, l = 0.0f;

  // compute(cur, t0, FULL): tile t0 from the register image cur; FULL tiles
  // have all 32 tokens inside the range.
  auto compute = [&](const TR& cur, const int t0, auto full_c) {
    constexpr bool FULL = decltype(full_c)::value;

    // ---- K rows -> LDS (raw storage format, padded rows) ----
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i = 0; i < LPB; ++i) {
        const int tok = 16 * blk + (lane / R) + RPI * i;
        *reinterpret_cast<u32x4*>(lds + tok * K_LDS_ROW + (lane % R) * 16) = cur.k[blk * LPB + i];
      }

    // ---- S^T = K Q^T for the two 16-token blocks ----
    // A operand of step kk, lane (g, n): token n, 16-byte piece 4*(kk / SPP) + g
    // (SPP = MFMA steps per piece: 1 for bf16, 2 for 8-bit codes).
    f32x4 s[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      f32x4 acc = {0, 0, 0, 0};
      const uint8_t* krow = lds + (16 * blk + h) * K_LDS_ROW + 16 * g4;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        u32x4 ka;
        if constexpr (KvCoded<KVT>::value) {
          const u32x4 src = *reinterpret_cast<const u32x4*>(krow + 64 * (kk >> 1));
          const int o2 = (kk & 1) * 2;
          ka[0] = code2_to_bf16x2<KVT, false>(src[o2]);
          ka[1] = code2_to_bf16x2<KVT, true>(src[o2]);
          ka[2] = code2_to_bf16x2<KVT, false>(src[o2 + 1]);
          ka[3] = code2_to_bf16x2<KVT, true>(src[o2 + 1]);
        } else {
          ka = *reinterpret_cast<const u32x4*>(krow + 64 * kk);
        }
        acc = mfma16(ka, qb[kk], acc);
      }
      s[blk] = acc;
    }

    // ---- online softmax for head h over the tile's 32 tokens ----
    // lane (g, h) holds tokens 4g + r (block 0) and 16 + 4g + r (block 1)
    float sv[8];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = 16 * blk + 4 * g4 + r;
        sv[4 * blk + r] = (FULL || t0 + tok < t_end) ? s[blk][r] : -INFINITY;
      }
    // Each lane checks its own 8 scores against the head's running max; only
    // when some score exceeds it by more than kSlack (always on the first
    // tile, rarely afterwards) does the wave reduce the max over each head's
    // 4 lanes and rescale.  Until then p stays below 2^kSlack.  Every head
    // has a valid token in every tile, so m is finite from the first tile on.
    float mx = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
    if (__any(mx * smul > m + kSlack)) {
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mn = fmaxf(m, mx * smul);
      const float alpha = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
      l *= alpha;
#pragma unroll
      for (int i = 0; i < DT; ++i) o[i] *= alpha;
      m = mn;
    }
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = __builtin_amdgcn_exp2f(fmaf(sv[i], smul, -m));
      l += p[i];
    }
    u32x4 pb;                                    // P^T as B operand (token order above)
    pb[0] = pack_bf16x2(p[0], p[1]);
    pb[1] = pack_bf16x2(p[2], p[3]);
    pb[2] = pack_bf16x2(p[4], p[5]);
    pb[3] = pack_bf16x2(p[6], p[7]);

    // ---- V rows -> LDS (row-major bf16), zeroing rows past the end ----
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int i = 0; i < LPB; ++i) {
        const int rr = (lane / R) + RPI * i;
        const int tok = 16 * blk + rr;
        u32x4 x = cur.v[blk * LPB + i];
        if (!FULL && t0 + tok >= t_end) x = u32x4{0, 0, 0, 0};
        if constexpr (KvCoded<KVT>::value) {
          u32x4 lo, hi;
          code16_to_bf16<KVT>(x, lo, hi);
          uint8_t* dst = lds + tok * LDS_ROW + (lane % R) * 32;
          *reinterpret_cast<u32x4*>(dst) = lo;
          *reinterpret_cast<u32x4*>(dst + 16) = hi;
        } else {
          *reinterpret_cast<u32x4*>(lds + tok * LDS_ROW + (lane % R) * 16) = x;
        }
      }
    }

    // ---- O^T += V^T P^T, V^T from the LDS image by transpose reads ----
    // lane (g, i) of a 16-lane group reads 4 bf16 of row 4g + i/4 (and 16 + ...)
    // at columns n0 + 4*(i%4); the hardware hands lane i column n0 + i.
    const int rd_row0 = 4 * g4 + (h >> 2);
    const int rd_col = 4 * (h & 3);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      typedef s16x4 __attribute__((address_space(3))) * lds_s16x4_ptr;
      const uint32_t off0 = (uint32_t)(rd_row0 * LDS_ROW + (16 * dt + rd_col) * 2);
      const uint32_t off1 = off0 + 16 * LDS_ROW;
      __attribute__((address_space(3))) uint8_t* base =
          (__attribute__((address_space(3))) uint8_t*)(lds);
      s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(base + off0));
      s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(base + off1));
      u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
      u32x4 va = {w0[0], w0[1], w1[0], w1[1]};
      o[dt] = mfma16(va, pb, o[dt]);
    }
  };
  const std::integral_constant<bool, true> kFull;
  const std::integral_constant<bool, false> kPartial;
  // step(k, cur, nxt): load tile k+1 into nxt (its pages are pn0/pn1), read
  // the pages of tile k+2, compute tile k (never the range's last) from cur.
  auto step = [&](int k, const TR& cur, TR& nxt) {
    const int tn = tw0 + (k + 1) * STRIDE;
    load_tile<KVT, D>(nxt, kp, vp, pn0, pn1, tn, t_end, Hkv, j, pshift, loff);
    if (k + 2 < nt) tile_pages(pages, first, tn + STRIDE, t_end, pshift, pn0, pn1);
    compute(cur, tw0 + k * STRIDE, kFull);
  };
  auto last = [&](const TR& cur, const int t0) { compute(cur, t0, kPartial); };
  int k = 0;
  for (; k + 2 < nt; k += 2) {
    step(k, buf0, buf1);
    step(k + 1, buf1, buf0);
  }
  if (k + 1 < nt) {                              // two tiles left: buf0 holds tile k
    step(k, buf0, buf1);
    last(buf1, tw0 + (k + 1) * STRIDE);
  } else if (k < nt) {                           // one tile left
    last(buf0, tw0 + k * STRIDE);
  }

  // ---- merge: 4 lanes per head within the wave (l is lane-partial) ----
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);

  // ---- merge the 4 waves through LDS ----
  __syncthreads();                               // all V slices consumed
  float* sm_o = reinterpret_cast<float*>(smem);  // [kWaves][16][OROW]
  float* sm_ml = sm_o + kWaves * 16 * OROW;      // [kWaves][16][2]
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) sm_o[(w * 16 + h) * OROW + 16 * dt + 4 * g4 + r] = o[dt][r];
  if (g4 == 0) { sm_ml[(w * 16 + h) * 2] = m; sm_ml[(w * 16 + h) * 2 + 1] = l; }
  __syncthreads();
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
    const int hh = i / D, d = i - hh * D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm_ml[(ww * 16 + hh) * 2]);
    float lt = 0.0f, at = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float mw = sm_ml[(ww * 16 + hh) * 2];
      const float f = (mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
      lt = fmaf(sm_ml[(ww * 16 + hh) * 2 + 1], f, lt);
      at = fmaf(sm_o[(ww * 16 + hh) * OROW + d], f, at);
    }
    const int hq = j * G + hh;
    if (n_split == 1) {
      static_cast<uint16_t*>(a.out)[(qrow * Hq + hq) * D + d] = f32_to_bf16_rne(at * vscale / lt);
      if (d == 0 && a.lse) a.lse[qrow * Hq + hq] = (M + __log2f(lt)) * kLn2;
    } else {
      const size_t slot = ((size_t)z * Hq + hq) * a.max_splits + split;
      a.ws_acc[slot * D + d] = at * vscale;
      if (d == 0) { a.ws_ml[slot * 2] = M; a.ws_ml[slot * 2 + 1] = lt; }
    }
  }
}

}  // namespace

bool decode_mfma_supported(const AttnArgs& a) {
  const int G = a.num_q_heads / a.c.num_kv_heads;
  return !a.prefill && G >= 3 && G <= 16 && a.c.kv_dtype != KV_F32 &&
         (a.c.head_dim == 64 || a.c.head_dim == 128) &&
         (a.split_tokens >> a.page_shift) + 2 <= kMaxRangePages;
}

namespace {
template <bool STEP>
void launch_mfma_step(const AttnArgs& a, dim3 grid, hipStream_t s) {
  const dim3 block(256);
  if (a.c.kv_dtype == KV_BF16) {
    if (a.c.head_dim == 128) hipLaunchKernelGGL((decode_partial_mfma<KV_BF16, 128, STEP>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((decode_partial_mfma<KV_BF16, 64, STEP>), grid, block, 0, s, a);
  } else if (a.c.kv_dtype == KV_FP8) {
    if (a.c.head_dim == 128) hipLaunchKernelGGL((decode_partial_mfma<KV_FP8, 128, STEP>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((decode_partial_mfma<KV_FP8, 64, STEP>), grid, block, 0, s, a);
  } else {
    if (a.c.head_dim == 128) hipLaunchKernelGGL((decode_partial_mfma<KV_INT8, 128, STEP>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((decode_partial_mfma<KV_INT8, 64, STEP>), grid, block, 0, s, a);
  }
}
}  // namespace

hipError_t launch_decode_partial_mfma(const AttnArgs& a, hipStream_t s) {
  const dim3 grid = a.plan ? decode_plan_grid(a) : dim3(a.c.num_kv_heads, a.num_rows, a.max_splits);
  if (a.new_k) launch_mfma_step<true>(a, grid, s);
  else launch_mfma_step<false>(a, grid, s);
  return hipGetLastError();
}

}  // namespace pkv
