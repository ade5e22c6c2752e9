// Chunked prefill on the matrix cores.
//
// Method: a context chunk of C new tokens of request r (already appended to
// its pages after P_r cached tokens) attends causally: chunk row i, at
// absolute position P_r + i, sees keys 0 .. P_r + i through the request's
// block table ("TensorRT-LLM框架解析与高性能推理优化实践" §5.3 分块上下文处理; causal
// mask and scaled dot-product attention of the fused-MHA pseudocode in
// "TensorRT-LLM性能调优：提升LLM推理效率"; running max / sum, §6.1).
//
// Work decomposition (MI355X): the G query heads that share KV head j, times
// the chunk's tokens, form "rows" (row = token*G + head).  A workgroup owns 128
// consecutive rows of one (request, KV head) — 32 per wave, two MFMA N-tiles
// that share every K and V^T operand read from LDS — and one range of
// split_tokens keys out of 0 .. (its last row's position), walked in 32-token
// tiles.  Long contexts thus spread over several workgroups instead of one
// long serial walk; rows whose keys span several ranges leave (m, l, acc)
// partials that the log-sum-exp merge combines, the same way split decode
// does.  Each K/V tile is fetched from the pages once per workgroup into LDS
// and shared by the four waves, with the range's block-table entries staged
// in LDS so no load waits on another.  Two kernels share this decomposition:
// prefill_mfma_lds (bf16 caches) loads tiles straight into LDS, two tiles
// ahead; prefill_mfma (8-bit caches) stages them through registers, three
// tiles ahead, widening the codes to bf16 on the way.  Both compute
//
//   S^T[t][row] = sum_d K[t][d] Q[row][d]    A = K from LDS (16-byte reads),
//                                            B = Q^T in registers
//   O^T[d][row] += sum_t V[t][d] P^T[t][row] A = V^T by LDS transpose reads,
//                                            B = P^T straight from S^T's layout
//
// with the operand layouts described in decode_mfma.hip.  Bank conflicts of
// the 16-byte K reads and the transpose reads of V are avoided by padded LDS
// rows in prefill_mfma (K by 16 bytes, V by 32) and by a slot permutation of
// unpadded rows in prefill_mfma_lds (see lds_swz).  Workgroups that share a
// (request, KV head) — and so the same K/V tiles — are mapped to the same
// XCD so those tiles are served from that XCD's L2.
#include <math.h>

#include <type_traits>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;
constexpr int kNt = 2;                      // 16-row MFMA N-tiles per wave
constexpr int kRows = 16 * kNt * kWaves;    // rows per workgroup
constexpr int kTile = 32;                   // keys per tile
constexpr int kMaxPages = 512;              // block-table entries staged per workgroup
// Tile buffers of the bf16 kernel: three (two tiles in flight) measured better
// than four, whose 66 KiB of LDS per workgroup crowd out decode workgroups in
// a mixed step.
constexpr int kTileBufs = 3;

typedef __bf16 bf16x8_t __attribute__((__vector_size__(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}


template <int KVT, int D>
struct PfShape {
  static constexpr int KVB = KvBytes<KVT>::value;
  static constexpr int ROWB = D * KVB;                     // pool bytes per token row
  static constexpr int PIECES = kTile * ROWB / 16;         // 16-byte pieces per K (or V) tile
  static constexpr int PPT = (PIECES + 255) / 256;         // pieces per thread per tile
  static constexpr int K_LDS = D * 2 + 16;                 // padded bf16 rows in LDS
  static constexpr int V_LDS = D * 2 + 32;
  static constexpr int STAGE = kTile * (K_LDS + V_LDS);    // one buffer (K + V)
  static_assert(PIECES % 256 == 0 || PIECES < 256, "tile must split evenly over the workgroup");
};

// Global loads of one K/V tile (pool storage format) into registers.
template <int KVT, int D>
struct PfRegs {
  u32x4 k[PfShape<KVT, D>::PPT];
  u32x4 v[PfShape<KVT, D>::PPT];
};

// K/V rows come from the pages (PAGED) or, for context attention over a
// whole prompt, from contiguous packed [tokens][Hkv][D] arrays whose request
// r starts at row c0.
template <int KVT, int D, bool PAGED>
__device__ __forceinline__ void pf_load(PfRegs<KVT, D>& r, const uint8_t* kp, const uint8_t* vp,
                                        const int32_t* pages, int pg0, int c0, int t0, int kmax,
                                        int Hkv, int j, int pshift) {
  // Every call issues the same loads: pieces past kmax (or past the tile)
  // read the first 16 bytes of the pools instead, and pf_store zeroes them.
  // A fixed load count keeps the waits for older tiles exact.
  using S = PfShape<KVT, D>;
  constexpr int PR = S::ROWB / 16;                          // pieces per row
  const int pmask = (1 << pshift) - 1;
#pragma unroll
  for (int i = 0; i < S::PPT; ++i) {
    const int piece = threadIdx.x + 256 * i;
    const int tok = piece / PR, pc = piece % PR;
    const int t = t0 + tok;
    const bool ok = piece < S::PIECES && t < kmax;
    size_t off = 0;
    if constexpr (PAGED) {
      const int page = ok ? pages[(t >> pshift) - pg0] : 0;
      off = ok ? ((((size_t)page * Hkv + j) << pshift | (size_t)(t & pmask)) * S::ROWB) +
                     (size_t)pc * 16
               : 0;
    } else {
      off = ok ? ((size_t)(c0 + t) * Hkv + j) * S::ROWB + (size_t)pc * 16 : 0;
    }
    r.k[i] = ld16(kp + off);
    r.v[i] = ld16(vp + off);
  }
}

// Registers -> LDS (bf16 rows, padded); rows at or past kmax (the range end) become zeros
// (masked keys must carry finite values: their probability is exactly 0).
template <int KVT, int D>
__device__ __forceinline__ void pf_store(PfRegs<KVT, D> r, uint8_t* kl, uint8_t* vl, int t0,
                                         int kmax) {
  using S = PfShape<KVT, D>;
  constexpr int PR = S::ROWB / 16;
  if (t0 + kTile > kmax) {                       // last tile of the range only
#pragma unroll
    for (int i = 0; i < S::PPT; ++i) {
      const int piece = threadIdx.x + 256 * i;
      if (t0 + piece / PR >= kmax) {
        r.k[i] = u32x4{0, 0, 0, 0};
        r.v[i] = u32x4{0, 0, 0, 0};
      }
    }
  }
#pragma unroll
  for (int i = 0; i < S::PPT; ++i) {
    const int piece = threadIdx.x + 256 * i;
    const int tok = piece / PR, pc = piece % PR;
    if (piece >= S::PIECES) continue;
    if constexpr (KvCoded<KVT>::value) {
      u32x4 klo, khi, vlo, vhi;
      code16_to_bf16<KVT>(r.k[i], klo, khi);
      code16_to_bf16<KVT>(r.v[i], vlo, vhi);
      *reinterpret_cast<u32x4*>(kl + tok * S::K_LDS + pc * 32) = klo;
      *reinterpret_cast<u32x4*>(kl + tok * S::K_LDS + pc * 32 + 16) = khi;
      *reinterpret_cast<u32x4*>(vl + tok * S::V_LDS + pc * 32) = vlo;
      *reinterpret_cast<u32x4*>(vl + tok * S::V_LDS + pc * 32 + 16) = vhi;
    } else {
      *reinterpret_cast<u32x4*>(kl + tok * S::K_LDS + pc * 16) = r.k[i];
      *reinterpret_cast<u32x4*>(vl + tok * S::V_LDS + pc * 16) = r.v[i];
    }
  }
}

// A row's running max moves only when one of its scores exceeds it by more
// than this (log2 units): until then probabilities are taken against the
// older, smaller max and stay below 2^kSlack — well inside fp32 and bf16
// range — and both the cross-lane max and the O / l rescale are skipped.
// The final (m, l, acc) describes the same softmax whichever shift was used.
constexpr float kSlack = 8.0f;

template <int KVT, int D, bool PAGED>
__global__ __launch_bounds__(256, 2) void prefill_mfma(AttnArgs a, int nqb, int npg) {
  using S = PfShape<KVT, D>;
  constexpr int KK = D / 32, DT = D / 16;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * S::STAGE + kMaxPages * 4];

  const int Hq = a.num_q_heads, Hkv = a.c.num_kv_heads, G = Hq / Hkv;
  // XCD-aware order: the hardware places workgroup b on XCD b % 8.  Pair
  // p = (request, KV head) goes to XCD p % 8 — all query blocks of a pair
  // share that XCD's L2, and consecutive pairs (the heads of one request)
  // spread over all XCDs so no XCD gets one request's whole load.  Within an
  // XCD the order is key range (outermost), pair group, then query block
  // from the last (heaviest) down.  Grid size is 8 * npg * nqb * ranges with
  // npg = ceil(pairs / 8); items past the last pair or the block's keys exit.
  const int b = blockIdx.x;
  const int xcd = b % 8, k = b / 8;
  const int per_range = npg * nqb;
  const int rng = k / per_range, kr = k - rng * per_range;
  const int pair = (kr / nqb) * 8 + xcd;
  const int qb_rev = kr % nqb;
  if (pair >= a.num_rows * Hkv) return;
  const int j = pair % Hkv, r = pair / Hkv;
  const int c0 = a.cu_q[r], C = a.cu_q[r + 1] - c0;
  const int qb = nqb - 1 - qb_rev;               // later (heavier) query blocks first
  const int row0 = qb * kRows;                   // first flat row (token*G + head) of the block
  if (row0 >= C * G) return;
  const int Pr = PAGED ? a.ctx_before[r] : 0;    // a whole prompt has nothing cached before it
  const int last_row = min(C * G, row0 + kRows) - 1;
  const int kneed = Pr + last_row / G + 1;       // keys needed by the block's last row
  const int t_begin = rng * a.split_tokens;      // this workgroup's key range
  if (t_begin >= kneed) return;
  const int kmax = min(kneed, t_begin + a.split_tokens);

  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int g4 = lane >> 4, n = lane & 15;
  const int wrow0 = row0 + kNt * 16 * w;         // first row of this wave
  const int wave_last = min(C * G, wrow0 + kNt * 16) - 1;    // last real row of this wave
  const int wave_kmax = wave_last >= wrow0 ? Pr + wave_last / G + 1 : 0;
  const int wave_min_lim = Pr + wrow0 / G;       // smallest key limit in the wave

  float kscale = 1.0f, vscale = 1.0f;
  if constexpr (KvCoded<KVT>::value) { kscale = a.c.k_scale[j]; vscale = a.c.v_scale[j]; }
  const float smul = a.sm_scale * kLog2e * kscale;

  // Per N-tile nt: this lane's row (column n of S^T / O^T) and its Q^T
  // B operand: lane (g4, n) holds Q[row][g4*D/4 + 8kk + e].
  int my_lim[kNt];
  bool row_ok[kNt];
  size_t row_off[kNt];
  u32x4 qb_reg[kNt][KK];
#pragma unroll
  for (int nt = 0; nt < kNt; ++nt) {
    const int my_row = wrow0 + 16 * nt + n;
    row_ok[nt] = my_row < C * G;
    const int my_tok = my_row / G, my_head = my_row - my_tok * G;
    my_lim[nt] = Pr + my_tok;
    row_off[nt] = ((size_t)(c0 + my_tok) * Hq + (size_t)j * G + my_head) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qb_reg[nt][kk] = u32x4{0, 0, 0, 0};
    if (row_ok[nt]) {
      const uint16_t* q = static_cast<const uint16_t*>(a.q) + row_off[nt];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) qb_reg[nt][kk] = ld16(q + (D / 4) * g4 + 8 * kk);
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) settle(qb_reg[nt][kk]);
  }

  // Row sums l come from the matrix cores too: an all-ones A operand times
  // P^T gives sum_t P[row][t] in every element of the row's lanes — from the
  // same bf16 P that multiplies V, with no VALU adds or cross-lane sums.
  f32x4 o[kNt][DT];
  f32x4 lsum[kNt];
  float m[kNt];
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};   // bf16 1.0 pairs
#pragma unroll
  for (int nt = 0; nt < kNt; ++nt) {
#pragma unroll
    for (int i = 0; i < DT; ++i) o[nt][i] = f32x4{0, 0, 0, 0};
    m[nt] = -INFINITY;
    lsum[nt] = f32x4{0, 0, 0, 0};
  }

  const uint8_t* kp = static_cast<const uint8_t*>(a.c.k_pool);
  const uint8_t* vp = static_cast<const uint8_t*>(a.c.v_pool);
  const int ntiles = (kmax - t_begin + kTile - 1) / kTile;
  const int pshift = a.page_shift;

  // The block-table entries for keys t_begin .. kmax-1, staged in LDS once;
  // pf_load indexes them by absolute page number minus pg0.
  int32_t* pages = reinterpret_cast<int32_t*>(smem + 2 * S::STAGE);
  const int pg0 = t_begin >> pshift;
  if constexpr (PAGED) {
    const int32_t* btrow = a.bt + (size_t)r * a.bt_stride;
    const int npages = ((kmax - 1) >> pshift) - pg0 + 1;
    for (int i = threadIdx.x; i < npages; i += blockDim.x) pages[i] = btrow[pg0 + i];
    __syncthreads();
  }

  // Pipeline: tile t is staged in register set t % 3 and LDS buffer t % 2.
  // While tile i is computed, the loads of tiles i+2 and i+3 are in flight
  // and tile i+1 (loaded two steps earlier) is written to the other LDS
  // buffer, so each load has two compute steps to land.
  PfRegs<KVT, D> r0, r1, r2;
  pf_load<KVT, D, PAGED>(r0, kp, vp, pages, pg0, c0, t_begin, kmax, Hkv, j, pshift);
  pf_load<KVT, D, PAGED>(r1, kp, vp, pages, pg0, c0, t_begin + kTile, kmax, Hkv, j, pshift);
  pf_load<KVT, D, PAGED>(r2, kp, vp, pages, pg0, c0, t_begin + 2 * kTile, kmax, Hkv, j, pshift);
  pf_store<KVT, D>(r0, smem, smem + kTile * S::K_LDS, t_begin, kmax);
  __syncthreads();

  auto step = [&](int it, PfRegs<KVT, D>& rfree, const PfRegs<KVT, D>& rnext) {
    const int t0 = t_begin + it * kTile;
    uint8_t* kl = smem + (it & 1) * S::STAGE;
    uint8_t* vl = kl + kTile * S::K_LDS;
    pf_load<KVT, D, PAGED>(rfree, kp, vp, pages, pg0, c0, t0 + 3 * kTile, kmax, Hkv, j, pshift);

    if (t0 < wave_kmax) {                        // skip tiles wholly above this wave's diagonal
      // ---- S^T for the two 16-key blocks; each K operand feeds every N-tile ----
      f32x4 s[kNt][2];
#pragma unroll
      for (int nt = 0; nt < kNt; ++nt) s[nt][0] = s[nt][1] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const uint8_t* krow = kl + (16 * blk + n) * S::K_LDS + g4 * (D / 4) * 2;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const u32x4 ka = *reinterpret_cast<const u32x4*>(krow + 16 * kk);
#pragma unroll
          for (int nt = 0; nt < kNt; ++nt) s[nt][blk] = mfma16(ka, qb_reg[nt][kk], s[nt][blk]);
        }
      }
      // ---- online softmax per N-tile; the scale enters the exponent as one FMA ----
      const bool diag = t0 + kTile - 1 > wave_min_lim;
      u32x4 pb[kNt];
#pragma unroll
      for (int nt = 0; nt < kNt; ++nt) {
        float sv[8];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) sv[4 * blk + rr] = s[nt][blk][rr];
        if (diag) {
#pragma unroll
          for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
              if (t0 + 16 * blk + 4 * g4 + rr > my_lim[nt]) sv[4 * blk + rr] = -INFINITY;
        }
        // Each lane checks its own 8 scores against the row's running max;
        // only when some score exceeds it by more than kSlack (always on a
        // row's first visible key, rarely afterwards) does the wave reduce
        // the row max over the row's 4 lanes and rescale.  A row whose keys
        // all lie past this range's start sees only masked keys: its m stays
        // -inf and every p below is exp2(-inf) = 0.
        float mx = sv[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
        if (__any(mx * smul > m[nt] + kSlack)) {
          mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
          mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
          const float mn = fmaxf(m[nt], mx * smul);
          // (a row still at -inf has l = 0 and O = 0: any finite factor will do)
          const float alpha = m[nt] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m[nt] - mn);
          lsum[nt] *= alpha;
#pragma unroll
          for (int i = 0; i < DT; ++i) o[nt][i] *= alpha;
          m[nt] = mn;
        }
        const float msub = m[nt] == -INFINITY ? 0.0f : m[nt];
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          p[i] = __builtin_amdgcn_exp2f(fmaf(sv[i], smul, -msub));
        }
        pb[nt][0] = pack_bf16x2(p[0], p[1]);
        pb[nt][1] = pack_bf16x2(p[2], p[3]);
        pb[nt][2] = pack_bf16x2(p[4], p[5]);
        pb[nt][3] = pack_bf16x2(p[6], p[7]);
        lsum[nt] = mfma16(ones, pb[nt], lsum[nt]);
      }
      // ---- O^T += V^T P^T; each V^T operand feeds every N-tile ----
      const int rd_row0 = 4 * g4 + (n >> 2);
      const int rd_col = 4 * (n & 3);
      typedef s16x4 __attribute__((address_space(3))) * lds_s16x4_ptr;
      __attribute__((address_space(3))) uint8_t* vbase = (__attribute__((address_space(3))) uint8_t*)(vl);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint32_t off0 = (uint32_t)(rd_row0 * S::V_LDS + (16 * dt + rd_col) * 2);
        const uint32_t off1 = off0 + 16 * S::V_LDS;
        s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(vbase + off0));
        s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(vbase + off1));
        u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
        const u32x4 va = {w0[0], w0[1], w1[0], w1[1]};
#pragma unroll
        for (int nt = 0; nt < kNt; ++nt) o[nt][dt] = mfma16(va, pb[nt], o[nt][dt]);
      }
    }
    if (it + 1 < ntiles) {
      uint8_t* kn = smem + ((it + 1) & 1) * S::STAGE;
      pf_store<KVT, D>(rnext, kn, kn + kTile * S::K_LDS, t0 + kTile, kmax);
    }
    __syncthreads();
  };

  for (int it = 0; it < ntiles; it += 3) {
    step(it, r0, r1);
    if (it + 1 < ntiles) step(it + 1, r1, r2);
    if (it + 2 < ntiles) step(it + 2, r2, r0);
  }

  // ---- finish rows.  A row whose
  // keys fit one range (L <= split_tokens) is final here; otherwise this
  // range's (m, l, acc) goes to the workspace for the merge, if the row has
  // keys in it. ----
#pragma unroll
  for (int nt = 0; nt < kNt; ++nt) {
    const float lt = lsum[nt][0];
    const int L = my_lim[nt] + 1;                // keys this row attends
    const bool single = L <= a.split_tokens;     // all of them in range 0
    if (row_ok[nt] && single && rng == 0) {
      const float inv = vscale / lt;
      uint16_t* out = static_cast<uint16_t*>(a.out) + row_off[nt];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint32_t lo = pack_bf16x2(o[nt][dt][0] * inv, o[nt][dt][1] * inv);
        const uint32_t hi = pack_bf16x2(o[nt][dt][2] * inv, o[nt][dt][3] * inv);
        *reinterpret_cast<u32x2*>(out + 16 * dt + 4 * g4) = u32x2{lo, hi};
      }
      if (g4 == 0 && a.lse) a.lse[row_off[nt] / D] = (m[nt] + __log2f(lt)) * kLn2;
    } else if (row_ok[nt] && !single && t_begin < L) {
      const size_t slot = (row_off[nt] / D) * a.max_splits + rng;
      float* acc = a.ws_acc + slot * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<f32x4*>(acc + 16 * dt + 4 * g4) = o[nt][dt] * vscale;
      if (g4 == 0) { a.ws_ml[slot * 2] = m[nt]; a.ws_ml[slot * 2 + 1] = lt; }
    }
  }
}


// ---- bf16 caches: K/V tiles loaded straight into LDS ----
//
// gfx950's 16-byte global-to-LDS load writes lane l's data at (the
// instruction's LDS base) + 16 l, so one wave instruction fills 1 KiB of
// consecutive LDS and no register holds the tile on its way.  Rows are
// therefore stored unpadded (2D bytes); instead of padding, the 16-byte piece
// p of row r sits in slot p ^ lds_swz(r), which keeps the K reads and the V
// transpose reads on distinct banks.  NB tile buffers: while tile i is computed, tiles i+1 .. i+NB-1
// are in flight, and one barrier per tile both publishes tile i and frees
// the buffer of tile i-1 for the load of tile i+NB-1.

// Slot permutation of row r (its low 4 bits r3..r0), chosen so that both
// reads stay on distinct banks whether the LDS serves 128 or 256 bytes per
// clock: the K reads (ds_read_b128: 8 or 16 lanes per clock, rows n of one
// 16-row block, one piece) need distinct slots over 8 and over 16 rows; the
// V transpose reads (ds_read_b64: 16 or 32 lanes, 4 or 8 rows, a 32-byte
// slot pair each) need distinct pairs over 4 and over 8 rows.
//   D = 128 (16 slots): s = (r2 ^ r3, r1, r0, r2)   (bits 3..0)
//   D =  64 ( 8 slots): s = (r0 ^ r2, r1, r2 ^ r3)  (bits 2..0; rows are
//                        128 bytes, so r0 already separates row pairs)
template <int D>
__device__ __forceinline__ int lds_swz(int r) {
  const int r0 = r & 1, r1 = (r >> 1) & 1, r2 = (r >> 2) & 1, r3 = (r >> 3) & 1;
  if constexpr (D == 128) return r2 | (r0 << 1) | (r1 << 2) | ((r2 ^ r3) << 3);
  else return (r2 ^ r3) | (r1 << 1) | ((r0 ^ r2) << 2);
}

// s_waitcnt with only the vector-memory counter constrained (<= n).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Workgroup barrier without a memory fence: a fence would also wait for the
// tiles still in flight.  LDS reads of the previous tile have completed (their
// results fed the matrix cores before the barrier is reached); the asm
// statements stop the compiler from moving memory accesses across it.
__device__ __forceinline__ void bar_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// V^T operands of four 16-column d-tiles: for each, the two 16-key halves
// (LDS offsets BASE and BASE + HALF from the lane's address).  Written as
// one asm block that waits for its own reads: the builtin form of this read
// makes the compiler wait for every global-to-LDS load still in flight.
template <int BASE, int HALF>
__device__ __forceinline__ void vt_read4(u32x4 (&va)[4], const uint32_t* addr) {
  u32x2 a0, b0, a1, b1, a2, b2, a3, b3;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%12\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:%13\n\t"
      "ds_read_b64_tr_b16 %2, %9 offset:%12\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:%13\n\t"
      "ds_read_b64_tr_b16 %4, %10 offset:%12\n\t"
      "ds_read_b64_tr_b16 %5, %10 offset:%13\n\t"
      "ds_read_b64_tr_b16 %6, %11 offset:%12\n\t"
      "ds_read_b64_tr_b16 %7, %11 offset:%13\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a0), "=&v"(b0), "=&v"(a1), "=&v"(b1), "=&v"(a2), "=&v"(b2), "=&v"(a3), "=&v"(b3)
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "i"(BASE), "i"(BASE + HALF));
  va[0] = u32x4{a0[0], a0[1], b0[0], b0[1]};
  va[1] = u32x4{a1[0], a1[1], b1[0], b1[1]};
  va[2] = u32x4{a2[0], a2[1], b2[0], b2[1]};
  va[3] = u32x4{a3[0], a3[1], b3[0], b3[1]};
}

// V^T operands of eight 16-column d-tiles (16 transpose reads, one wait).
template <int BASE, int HALF>
__device__ __forceinline__ void vt_read8(u32x4 (&va)[8], const uint32_t* addr) {
  u32x2 a0, b0, a1, b1, a2, b2, a3, b3, a4, b4, a5, b5, a6, b6, a7, b7;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16 offset:%24\n\t"
      "ds_read_b64_tr_b16 %1, %16 offset:%25\n\t"
      "ds_read_b64_tr_b16 %2, %17 offset:%24\n\t"
      "ds_read_b64_tr_b16 %3, %17 offset:%25\n\t"
      "ds_read_b64_tr_b16 %4, %18 offset:%24\n\t"
      "ds_read_b64_tr_b16 %5, %18 offset:%25\n\t"
      "ds_read_b64_tr_b16 %6, %19 offset:%24\n\t"
      "ds_read_b64_tr_b16 %7, %19 offset:%25\n\t"
      "ds_read_b64_tr_b16 %8, %20 offset:%24\n\t"
      "ds_read_b64_tr_b16 %9, %20 offset:%25\n\t"
      "ds_read_b64_tr_b16 %10, %21 offset:%24\n\t"
      "ds_read_b64_tr_b16 %11, %21 offset:%25\n\t"
      "ds_read_b64_tr_b16 %12, %22 offset:%24\n\t"
      "ds_read_b64_tr_b16 %13, %22 offset:%25\n\t"
      "ds_read_b64_tr_b16 %14, %23 offset:%24\n\t"
      "ds_read_b64_tr_b16 %15, %23 offset:%25\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a0), "=&v"(b0), "=&v"(a1), "=&v"(b1), "=&v"(a2), "=&v"(b2), "=&v"(a3), "=&v"(b3),
        "=&v"(a4), "=&v"(b4), "=&v"(a5), "=&v"(b5), "=&v"(a6), "=&v"(b6), "=&v"(a7), "=&v"(b7)
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]),
        "v"(addr[6]), "v"(addr[7]), "i"(BASE), "i"(BASE + HALF));
  va[0] = u32x4{a0[0], a0[1], b0[0], b0[1]};
  va[1] = u32x4{a1[0], a1[1], b1[0], b1[1]};
  va[2] = u32x4{a2[0], a2[1], b2[0], b2[1]};
  va[3] = u32x4{a3[0], a3[1], b3[0], b3[1]};
  va[4] = u32x4{a4[0], a4[1], b4[0], b4[1]};
  va[5] = u32x4{a5[0], a5[1], b5[0], b5[1]};
  va[6] = u32x4{a6[0], a6[1], b6[0], b6[1]};
  va[7] = u32x4{a7[0], a7[1], b7[0], b7[1]};
}

template <int D, bool PAGED, int NB, bool HOIST>
__global__ __launch_bounds__(256, 2) void prefill_mfma_lds(AttnArgs a, int nqb, int npg) {
  static_assert(NB == 3 || NB == 4, "three or four tile buffers");
  constexpr int KK = D / 32, DT = D / 16;
  constexpr int ROWB = 2 * D;                      // bytes per bf16 row
  constexpr int SPR = ROWB / 16;                   // 16-byte slots per row
  constexpr int RPC = 1024 / ROWB;                 // rows per 1 KiB wave load
  constexpr int CPW = kTile * ROWB / 1024 / 4;     // K (and V) loads per wave per tile
  constexpr int NLT = 2 * CPW;                     // loads per thread per tile
  constexpr int KBYTES = kTile * ROWB;
  constexpr int STAGE = 2 * KBYTES;                // K then V
  static_assert(CPW >= 1 && kTile * ROWB == 4096 * CPW, "tile must split evenly over four waves");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NB * STAGE + kMaxPages * 4];

  const int Hq = a.num_q_heads, Hkv = a.c.num_kv_heads, G = Hq / Hkv;
  // Block order as in prefill_mfma: pair p = (request, KV head) on XCD p % 8,
  // key range outermost, heaviest query block first.
  const int b = blockIdx.x;
  const int xcd = b % 8, k = b / 8;
  const int per_range = npg * nqb;
  const int rng = k / per_range, kr = k - rng * per_range;
  const int pair = (kr / nqb) * 8 + xcd;
  const int qb_rev = kr % nqb;
  if (pair >= a.num_rows * Hkv) return;
  const int j = pair % Hkv, r = pair / Hkv;
  const int c0 = a.cu_q[r], C = a.cu_q[r + 1] - c0;
  const int qb = nqb - 1 - qb_rev;
  const int row0 = qb * kRows;
  if (row0 >= C * G) return;
  const int Pr = PAGED ? a.ctx_before[r] : 0;
  const int last_row = min(C * G, row0 + kRows) - 1;
  const int kneed = Pr + last_row / G + 1;
  const int t_begin = rng * a.split_tokens;
  if (t_begin >= kneed) return;
  const int kmax = min(kneed, t_begin + a.split_tokens);

  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int g4 = lane >> 4, n = lane & 15;
  const int wrow0 = row0 + kNt * 16 * w;
  const int wave_last = min(C * G, wrow0 + kNt * 16) - 1;
  const int wave_kmax = wave_last >= wrow0 ? Pr + wave_last / G + 1 : 0;
  const int wave_min_lim = Pr + wrow0 / G;
  const float smul = a.sm_scale * kLog2e;

  int my_lim[kNt];
  bool row_ok[kNt];
  size_t row_off[kNt];
  u32x4 qb_reg[kNt][KK];
#pragma unroll
  for (int nt = 0; nt < kNt; ++nt) {
    const int my_row = wrow0 + 16 * nt + n;
    row_ok[nt] = my_row < C * G;
    const int my_tok = my_row / G, my_head = my_row - my_tok * G;
    my_lim[nt] = Pr + my_tok;
    row_off[nt] = ((size_t)(c0 + my_tok) * Hq + (size_t)j * G + my_head) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qb_reg[nt][kk] = u32x4{0, 0, 0, 0};
    if (row_ok[nt]) {
      const uint16_t* q = static_cast<const uint16_t*>(a.q) + row_off[nt];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) qb_reg[nt][kk] = ld16(q + (D / 4) * g4 + 8 * kk);
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) settle(qb_reg[nt][kk]);
  }

  f32x4 o[kNt][DT];
  f32x4 lsum[kNt];
  float m[kNt];
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
  for (int nt = 0; nt < kNt; ++nt) {
#pragma unroll
    for (int i = 0; i < DT; ++i) o[nt][i] = f32x4{0, 0, 0, 0};
    m[nt] = -INFINITY;
    lsum[nt] = f32x4{0, 0, 0, 0};
  }

  const uint8_t* kp = static_cast<const uint8_t*>(a.c.k_pool);
  const uint8_t* vp = static_cast<const uint8_t*>(a.c.v_pool);
  const int ntiles = (kmax - t_begin + kTile - 1) / kTile;
  const int pshift = a.page_shift;
  const int pmask = (1 << pshift) - 1;

  int32_t* pages = reinterpret_cast<int32_t*>(smem + NB * STAGE);
  const int pg0 = t_begin >> pshift;
  if constexpr (PAGED) {
    const int32_t* btrow = a.bt + (size_t)r * a.bt_stride;
    const int npages = ((kmax - 1) >> pshift) - pg0 + 1;
    for (int i = threadIdx.x; i < npages; i += blockDim.x) pages[i] = btrow[pg0 + i];
  }
  __syncthreads();

  // This lane's part of each wave load: row ld_row[i] of the tile, the
  // swizzled piece that belongs in the lane's slot.
  int ld_row[CPW];
  uint32_t ld_pb[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int c = w * CPW + i;                     // 1 KiB chunk of the K (and V) tile
    ld_row[i] = c * RPC + lane / SPR;
    ld_pb[i] = (uint32_t)(((lane % SPR) ^ lds_swz<D>(ld_row[i])) * 16);
  }
  // Loads of tile `it` into buffer `buf`.  Keys past kmax (only in a range's
  // last tile, all above every row's causal limit) re-read key kmax-1: finite
  // values whose probability is exactly 0.  A wave load's RPC rows are
  // consecutive and RPC-aligned, so they lie in one page (pages hold at least
  // 16 tokens; clamped rows fall in the same page, or the whole load is past
  // kmax): the row base is wave-uniform (scalar registers) and each lane adds
  // a 32-bit offset.
  auto issue = [&](int it, int buf) {
    const int t0 = t_begin + it * kTile;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int tc = uniform(min(t0 + (w * CPW + i) * RPC, kmax - 1));
      const int t = min(t0 + ld_row[i], kmax - 1);
      size_t base;
      uint32_t lo;
      if constexpr (PAGED) {
        const int page = uniform(pages[(tc >> pshift) - pg0]);
        base = (((size_t)page * Hkv + j) << pshift) * ROWB;
        lo = (uint32_t)(t & pmask) * ROWB + ld_pb[i];
      } else {
        base = ((size_t)(c0 + tc) * Hkv + j) * ROWB;
        lo = (uint32_t)(t - tc) * (uint32_t)(Hkv * ROWB) + ld_pb[i];
      }
      uint8_t* kdst = smem + buf * STAGE + (w * CPW + i) * 1024;
      __builtin_amdgcn_global_load_lds(kp + base + lo, (__attribute__((address_space(3))) void*)kdst, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vp + base + lo, (__attribute__((address_space(3))) void*)(kdst + KBYTES), 16, 0, 0);
    }
  };

  typedef u32x4 __attribute__((address_space(3))) * lds_u32x4_ptr;
  __attribute__((address_space(3))) uint8_t* lds = (__attribute__((address_space(3))) uint8_t*)(smem);
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

  // Per-lane LDS read offsets (the buffer and 16-row block enter as
  // constants); the V^T ones are absolute LDS addresses for the asm reads.
  uint32_t k_off[KK], v_off[DT];
  {
    const int sk = lds_swz<D>(n);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) k_off[kk] = n * ROWB + (((g4 * KK + kk) ^ sk) << 4);
    const int vr = 4 * g4 + (n >> 2);
    const int sv = lds_swz<D>(vr);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      v_off[dt] = lds_base + vr * ROWB + (((2 * dt + ((n >> 1) & 1)) ^ sv) << 4) + 8 * (n & 1);
  }

  auto compute = [&](int it, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int t0 = t_begin + it * kTile;
    if (t0 >= wave_kmax) return;                  // tile wholly above this wave's diagonal
    __attribute__((address_space(3))) uint8_t* kl = lds + buf * STAGE;
    // HOIST: the tile's K fragments are all read before its first MFMA (one
    // round of LDS latency instead of one per pair of fragments), and its
    // V^T fragments in one batch after the softmax.  That shortens each
    // workgroup's chain of waits, which decides a launch of about one round
    // of workgroups; with several rounds, the compiler's interleaving of
    // reads and MFMAs lets the two waves of a SIMD overlap better and is
    // kept.
    u32x4 ka[2][KK];
    if constexpr (HOIST) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          ka[blk][kk] = *(lds_u32x4_ptr)(kl + blk * 16 * ROWB + k_off[kk]);
      __builtin_amdgcn_sched_barrier(0);
    }
    f32x4 s[kNt][2];
#pragma unroll
    for (int nt = 0; nt < kNt; ++nt) s[nt][0] = s[nt][1] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if constexpr (!HOIST) ka[blk][kk] = *(lds_u32x4_ptr)(kl + blk * 16 * ROWB + k_off[kk]);
#pragma unroll
        for (int nt = 0; nt < kNt; ++nt) s[nt][blk] = mfma16(ka[blk][kk], qb_reg[nt][kk], s[nt][blk]);
      }
    }
    const bool diag = t0 + kTile - 1 > wave_min_lim;
    u32x4 pb[kNt];
#pragma unroll
    for (int nt = 0; nt < kNt; ++nt) {
      float sv[8];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) sv[4 * blk + rr] = s[nt][blk][rr];
      if (diag) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            if (t0 + 16 * blk + 4 * g4 + rr > my_lim[nt]) sv[4 * blk + rr] = -INFINITY;
      }
      float mx = sv[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
      if (__any(mx * smul > m[nt] + kSlack)) {
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mn = fmaxf(m[nt], mx * smul);
        const float alpha = m[nt] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m[nt] - mn);
        lsum[nt] *= alpha;
#pragma unroll
        for (int i = 0; i < DT; ++i) o[nt][i] *= alpha;
        m[nt] = mn;
      }
      const float msub = m[nt] == -INFINITY ? 0.0f : m[nt];
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(sv[i], smul, -msub));
      pb[nt][0] = pack_bf16x2(p[0], p[1]);
      pb[nt][1] = pack_bf16x2(p[2], p[3]);
      pb[nt][2] = pack_bf16x2(p[4], p[5]);
      pb[nt][3] = pack_bf16x2(p[6], p[7]);
      lsum[nt] = mfma16(ones, pb[nt], lsum[nt]);
    }
    if constexpr (HOIST && DT == 8) {
      u32x4 va[DT];
      vt_read8<buf * STAGE + KBYTES, 16 * ROWB>(va, v_off);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int nt = 0; nt < kNt; ++nt) o[nt][dt] = mfma16(va[dt], pb[nt], o[nt][dt]);
    } else {
#pragma unroll
      for (int d4 = 0; d4 < DT / 4; ++d4) {
        u32x4 va[4];
        vt_read4<buf * STAGE + KBYTES, 16 * ROWB>(va, v_off + 4 * d4);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int nt = 0; nt < kNt; ++nt) o[nt][4 * d4 + i] = mfma16(va[i], pb[nt], o[nt][4 * d4 + i]);
      }
    }
  };

  // Tile it: wait for its loads (only later tiles may stay in flight), one
  // barrier, start tile it+NB-1 in the buffer tile it-1 used, compute tile it.
  auto step = [&](int it, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int pend = min(ntiles - 1 - it, NB - 2);  // tiles after `it` already issued
    if (pend == 2) wait_vm<2 * NLT>();
    else if (pend == 1) wait_vm<NLT>();
    else wait_vm<0>();
    bar_nofence();
    if (it + NB - 1 < ntiles) issue(it + NB - 1, (buf + NB - 1) % NB);
    compute(it, bufc);
  };

  for (int i = 0; i < NB - 1; ++i)
    if (i < ntiles) issue(i, i);
  for (int it = 0; it < ntiles; it += NB) {
    step(it, std::integral_constant<int, 0>());
    if (it + 1 < ntiles) step(it + 1, std::integral_constant<int, 1>());
    if (it + 2 < ntiles) step(it + 2, std::integral_constant<int, 2>());
    if constexpr (NB == 4)
      if (it + 3 < ntiles) step(it + 3, std::integral_constant<int, 3>());
  }

#pragma unroll
  for (int nt = 0; nt < kNt; ++nt) {
    const float lt = lsum[nt][0];
    const int L = my_lim[nt] + 1;
    const bool single = L <= a.split_tokens;
    if (row_ok[nt] && single && rng == 0) {
      const float inv = 1.0f / lt;
      uint16_t* out = static_cast<uint16_t*>(a.out) + row_off[nt];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint32_t lo = pack_bf16x2(o[nt][dt][0] * inv, o[nt][dt][1] * inv);
        const uint32_t hi = pack_bf16x2(o[nt][dt][2] * inv, o[nt][dt][3] * inv);
        *reinterpret_cast<u32x2*>(out + 16 * dt + 4 * g4) = u32x2{lo, hi};
      }
      if (g4 == 0 && a.lse) a.lse[row_off[nt] / D] = (m[nt] + __log2f(lt)) * kLn2;
    } else if (row_ok[nt] && !single && t_begin < L) {
      const size_t slot = (row_off[nt] / D) * a.max_splits + rng;
      float* acc = a.ws_acc + slot * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<f32x4*>(acc + 16 * dt + 4 * g4) = o[nt][dt];
      if (g4 == 0) { a.ws_ml[slot * 2] = m[nt]; a.ws_ml[slot * 2 + 1] = lt; }
    }
  }
}

}  // namespace

// The block-table slice of one key range must fit the LDS staging area: a
// range of split_tokens keys touches at most split/page + 1 pages.  Context
// attention (contiguous bf16 K/V) has no table.
bool prefill_mfma_supported(const AttnArgs& a) {
  if (!a.prefill || (a.c.head_dim != 64 && a.c.head_dim != 128) || a.split_tokens % kTile != 0)
    return false;
  if (a.contiguous) return a.c.kv_dtype == KV_BF16;
  return a.c.kv_dtype != KV_F32 && (a.split_tokens >> a.page_shift) + 1 <= kMaxPages;
}

long long prefill_mfma_grid(const AttnArgs& a) {
  const int G = a.num_q_heads / a.c.num_kv_heads;
  const long long nqb = ((long long)a.max_chunk * G + kRows - 1) / kRows;
  const long long pairs = (long long)a.c.num_kv_heads * a.num_rows;
  return (pairs + 7) / 8 * 8 * nqb * a.max_splits;
}

// Launches of at most this many workgroups (about one round of the
// device's two workgroups per CU, counting the ones that exit at once) take
// the hoisted-read schedule of the bf16 kernel.
constexpr long long kHoistMaxGrid = 1024;

template <int KVT, bool PAGED>
void launch_pf(const AttnArgs& a, dim3 grid, hipStream_t s, int nqb, int npg) {
  if constexpr (KVT == KV_BF16) {
    constexpr int NB = kTileBufs;
    const bool hoist = grid.x <= kHoistMaxGrid;
    if (a.c.head_dim == 128) {
      if (hoist) hipLaunchKernelGGL((prefill_mfma_lds<128, PAGED, NB, true>), grid, dim3(256), 0, s, a, nqb, npg);
      else hipLaunchKernelGGL((prefill_mfma_lds<128, PAGED, NB, false>), grid, dim3(256), 0, s, a, nqb, npg);
    } else {
      if (hoist) hipLaunchKernelGGL((prefill_mfma_lds<64, PAGED, NB, true>), grid, dim3(256), 0, s, a, nqb, npg);
      else hipLaunchKernelGGL((prefill_mfma_lds<64, PAGED, NB, false>), grid, dim3(256), 0, s, a, nqb, npg);
    }
  } else {
    if (a.c.head_dim == 128) hipLaunchKernelGGL((prefill_mfma<KVT, 128, PAGED>), grid, dim3(256), 0, s, a, nqb, npg);
    else hipLaunchKernelGGL((prefill_mfma<KVT, 64, PAGED>), grid, dim3(256), 0, s, a, nqb, npg);
  }
}

hipError_t launch_prefill_mfma(const AttnArgs& a, hipStream_t s) {
  const int G = a.num_q_heads / a.c.num_kv_heads;
  const int nqb = (a.max_chunk * G + kRows - 1) / kRows;
  const int npg = (a.c.num_kv_heads * a.num_rows + 7) / 8;
  const long long nwg = prefill_mfma_grid(a);
  if (nwg == 0) return hipSuccess;
  if (nwg > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nwg);
  if (a.contiguous) launch_pf<KV_BF16, false>(a, grid, s, nqb, npg);
  else if (a.c.kv_dtype == KV_BF16) launch_pf<KV_BF16, true>(a, grid, s, nqb, npg);
  else if (a.c.kv_dtype == KV_FP8) launch_pf<KV_FP8, true>(a, grid, s, nqb, npg);
  else launch_pf<KV_INT8, true>(a, grid, s, nqb, npg);
  return hipGetLastError();
}

}  // namespace pkv
