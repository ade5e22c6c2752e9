// Device helpers for the paged KV-cache kernels (gfx950, wave64).
//
// Storage conversions:
//   bf16  : the upper 16 bits of an IEEE float32 (float32 -> bf16 rounds to
//           nearest even).
//   fp8   : OCP e4m3fn, bias 7, largest finite 448, no infinities, NaN = S.1111.111.
//           Decode uses gfx950's hardware conversion (v_cvt_pk_f32_fp8, OCP
//           formats on this target), checked against the format definition
//           by the library's own tests.  Encode is written here from the
//           definition: round to nearest even on the 3-bit mantissa,
//           saturate to +-448, keep NaN and the sign.
// KV-cache quantization keeps one scale per attention head and dequantises
// inside the attention kernel ("TensorRT-LLM框架解析与高性能推理优化实践", §7.2).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

enum KvType : int { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2, KV_INT8 = 3 };

template <int KVT> struct KvBytes;
template <> struct KvBytes<KV_F32> { static constexpr int value = 4; };
template <> struct KvBytes<KV_BF16> { static constexpr int value = 2; };
template <> struct KvBytes<KV_FP8> { static constexpr int value = 1; };
template <> struct KvBytes<KV_INT8> { static constexpr int value = 1; };

// 8-bit codes with one scale per KV head (fp8 e4m3fn or symmetric int8):
// stored code = encode(x / scale), value = code * scale.
template <int KVT> struct KvCoded { static constexpr bool value = KVT == KV_FP8 || KVT == KV_INT8; };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float32 -> bf16 bits, round to nearest even; NaN -> quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Two floats -> packed bf16 pair (low = a), round to nearest even
// (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
  const f2_t x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, b2_t));
}

// Four fp8 e4m3fn codes (one dword, byte 0 first) -> four floats.
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* o) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(w), false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(w), true);
  o[0] = lo.x; o[1] = lo.y; o[2] = hi.x; o[3] = hi.y;
}

// Two fp8 e4m3fn codes (bytes 2*HI, 2*HI+1 of w) -> two bf16 packed in a dword
// (exact: every e4m3fn value is a bf16 value).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  typedef __bf16 bf16x2_t __attribute__((__vector_size__(4)));
  bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(w), 1.0f, HI);
  return __builtin_bit_cast(uint32_t, r);
}

// float32 -> e4m3fn code.
//   |y| >= 448 (or inf)      -> 448 with y's sign (saturation)
//   2^-6 <= |y| < 448 (normal): keep exponent E, round the 23-bit mantissa to
//                             3 bits to nearest even; a carry into bit 3 moves
//                             to the next binade by plain addition of codes.
//   |y| < 2^-6 (subnormal)   : code = rint(|y| * 2^9) in 0..8 (8 is the
//                             smallest normal, which is also code 8).
__device__ __forceinline__ uint32_t f32_to_e4m3fn(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;              // NaN
  const float af = __uint_as_float(a);
  if (af >= 448.0f) return sign | 0x7Eu;
  if (af < 0.015625f) {                                    // below 2^-6
    return sign | uint32_t(__builtin_rintf(af * 512.0f));  // exact scaling, RNE
  }
  const uint32_t e = (a >> 23) - 127u + 7u;                // biased e4m3 exponent, 1..15
  const uint32_t mant = a & 0x7FFFFFu;
  const uint32_t keep = mant >> 20;                        // top 3 mantissa bits
  const uint32_t rest = mant & 0xFFFFFu;                   // 20 dropped bits
  const uint32_t half = 0x80000u;
  const uint32_t up = (rest > half) || (rest == half && (keep & 1u));
  return sign | ((e << 3) + keep + up);
}

// Symmetric int8 code of a float32 quotient q = x / scale: the nearest
// integer, ties to even (v_rndne), saturated to [-127, 127]; NaN -> 0.
__device__ __forceinline__ uint32_t f32_to_int8_sym(float q) {
  if (q != q) return 0u;
  const float r = fminf(fmaxf(__builtin_rintf(q), -127.0f), 127.0f);
  return uint32_t(int32_t(r)) & 0xFFu;
}

template <int KVT>
__device__ __forceinline__ uint32_t f32_to_code(float q) {
  if constexpr (KVT == KV_FP8) return f32_to_e4m3fn(q);
  else return f32_to_int8_sym(q);
}

// Four int8 codes (one dword, byte 0 first) -> four floats (exact).
__device__ __forceinline__ void int8x4_to_f32(uint32_t w, float* o) {
  o[0] = float(int8_t(w));
  o[1] = float(int8_t(w >> 8));
  o[2] = float(int8_t(w >> 16));
  o[3] = float(int8_t(w >> 24));
}

// Two int8 codes (bytes 2*HI, 2*HI+1 of w) -> two bf16 in a dword (exact:
// integers of magnitude <= 128 are bf16 values).
template <bool HI>
__device__ __forceinline__ uint32_t int8x2_to_bf16x2(uint32_t w) {
  const uint32_t x = HI ? (w >> 16) : w;
  return pack_bf16x2(float(int8_t(x)), float(int8_t(x >> 8)));
}

// 16 bytes from global memory.
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// 16 bytes with the non-temporal hint: for K/V rows that one pass reads once
// (decode).  On MI355X streaming reads sustain markedly more bandwidth with
// the hint than without it.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// DPP lane moves within a row of 16 lanes (gfx9 DPP controls).
enum : int {
  DPP_XOR1 = 0xB1,        // quad_perm [1,0,3,2]
  DPP_XOR2 = 0x4E,        // quad_perm [2,3,0,1]
  DPP_HALF_MIRROR = 0x141,  // lane i <-> 7-i inside each half row
  DPP_MIRROR = 0x140,       // lane i <-> 15-i inside each row
};

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N consecutive lanes (N a power of two <= 64);
// every lane of a group receives the group's sum.  Inside a 16-lane row the
// steps are DPP moves folded into the adds; wider groups cross rows with a
// lane shuffle.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp_mov<DPP_XOR1>(x);
  if constexpr (N >= 4) x += dpp_mov<DPP_XOR2>(x);
  if constexpr (N >= 8) x += dpp_mov<DPP_HALF_MIRROR>(x);
  if constexpr (N >= 16) x += dpp_mov<DPP_MIRROR>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16, 64);
  if constexpr (N >= 64) x += __shfl_xor(x, 32, 64);
  return x;
}

// Marks a loaded register as consumed here.  Registers that are loaded before
// a loop and only read inside it (MFMA operands held for the whole loop) would
// otherwise be treated as possibly in flight at every iteration, and since
// vector-memory counters retire in order, each wait for them would also wait
// for the prefetch loads issued in that iteration.
__device__ __forceinline__ void settle(const u32x4& x) { asm volatile("" ::"v"(x)); }

// Wave-uniform copy of a value (lets the compiler keep it in an SGPR).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Generic 8-bit code converters (fp8 e4m3fn or int8), exact.
template <int KVT>
__device__ __forceinline__ void code4_to_f32(uint32_t w, float* o) {
  if constexpr (KVT == KV_FP8) fp8x4_to_f32(w, o);
  else int8x4_to_f32(w, o);
}

template <int KVT, bool HI>
__device__ __forceinline__ uint32_t code2_to_bf16x2(uint32_t w) {
  if constexpr (KVT == KV_FP8) return fp8x2_to_bf16x2<HI>(w);
  else return int8x2_to_bf16x2<HI>(w);
}

// 16 codes -> 16 bf16 (lo: codes 0..7, hi: codes 8..15).
template <int KVT>
__device__ __forceinline__ void code16_to_bf16(const u32x4& x, u32x4& lo, u32x4& hi) {
  lo[0] = code2_to_bf16x2<KVT, false>(x[0]); lo[1] = code2_to_bf16x2<KVT, true>(x[0]);
  lo[2] = code2_to_bf16x2<KVT, false>(x[1]); lo[3] = code2_to_bf16x2<KVT, true>(x[1]);
  hi[0] = code2_to_bf16x2<KVT, false>(x[2]); hi[1] = code2_to_bf16x2<KVT, true>(x[2]);
  hi[2] = code2_to_bf16x2<KVT, false>(x[3]); hi[3] = code2_to_bf16x2<KVT, true>(x[3]);
}

}  // namespace pkv
