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

enum KvType : int { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2 };

template <int KVT> struct KvBytes;
template <> struct KvBytes<KV_F32> { static constexpr int value = 4; };
template <> struct KvBytes<KV_BF16> { static constexpr int value = 2; };
template <> struct KvBytes<KV_FP8> { static constexpr int value = 1; };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
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

// Four fp8 e4m3fn codes (one dword, byte 0 first) -> four floats.
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* o) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(w), false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(w), true);
  o[0] = lo.x; o[1] = lo.y; o[2] = hi.x; o[3] = hi.y;
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

// 16 bytes from global memory (non-temporal hint off: K/V pages may be reused
// by other work items through the shared prefix).
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Sum / max over aligned groups of N lanes (N a power of two <= 64).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = 1; m < N; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

}  // namespace pkv
