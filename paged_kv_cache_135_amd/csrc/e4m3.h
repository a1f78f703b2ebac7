// f32 -> OCP E4M3 ("FN" variant) encoder shared by the HIP kernels that store
// into an E4M3 cache.  Device code only: include from .hip sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Round to nearest, ties to even; |y| >= 448 and infinities saturate to +-448;
// NaN gives 0x7F.
__device__ __forceinline__ uint32_t e4m3_from_f32(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;             // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;     // >= 448 or inf
  if (a < 0x3c800000u) {                         // < 2^-6: multiples of 2^-9
    const float f = __uint_as_float(a) * 512.0f; // exact power-of-two scaling
    return sign | (uint32_t)__builtin_rintf(f);  // 8 rounds up to the smallest normal
  }
  // keep 3 mantissa bits, ties to even, carry into the exponent
  const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
  return sign | ((r >> 20) - (120u << 3));       // rebias 127 -> 7
}

// Four bf16 values (two packed dwords) -> four E4M3 codes in one dword,
// element order preserved (low half first).
__device__ __forceinline__ uint32_t e4m3x4_from_bf16x4(uint32_t w0, uint32_t w1, float inv) {
  const float x0 = __uint_as_float(w0 << 16), x1 = __uint_as_float(w0 & 0xffff0000u);
  const float x2 = __uint_as_float(w1 << 16), x3 = __uint_as_float(w1 & 0xffff0000u);
  return e4m3_from_f32(x0 * inv) | (e4m3_from_f32(x1 * inv) << 8) |
         (e4m3_from_f32(x2 * inv) << 16) | (e4m3_from_f32(x3 * inv) << 24);
}

// The same four codes through gfx950's pack-convert (round to nearest even).
// The inputs are first clamped to +-448 with the NaN-propagating minimum /
// maximum, so the instruction never overflows (the saturating behaviour above)
// and a NaN input stays NaN; the convert gives 0x7F or 0xFF for it.  No
// clamped finite value has all seven low bits set (448 is 0x7E), so those
// bytes are exactly the NaNs, and clearing their sign bit makes them 0x7F.
// Equal to the encoder above on every bf16 value at several scales (checked
// exhaustively on the GPU).
__device__ __forceinline__ uint32_t e4m3x4_cvt(float y0, float y1, float y2, float y3) {
  auto c = [](float v) {
    return __builtin_elementwise_minimum(__builtin_elementwise_maximum(v, -448.0f), 448.0f);
  };
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c(y0), c(y1), 0, false);
  w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c(y2), c(y3), (int)w, true);
  const uint32_t nan_sign = ((w & 0x7f7f7f7fu) + 0x01010101u) & 0x80808080u;
  return w & ~nan_sign;
}

// Four bf16 values (two packed dwords, low half first) times inv -> four codes.
__device__ __forceinline__ uint32_t e4m3x4_cvt_bf16(uint32_t w0, uint32_t w1, float inv) {
  return e4m3x4_cvt(__uint_as_float(w0 << 16) * inv, __uint_as_float(w0 & 0xffff0000u) * inv,
                    __uint_as_float(w1 << 16) * inv, __uint_as_float(w1 & 0xffff0000u) * inv);
}

// Four f32 values -> four E4M3 codes in one dword.
__device__ __forceinline__ uint32_t e4m3x4_from_f32x4(float x0, float x1, float x2, float x3,
                                                      float inv) {
  return e4m3_from_f32(x0 * inv) | (e4m3_from_f32(x1 * inv) << 8) |
         (e4m3_from_f32(x2 * inv) << 16) | (e4m3_from_f32(x3 * inv) << 24);
}

}  // namespace pkv
