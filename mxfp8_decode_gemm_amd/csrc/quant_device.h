// Device side of the MXFP8 activation quantizer (gfx950): BF16 values, one
// E8M0 scale per 32 consecutive values along K, e4m3fn codes. Shared by the
// GEMM's quantizing activation stage and the stand-alone quantize kernel.
//
// The rule (the one the GEMM's MXFP8 inputs follow; the pages hand the GEMM
// an MXFP8 activation whose original dtype is BF16, publishing_gemm page,
// PublishingMxfp8Linear.__call__, and do not print the quantizer):
//   * e = the smallest integer with amax <= 448 * 2^e, clamped to
//     [-127, 127] (an all-zero block: -127); scale byte e + 127;
//   * code = e4m3fn nearest to v / 2^e, ties to even, subnormals kept, the
//     sign of the input kept (also when the value rounds to zero);
//   * a block whose largest magnitude is infinite or NaN: scale 0xFF (E8M0
//     NaN) and every code 0x7F with the element's sign (e4m3fn NaN).
//
// Lane layout: each lane holds 8 consecutive BF16 values (one 16-byte
// chunk); the 4 chunks of a 32-value block sit in 4 consecutive lanes
// starting at a multiple of 4, and every lane of the wave takes part (the
// block maximum is exchanged with DPP quad permutes).
//
// The codes come from gfx950's FP8 conversion (v_cvt_pk_fp8_f32: OCP e4m3fn,
// nearest even, sign kept), applied to v * 2^-e. The product is exact:
// 2^-e is a normal FP32 power of two for every finite block, BF16 values
// (subnormals included; the library is built with FP32 denormals kept) are
// exact in FP32, and |v * 2^-e| <= 448, so the conversion never saturates;
// products below 2^-126 are far under half the smallest e4m3 step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxg {

// Largest BF16 magnitude (15-bit pattern) of the 8 values of a chunk. The
// magnitude patterns of finite values order like the values; infinities
// and NaNs order above every finite value.
typedef unsigned short mxg_u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t chunk_amax(const uint4 v) {
  // Two 16-bit lanes at a time (packed integer max), then the two halves.
  const mxg_u16x2 a = __builtin_bit_cast(mxg_u16x2, v.x & 0x7FFF7FFFu);
  const mxg_u16x2 b = __builtin_bit_cast(mxg_u16x2, v.y & 0x7FFF7FFFu);
  const mxg_u16x2 c = __builtin_bit_cast(mxg_u16x2, v.z & 0x7FFF7FFFu);
  const mxg_u16x2 d = __builtin_bit_cast(mxg_u16x2, v.w & 0x7FFF7FFFu);
  const mxg_u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                                __builtin_elementwise_max(c, d));
  return max((uint32_t)m.x, (uint32_t)m.y);
}

// Maximum over the 4 lanes of a quad (lanes 4i .. 4i+3); all lanes active.
__device__ __forceinline__ uint32_t quad_max(uint32_t a) {
  // quad_perm [1,0,3,2] then [2,3,0,1]: the partner at lane ^ 1, then ^ 2.
  a = max(a, (uint32_t)__builtin_amdgcn_mov_dpp((int)a, 0xB1, 0xF, 0xF, true));
  a = max(a, (uint32_t)__builtin_amdgcn_mov_dpp((int)a, 0x4E, 0xF, 0xF, true));
  return a;
}

// Block exponent e from the block's largest magnitude pattern: for a normal
// amax = (128 + f) 2^(E - 134), amax <= 448 2^e = 7 2^(6 + e) holds first at
// e = E - 135 when f <= 96 (1 + f/128 <= 1.75) and at e = E - 134 otherwise.
// Subnormal and zero maxima clamp to -127. Returns the scale byte.
__device__ __forceinline__ uint32_t block_scale_byte(uint32_t amax) {
  const int E = (int)(amax >> 7);
  const int f = (int)(amax & 0x7Fu);
  if (E == 0xFF) return 0xFFu;  // infinite or NaN block
  int e = E - 135 + (f > 96 ? 1 : 0);
  e = e < -127 ? -127 : e;      // largest finite: E = 254 -> e <= 120
  return (uint32_t)(e + 127);
}

// Four codes (value order, one per byte) of the BF16 values in words p, q,
// scaled by inv = 2^-e.
__device__ __forceinline__ uint32_t codes4(uint32_t p, uint32_t q, float inv) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(p << 16) * inv,
                                          __uint_as_float(p & 0xFFFF0000u) * inv, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(q << 16) * inv,
                                      __uint_as_float(q & 0xFFFF0000u) * inv, r, true);
  return (uint32_t)r;
}

// 0x7F with the sign of each of the four BF16 values in words p, q.
__device__ __forceinline__ uint32_t nan_codes4(uint32_t p, uint32_t q) {
  return 0x7F7F7F7Fu | ((p >> 8) & 0x80u) | ((p >> 16) & 0x8000u) | ((q << 8) & 0x800000u) |
         (q & 0x80000000u);
}

// The 8 codes of a chunk as two little-endian words (value order).
__device__ __forceinline__ uint2 chunk_codes(const uint4 v, uint32_t sb) {
  // 2^-e, e = sb - 127 in [-127, 120] for a finite block: biased exponent
  // 254 - sb in [7, 254].
  const float inv = __uint_as_float((254u - sb) << 23);
  uint2 r;
  if (sb == 0xFFu) {
    r.x = nan_codes4(v.x, v.y);
    r.y = nan_codes4(v.z, v.w);
  } else {
    r.x = codes4(v.x, v.y, inv);
    r.y = codes4(v.z, v.w, inv);
  }
  return r;
}

}  // namespace mxg
