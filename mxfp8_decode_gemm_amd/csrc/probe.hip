// Measurement aid: the block-scaled MFMA that the pages' design names
// (gfx950's v_mfma_scale_f32_16x16x128_f8f6f4 on e4m3 with E8M0 scales per
// 32 K), beside the arithmetic this library's GEMM uses instead (each e4m3
// code times its scale converted to an exact BF16 value, then
// v_mfma_f32_16x16x32_bf16), on the same 16 x K and K x 16 operands. Both
// accumulate in FP32 in ascending K. It exists so that the numerical reason
// for not using the scaled instruction can be checked on the device from
// committed inputs.
//
// Operand layout of both instructions as this library measured it on gfx950
// (the packed W layout of mxgemm_pack_weight is the same): in each 128-wide
// K step, lane l holds row (or column) l % 16 and the 32 bytes at K
// 16 (l / 16) + 0..15 and 64 + 16 (l / 16) + 0..15; for the scaled MFMA
// lane l's scale byte covers row (or column) l % 16 and the 32-wide K block
// l / 16. The 16 x 16 result: lane l holds rows 4 (l / 16) + 0..3 of column
// l % 16.

#include <hip/hip_runtime.h>

#include "../../include/mxgemm.h"
#include "mxgemm_internal.h"

namespace mxg {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float e8m0_f32(uint32_t s) {
  return __builtin_amdgcn_ldexpf(__uint_as_float(0x00400000u), (int)s);  // 2^-127 * 2^s
}

__device__ __forceinline__ v8bf cvt8(uint32_t w0, uint32_t w1, float scale) {
  const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, false);
  const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, true);
  const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, false);
  const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, true);
  return v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// One wave. a, b: [16][k] e4m3 (row-major, K contiguous); as, bs: [16][k/32]
// E8M0; c: [16][16] FP32, c[row * 16 + col] = sum_k A[row][k] B[col][k] with
// the scales applied. scaled: the block-scaled fp8 MFMA, else BF16.
__global__ void __launch_bounds__(64)
    mfma_probe_kernel(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                      int k, int scaled, float* c) {
  const int lane = threadIdx.x;
  const int r = lane & 15, g = lane >> 4;
  const int kb32 = k >> 5;
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < k; k0 += 128) {
    const uint4 alo = *reinterpret_cast<const uint4*>(a + (size_t)r * k + k0 + 16 * g);
    const uint4 ahi = *reinterpret_cast<const uint4*>(a + (size_t)r * k + k0 + 64 + 16 * g);
    const uint4 blo = *reinterpret_cast<const uint4*>(b + (size_t)r * k + k0 + 16 * g);
    const uint4 bhi = *reinterpret_cast<const uint4*>(b + (size_t)r * k + k0 + 64 + 16 * g);
    if (scaled) {
      const v8i av = {(int)alo.x, (int)alo.y, (int)alo.z, (int)alo.w,
                      (int)ahi.x, (int)ahi.y, (int)ahi.z, (int)ahi.w};
      const v8i bv = {(int)blo.x, (int)blo.y, (int)blo.z, (int)blo.w,
                      (int)bhi.x, (int)bhi.y, (int)bhi.z, (int)bhi.w};
      const int sa = as[(size_t)r * kb32 + (k0 >> 5) + g];
      const int sb = bs[(size_t)r * kb32 + (k0 >> 5) + g];
      // Formats 0 and 0: e4m3 for both operands; the scale in byte 0.
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 0, 0, sa, 0, sb);
    } else {
      // This library's main loop: lane group g's 16-byte pieces lie in the
      // 32-wide blocks g / 2 and 2 + g / 2 of the step.
      const float fa0 = e8m0_f32(as[(size_t)r * kb32 + (k0 >> 5) + (g >> 1)]);
      const float fa1 = e8m0_f32(as[(size_t)r * kb32 + (k0 >> 5) + 2 + (g >> 1)]);
      const float fb0 = e8m0_f32(bs[(size_t)r * kb32 + (k0 >> 5) + (g >> 1)]);
      const float fb1 = e8m0_f32(bs[(size_t)r * kb32 + (k0 >> 5) + 2 + (g >> 1)]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cvt8(alo.x, alo.y, fa0), cvt8(blo.x, blo.y, fb0),
                                                    acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cvt8(alo.z, alo.w, fa0), cvt8(blo.z, blo.w, fb0),
                                                    acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cvt8(ahi.x, ahi.y, fa1), cvt8(bhi.x, bhi.y, fb1),
                                                    acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cvt8(ahi.z, ahi.w, fa1), cvt8(bhi.z, bhi.w, fb1),
                                                    acc, 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) c[(4 * g + i) * 16 + r] = acc[i];
}

}  // namespace

hipError_t launch_mfma_probe(const uint8_t* a, const uint8_t* as, const uint8_t* b,
                             const uint8_t* bs, int k, int scaled, float* c, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(1), dim3(64), 0, s, a, as, b, bs, k, scaled, c);
  return hipGetLastError();
}

}  // namespace mxg
