// Stand-alone MXFP8 activation quantizer (gfx950): [rows, K] BF16 ->
// [rows, K] e4m3fn codes and [rows, K/32] E8M0 scales, the rule and lane
// layout of quant_device.h. The GEMM quantizes in its activation stage
// instead; this kernel is the unfused form of the same step.

#include <hip/hip_runtime.h>

#include "../../include/mxgemm.h"
#include "mxgemm_internal.h"
#include "quant_device.h"

namespace mxg {
namespace {

constexpr int kThreads = 256;

// One lane per 16-byte chunk of 8 values, grid-stride. The loop bound is
// uniform across the workgroup so that every lane takes part in the quad
// exchange; lanes past the end re-read the last chunk and store nothing
// (chunks is a multiple of 4, so a quad is wholly inside or outside).
__global__ void quantize_kernel(const uint16_t* x, int64_t chunks, uint8_t* xq, uint8_t* xs) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t base = (int64_t)blockIdx.x * blockDim.x; base < chunks; base += stride) {
    const int64_t c = base + threadIdx.x;
    const int64_t cc = c < chunks ? c : chunks - 1;
    const uint4 v = *reinterpret_cast<const uint4*>(x + 8 * cc);
    const uint32_t sb = block_scale_byte(quad_max(chunk_amax(v)));
    const uint2 codes = chunk_codes(v, sb);
    if (c < chunks) {
      *reinterpret_cast<uint2*>(xq + 8 * c) = codes;
      if ((c & 3) == 0) xs[c >> 2] = (uint8_t)sb;
    }
  }
}

}  // namespace

hipError_t launch_quantize(const uint16_t* x, int rows, int k, uint8_t* xq, uint8_t* xs,
                           hipStream_t s) {
  const int64_t chunks = (int64_t)rows * (k / 8);
  int64_t blocks = (chunks + kThreads - 1) / kThreads;
  blocks = blocks < 1 ? 1 : (blocks > 4096 ? 4096 : blocks);
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, x, chunks,
                     xq, xs);
  return hipGetLastError();
}

}  // namespace mxg
