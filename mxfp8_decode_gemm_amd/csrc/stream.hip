// Plain HBM read stream (gfx950), the measurement context for the GEMM's
// roofline: how fast this device reads a buffer of a given size with no
// other work. Each workgroup reads one 32 KiB chunk with nontemporal 16-byte
// loads, eight per thread in flight, and stores the XOR of the chunk's
// 32-bit words (a checksum, so the loads cannot be dropped).

#include <hip/hip_runtime.h>

#include "../../include/mxgemm.h"
#include "mxgemm_internal.h"

namespace mxg {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr size_t kChunk16 = MXG_STREAM_CHUNK_BYTES / 16;

typedef unsigned v4u __attribute__((ext_vector_type(4)));

// Chunk blockIdx.x covers 16-byte words [blockIdx.x * kChunk16, +kChunk16),
// cut at total16; lanes past the end load nothing.
__global__ void __launch_bounds__(kThreads)
    stream_read_kernel(const v4u* src, size_t total16, uint32_t* sink) {
  __shared__ uint32_t part[kThreads / 64];
  const size_t base = (size_t)blockIdx.x * kChunk16;
  uint32_t acc = 0;
  for (size_t r = 0; r < kChunk16; r += (size_t)kThreads * kUnroll) {
    v4u v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + r + (size_t)u * kThreads + threadIdx.x;
      v[u] = i < total16 ? __builtin_nontemporal_load(src + i) : v4u{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // XOR over the workgroup: the wave by shuffles, then the waves in LDS.
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
    for (int w = 0; w < kThreads / 64; ++w) x ^= part[w];
    sink[blockIdx.x] = x;
  }
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s) {
  const size_t total16 = bytes / 16;
  const size_t grid = (bytes + MXG_STREAM_CHUNK_BYTES - 1) / MXG_STREAM_CHUNK_BYTES;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s,
                     static_cast<const v4u*>(src), total16, sink);
  return hipGetLastError();
}

}  // namespace mxg
