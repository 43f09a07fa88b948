// Plain HBM read streams (gfx950), the measurement context for the GEMM's
// roofline: how fast this device reads a buffer of a given size with no
// other work, and how that rate depends on the way the read is organised.
//
// stream_read_kernel (mxg_stream_read): each workgroup reads one 32 KiB
// chunk with nontemporal 16-byte loads, eight per thread in flight, and
// stores the XOR of the chunk's 32-bit words (a checksum, so the loads
// cannot be dropped).
//
// stream_cfg_kernel (mxg_stream_read_cfg): the same read with the knobs a
// streaming kernel chooses: threads per workgroup, 16-byte loads per thread
// in flight, the load instruction (global or raw buffer into registers, or
// global straight into LDS) and cache policy (nontemporal or default), and
// how the bytes are split over workgroups
// (one 32 KiB chunk each; a fixed grid with one contiguous range each, as
// the GEMM splits W; or a fixed grid taking 32 KiB chunks round-robin).
// Each workgroup stores the XOR of every 32-bit word it read.

#include <hip/hip_runtime.h>

#include "../../include/mxgemm.h"
#include "mxgemm_internal.h"

namespace mxg {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr size_t kChunk16 = MXG_STREAM_CHUNK_BYTES / 16;
constexpr int kBufferWord3 = 0x00020000;
constexpr int kNontemporal = 2;

typedef unsigned v4u __attribute__((ext_vector_type(4)));

// XOR of a workgroup's values into sink[blockIdx.x]: the wave by shuffles,
// then the waves in LDS.
template <int THREADS>
__device__ __forceinline__ void wg_xor_store(uint32_t acc, uint32_t* sink) {
  __shared__ uint32_t part[THREADS / 64];
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
    for (int w = 0; w < THREADS / 64; ++w) x ^= part[w];
    sink[blockIdx.x] = x;
  }
}

// Chunk blockIdx.x covers 16-byte words [blockIdx.x * kChunk16, +kChunk16),
// cut at total16; lanes past the end load nothing.
__global__ void __launch_bounds__(kThreads)
    stream_read_kernel(const v4u* src, size_t total16, uint32_t* sink) {
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
  wg_xor_store<kThreads>(acc, sink);
}

// One round of UNROLL 16-byte loads per thread at words w0 + u * THREADS +
// tid (u < UNROLL), words at or past `end` read as zero. KIND 0: global,
// nontemporal; 1: global, default policy; 2: raw buffer, nontemporal; 3: raw
// buffer, default policy (the buffer spans the whole source; a word past
// its end reads zero without a memory access); 4: global to LDS directly
// (global_load_lds_dwordx4, nontemporal: the data lands in the wave's LDS
// region, lane l's 16 bytes at l * 16, without passing through registers),
// then read back from LDS by the lane that loaded it.
template <int THREADS, int UNROLL, int KIND>
__device__ __forceinline__ uint32_t read_round(const v4u* src, __amdgpu_buffer_rsrc_t rs,
                                               size_t w0, size_t end, v4u* lds_wave) {
  v4u v[UNROLL];
  if constexpr (KIND == 4) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      // Lanes past the end load the last word again (w0 < end, so it
      // exists) and drop it on the read-back: no branch around the load.
      const size_t i = w0 + (size_t)u * THREADS + threadIdx.x;
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(src + (i < end ? i : end - 1)),
          (__attribute__((address_space(3))) void*)(lds_wave + u * 64), 16, 0, kNontemporal);
    }
    // Every load of the round has landed in LDS (vmcnt 0; lgkm and exp
    // counters left alone).
    __builtin_amdgcn_s_waitcnt(0x0F70);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const size_t i = w0 + (size_t)u * THREADS + threadIdx.x;
      v[u] = i < end ? lds_wave[u * 64 + lane] : v4u{0u, 0u, 0u, 0u};
    }
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    return acc;
  }
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const size_t i = w0 + (size_t)u * THREADS + threadIdx.x;
    if constexpr (KIND == 2 || KIND == 3) {
      // Offsets stay below 2^31 bytes (checked on the host); past the end a
      // zero-returning offset.
      const int off = i < end ? (int)(i * 16) : 0x7FFFFFF0;
      v[u] = __builtin_bit_cast(
          v4u, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, KIND == 2 ? kNontemporal : 0));
    } else if constexpr (KIND == 0) {
      v[u] = i < end ? __builtin_nontemporal_load(src + i) : v4u{0u, 0u, 0u, 0u};
    } else {
      v[u] = i < end ? src[i] : v4u{0u, 0u, 0u, 0u};
    }
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  return acc;
}

// interleave 0: workgroup g reads the contiguous words [g * per_wg, (g + 1) *
// per_wg); interleave 1: it reads the 32 KiB chunks g, g + G, g + 2 G, ... (G the
// grid size). Either way cut at total16.
template <int THREADS, int UNROLL, int KIND>
__global__ void __launch_bounds__(THREADS)
    stream_cfg_kernel(const v4u* src, size_t total16, size_t per_wg16, int interleave,
                      uint32_t* sink) {
  // KIND 4: each wave's LDS region of UNROLL x 64 16-byte slots.
  extern __shared__ v4u lds_dyn[];
  v4u* lds_wave = lds_dyn + (size_t)(threadIdx.x >> 6) * UNROLL * 64;
  // The whole source as one raw buffer (the host keeps it below 2^31 bytes
  // for the buffer kinds; the global kinds do not use it).
  const size_t nbytes = total16 * 16 < 0x7FFFFFF0u ? total16 * 16 : 0x7FFFFFF0u;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, (int)nbytes, kBufferWord3);
  constexpr size_t kRound = (size_t)THREADS * UNROLL;
  uint32_t acc = 0;
  if (!interleave) {
    const size_t lo = (size_t)blockIdx.x * per_wg16;
    const size_t hi = lo + per_wg16 < total16 ? lo + per_wg16 : total16;
    for (size_t w = lo; w < hi; w += kRound) acc ^= read_round<THREADS, UNROLL, KIND>(src, rs, w, hi, lds_wave);
  } else {
    const size_t chunks = (total16 + kChunk16 - 1) / kChunk16;
    for (size_t c = blockIdx.x; c < chunks; c += gridDim.x) {
      const size_t lo = c * kChunk16;
      const size_t hi = lo + kChunk16 < total16 ? lo + kChunk16 : total16;
      for (size_t w = lo; w < hi; w += kRound)
        acc ^= read_round<THREADS, UNROLL, KIND>(src, rs, w, hi, lds_wave);
    }
  }
  wg_xor_store<THREADS>(acc, sink);
}

template <int THREADS, int UNROLL>
const void* cfg_kernel(int kind) {
  switch (kind) {
    case 0: return reinterpret_cast<const void*>(&stream_cfg_kernel<THREADS, UNROLL, 0>);
    case 1: return reinterpret_cast<const void*>(&stream_cfg_kernel<THREADS, UNROLL, 1>);
    case 2: return reinterpret_cast<const void*>(&stream_cfg_kernel<THREADS, UNROLL, 2>);
    case 3: return reinterpret_cast<const void*>(&stream_cfg_kernel<THREADS, UNROLL, 3>);
    default: return reinterpret_cast<const void*>(&stream_cfg_kernel<THREADS, UNROLL, 4>);
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

hipError_t launch_stream_read_cfg(const void* src, size_t bytes, uint32_t* sink, int workgroups,
                                  int threads, int unroll, int kind, int interleave,
                                  hipStream_t s) {
  const size_t total16 = bytes / 16;
  size_t grid = workgroups > 0 ? (size_t)workgroups
                               : (bytes + MXG_STREAM_CHUNK_BYTES - 1) / MXG_STREAM_CHUNK_BYTES;
  const size_t per_wg16 = workgroups > 0 ? (total16 + grid - 1) / grid : kChunk16;
  const void* fn = nullptr;
  if (threads == 256) {
    fn = unroll == 4 ? cfg_kernel<256, 4>(kind)
                     : (unroll == 8 ? cfg_kernel<256, 8>(kind) : cfg_kernel<256, 16>(kind));
  } else {
    fn = unroll == 4 ? cfg_kernel<512, 4>(kind)
                     : (unroll == 8 ? cfg_kernel<512, 8>(kind) : cfg_kernel<512, 16>(kind));
  }
  const size_t lds = kind == 4 ? (size_t)threads * unroll * 16 : 0;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const v4u* srcv = static_cast<const v4u*>(src);
  void* args[] = {&srcv, const_cast<size_t*>(&total16), const_cast<size_t*>(&per_wg16),
                  &interleave, &sink};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(threads), args, lds, s);
}

}  // namespace mxg
