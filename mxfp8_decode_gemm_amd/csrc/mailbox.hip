// Mailbox kernels for gfx950: arm, unfused publish, the collects (rank-major
// copy, all-reduce) and the fused all-gather of the three-generation Lamport
// mailbox.
//
// all_gather page = the API page of
// vllm.models.deepseek_v41.nvidia.ops.cute_dsl.all_gather. Its module
// docstring (steps 1-3) and _AllGatherKernel.kernel define the protocol this
// file implements for emulated rank slots on one GPU:
//   * idle words hold the sentinel 0x80000000;
//   * a publish writes a rank's payload into its slot of a generation (here
//     with BF16 negative zero cleared, which also keeps the sentinel word out
//     of every payload): the owner's slot in generation NEXT, an emulated
//     peer's slot in that peer's own counter PEER_GEN[r];
//   * a collect polls each 16-byte pack of every rank's slot until none of
//     its words is the sentinel, copies it out rank-major (or sums it), and
//     stores the sentinel back; it takes the generation from ACTIVE, which
//     the owner's publish set (publishing_gemm page, "Ordering"), and sets
//     NEXT to the next one mod 3;
//   * the fused all-gather reads NEXT itself, and the last of its workgroups
//     to arrive advances it.
// The all-gather moves arbitrary 32-bit words (same module docstring, step
// 1): a word equal to the sentinel goes out as 0, every other word
// unchanged. All payload traffic moves as 32-bit integers, never through
// float registers (sync page, Mailbox.put_words: a NaN bit pattern would not
// survive a float move).

#include <hip/hip_runtime.h>

#include "../../include/mxgemm.h"
#include "mxgemm_internal.h"

namespace mxg {
namespace {

constexpr int kThreads = 256;
constexpr unsigned kMaxBlocks = 2048;

__device__ __forceinline__ uint32_t ld_agent_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_agent_u64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t clear_negative_zero(uint32_t w) {
  const uint32_t lo = (w & 0xFFFFu) == 0x8000u ? 0u : (w & 0xFFFFu);
  const uint32_t hi = (w >> 16) == 0x8000u ? 0u : (w & 0xFFFF0000u);
  return lo | hi;
}

__device__ __forceinline__ uint32_t clear_sentinel_word(uint32_t w) {
  return w == MXG_SENTINEL ? 0u : w;
}

__device__ __forceinline__ uint4 sanitize_pack(uint4 v, bool words) {
  if (words) {
    v.x = clear_sentinel_word(v.x);
    v.y = clear_sentinel_word(v.y);
    v.z = clear_sentinel_word(v.z);
    v.w = clear_sentinel_word(v.w);
  } else {
    v.x = clear_negative_zero(v.x);
    v.y = clear_negative_zero(v.y);
    v.z = clear_negative_zero(v.z);
    v.w = clear_negative_zero(v.w);
  }
  return v;
}

__global__ void fill_u32_kernel(uint32_t* p, size_t words, uint32_t value) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t quads = words / 4;
  uint4* q = reinterpret_cast<uint4*>(p);
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < quads; i += stride)
    q[i] = uint4{value, value, value, value};
  for (size_t i = quads * 4 + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += stride)
    p[i] = value;
}

__global__ void state_init_kernel(uint32_t* state) {
  const int i = threadIdx.x;
  if (i < MXG_STATE_WORDS) state[i] = 0u;
}

__global__ void workspace_header_kernel(uint32_t* hdr) {
  const int i = threadIdx.x;
  if (i < MXG_WS_HEADER_BYTES / 4) hdr[i] = i == MXG_WS_EPOCH ? 1u : 0u;
}

// Unfused publish: one thread per 16-byte pack. kWords selects the word
// rule (sentinel words become 0) over the BF16 rule (negative zero cleared).
// peer < 0 publishes the owner's slot in generation NEXT and sets ACTIVE; a
// peer slot publishes in its own generation PEER_GEN[peer], which the last
// workgroup to arrive advances at its end (the same hand-off as the collect:
// every workgroup counts itself only after its generation load returned).
template <bool kWords>
__global__ void publish_kernel(uint8_t* slot, int64_t gen_stride, uint32_t* state, int peer,
                               const uint8_t* src, int64_t packs) {
  uint32_t* gen_word = peer < 0 ? state + MXG_STATE_NEXT : state + MXG_STATE_PEER_GEN + peer;
  const uint32_t graw = ld_agent_u32(gen_word);
  const uint32_t gen = graw % MXG_GENERATIONS;
  uint32_t arrived = 0;
  if (peer >= 0 && threadIdx.x == 0)
    arrived = __hip_atomic_fetch_add(state + MXG_STATE_PEER_ARR + peer,
                                     1u + (graw == 0xFFFFFFFFu ? 1u : 0u), __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
  uint4* dst = reinterpret_cast<uint4*>(slot + (size_t)gen * gen_stride);
  const uint4* s = reinterpret_cast<const uint4*>(src);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < packs; p += stride)
    dst[p] = sanitize_pack(s[p], kWords);
  if (peer < 0) {
    if (blockIdx.x == 0 && threadIdx.x == 0) st_agent_u32(state + MXG_STATE_ACTIVE, gen);
  } else if (threadIdx.x == 0 && arrived == gridDim.x - 1u) {
    st_agent_u32(state + MXG_STATE_PEER_ARR + peer, 0u);
    st_agent_u32(gen_word, (gen + 1u) % MXG_GENERATIONS);
  }
}

// Collect: one thread per (rank, pack), grid-stride. Every thread loads the
// generation word together with its first pack in all three generations, so
// when the payload is already there (the usual case) the collect costs one
// round trip.
//
// The consumer of a publish takes the generation from state[ACTIVE], which
// the owner's publish set before this kernel started (publishing_gemm page,
// module docstring, "Ordering": the consumer reads stage_state[1] after the
// producer completed), and sets state[NEXT] = generation + 1 mod 3. No
// workgroup of this launch reads NEXT, so one store suffices and no
// workgroup waits for the others: a count of arriving workgroups on one word
// was measured to cost 0.6 us (28 workgroups) to 3 us (256).
//
// kGather is the fused all-gather, which has no producer before it: it reads
// the generation from NEXT, and since its own workgroups read that word, the
// last one to arrive advances it (all_gather page, step 3): each workgroup
// counts itself once after its generation load has returned (the count's
// operand depends on the loaded word), so no workgroup of the launch can read
// the advanced value. It also fuses the caller's own publish
// (all_gather page, _AllGatherKernel, module docstring steps 1 and 2): an
// item of rank `self` stores its pack of `src`, sentinel words sent as 0,
// into its own slot of the generation with device-scope stores, then polls
// that slot like every other rank's, its own included, copies it out and
// resets it. On one GPU the poll returns the thread's own store; with peers
// on other GPUs the same wait is what the page's own-slot poll is for, that
// the rank's own copy has landed before it is read back.
template <bool kGather>
__global__ void collect_kernel(uint8_t* slots, int64_t gen_stride, int64_t capacity, int ranks,
                               uint32_t* state, uint8_t* out, int64_t nbytes,
                               uint32_t spin_limit, const uint8_t* src, int self) {
  const int64_t packs = nbytes / MXG_PACK_BYTES;
  const int64_t total = packs * ranks;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t graw = ld_agent_u32(state + (kGather ? MXG_STATE_NEXT : MXG_STATE_ACTIVE));
  uint64_t lo0 = 0, hi0 = 0, lo1 = 0, hi1 = 0, lo2 = 0, hi2 = 0;
  if (i0 < total && !(kGather && i0 / packs == self)) {
    const int64_t r = i0 / packs;
    const uint64_t* s0 = reinterpret_cast<const uint64_t*>(
        slots + r * capacity + (i0 - r * packs) * MXG_PACK_BYTES);
    const int64_t gs = gen_stride / 8;
    lo0 = ld_agent_u64(s0);
    hi0 = ld_agent_u64(s0 + 1);
    lo1 = ld_agent_u64(s0 + gs);
    hi1 = ld_agent_u64(s0 + gs + 1);
    lo2 = ld_agent_u64(s0 + 2 * gs);
    hi2 = ld_agent_u64(s0 + 2 * gs + 1);
  }
  const uint32_t gen = graw % MXG_GENERATIONS;
  uint32_t arrived = 0;
  if (kGather && threadIdx.x == 0)
    arrived = __hip_atomic_fetch_add(state + MXG_STATE_COLLECT_ARR,
                                     1u + (graw == 0xFFFFFFFFu ? 1u : 0u), __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
  uint8_t* base = slots + (size_t)gen * gen_stride;
  bool timed_out = false;
  for (int64_t i = i0; i < total; i += stride) {
    const int64_t r = i / packs;
    const int64_t p = i - r * packs;
    uint64_t* slot = reinterpret_cast<uint64_t*>(base + r * capacity + p * MXG_PACK_BYTES);
    uint64_t lo, hi;
    if (kGather && r == self) {
      const uint4 v = sanitize_pack(*reinterpret_cast<const uint4*>(src + p * MXG_PACK_BYTES), true);
      st_agent_u64(slot, (uint64_t)v.x | ((uint64_t)v.y << 32));
      st_agent_u64(slot + 1, (uint64_t)v.z | ((uint64_t)v.w << 32));
      lo = ld_agent_u64(slot);
      hi = ld_agent_u64(slot + 1);
    } else if (i == i0) {
      lo = gen == 0 ? lo0 : (gen == 1 ? lo1 : lo2);
      hi = gen == 0 ? hi0 : (gen == 1 ? hi1 : hi2);
    } else {
      lo = ld_agent_u64(slot);
      hi = ld_agent_u64(slot + 1);
    }
    uint32_t polls = 0;
    for (;;) {
      const bool dirty = (uint32_t)lo == MXG_SENTINEL || (uint32_t)(lo >> 32) == MXG_SENTINEL ||
                         (uint32_t)hi == MXG_SENTINEL || (uint32_t)(hi >> 32) == MXG_SENTINEL;
      if (!dirty) break;
      if (++polls >= spin_limit) {
        timed_out = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      lo = ld_agent_u64(slot);
      hi = ld_agent_u64(slot + 1);
    }
    uint4 v;
    v.x = (uint32_t)lo;
    v.y = (uint32_t)(lo >> 32);
    v.z = (uint32_t)hi;
    v.w = (uint32_t)(hi >> 32);
    *reinterpret_cast<uint4*>(out + r * nbytes + p * MXG_PACK_BYTES) = v;
    *reinterpret_cast<uint4*>(slot) =
        uint4{MXG_SENTINEL, MXG_SENTINEL, MXG_SENTINEL, MXG_SENTINEL};
  }
  if (timed_out)
    __hip_atomic_fetch_or(state + MXG_STATE_ERROR, MXG_ERR_COLLECT_SPIN, __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_AGENT);
  if (kGather) {
    if (threadIdx.x == 0 && arrived == gridDim.x - 1u) {
      st_agent_u32(state + MXG_STATE_COLLECT_ARR, 0u);
      st_agent_u32(state + MXG_STATE_NEXT, (gen + 1u) % MXG_GENERATIONS);
    }
  } else if (blockIdx.x == 0 && threadIdx.x == 0) {
    st_agent_u32(state + MXG_STATE_NEXT, (gen + 1u) % MXG_GENERATIONS);
  }
}

// All-reduce collect: one thread per pack p < nbytes/16. Each rank's pack of
// generation g is polled until none of its words is the sentinel (all
// ranks' first loads issued together with the generation word), its eight
// BF16 values are added in FP32 in ascending rank order, the sums are rounded
// once to BF16 (nearest even) into out + 16 p, and every rank's pack is reset
// to the sentinel. Generation hand-off (from ACTIVE, NEXT set by one store)
// and timeout as in collect_kernel.
__global__ void collect_sum_kernel(uint8_t* slots, int64_t gen_stride, int64_t capacity,
                                   int ranks, uint32_t* state, uint8_t* out, int64_t nbytes,
                                   uint32_t spin_limit) {
  const int64_t packs = nbytes / MXG_PACK_BYTES;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const uint32_t gen = ld_agent_u32(state + MXG_STATE_ACTIVE) % MXG_GENERATIONS;
  uint8_t* base = slots + (size_t)gen * gen_stride;
  bool timed_out = false;
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < packs; p += stride) {
    uint64_t lo[MXG_MAX_RANKS], hi[MXG_MAX_RANKS];
#pragma unroll
    for (int r = 0; r < MXG_MAX_RANKS; ++r) {
      if (r < ranks) {
        const uint64_t* s = reinterpret_cast<const uint64_t*>(base + r * capacity + p * MXG_PACK_BYTES);
        lo[r] = ld_agent_u64(s);
        hi[r] = ld_agent_u64(s + 1);
      }
    }
    float acc[8];
#pragma unroll
    for (int r = 0; r < MXG_MAX_RANKS; ++r) {
      if (r >= ranks) continue;
      const uint64_t* s = reinterpret_cast<const uint64_t*>(base + r * capacity + p * MXG_PACK_BYTES);
      uint32_t polls = 0;
      for (;;) {
        const bool dirty =
            (uint32_t)lo[r] == MXG_SENTINEL || (uint32_t)(lo[r] >> 32) == MXG_SENTINEL ||
            (uint32_t)hi[r] == MXG_SENTINEL || (uint32_t)(hi[r] >> 32) == MXG_SENTINEL;
        if (!dirty) break;
        if (++polls >= spin_limit) {
          timed_out = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        lo[r] = ld_agent_u64(s);
        hi[r] = ld_agent_u64(s + 1);
      }
      const uint32_t w[4] = {(uint32_t)lo[r], (uint32_t)(lo[r] >> 32), (uint32_t)hi[r],
                             (uint32_t)(hi[r] >> 32)};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t half = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        const float v = __uint_as_float(half << 16);  // BF16 -> FP32 is exact
        acc[e] = r == 0 ? v : acc[e] + v;
      }
    }
    uint4 o;
    uint32_t* ow = reinterpret_cast<uint32_t*>(&o);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const __bf16 a = (__bf16)acc[2 * q];
      const __bf16 b = (__bf16)acc[2 * q + 1];
      ow[q] = (uint32_t)__builtin_bit_cast(uint16_t, a) |
              ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
    }
    *reinterpret_cast<uint4*>(out + p * MXG_PACK_BYTES) = o;
    for (int r = 0; r < ranks; ++r)
      *reinterpret_cast<uint4*>(base + r * capacity + p * MXG_PACK_BYTES) =
          uint4{MXG_SENTINEL, MXG_SENTINEL, MXG_SENTINEL, MXG_SENTINEL};
  }
  if (timed_out)
    __hip_atomic_fetch_or(state + MXG_STATE_ERROR, MXG_ERR_COLLECT_SPIN, __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_AGENT);
  if (blockIdx.x == 0 && threadIdx.x == 0)
    st_agent_u32(state + MXG_STATE_NEXT, (gen + 1u) % MXG_GENERATIONS);
}

unsigned blocks_for(int64_t items) {
  const int64_t b = (items + kThreads - 1) / kThreads;
  return (unsigned)(b < 1 ? 1 : (b > (int64_t)kMaxBlocks ? kMaxBlocks : b));
}

}  // namespace

hipError_t launch_fill_u32(uint32_t* p, size_t words, uint32_t value, hipStream_t s) {
  hipLaunchKernelGGL(fill_u32_kernel, dim3(blocks_for((int64_t)(words / 4 + 1))), dim3(kThreads),
                     0, s, p, words, value);
  return hipGetLastError();
}

hipError_t launch_state_init(uint32_t* state, hipStream_t s) {
  hipLaunchKernelGGL(state_init_kernel, dim3(1), dim3(64), 0, s, state);
  return hipGetLastError();
}

hipError_t launch_workspace_init(uint32_t* ws, size_t bytes, hipStream_t s) {
  const size_t words = bytes / 4;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(blocks_for((int64_t)(words / 4 + 1))), dim3(kThreads),
                     0, s, ws, words, 0u);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(workspace_header_kernel, dim3(1), dim3(64), 0, s, ws);
  return hipGetLastError();
}

hipError_t launch_mailbox_publish(uint8_t* slot, int64_t gen_stride, uint32_t* state,
                                  int peer, const uint8_t* src, int64_t nbytes, bool words,
                                  hipStream_t s) {
  const int64_t packs = nbytes / MXG_PACK_BYTES;
  if (words)
    hipLaunchKernelGGL(publish_kernel<true>, dim3(blocks_for(packs)), dim3(kThreads), 0, s,
                       slot, gen_stride, state, peer, src, packs);
  else
    hipLaunchKernelGGL(publish_kernel<false>, dim3(blocks_for(packs)), dim3(kThreads), 0, s,
                       slot, gen_stride, state, peer, src, packs);
  return hipGetLastError();
}

hipError_t launch_mailbox_collect(uint8_t* slots, int64_t gen_stride, int64_t capacity,
                                  int ranks, uint32_t* state, uint8_t* out, int64_t nbytes,
                                  uint32_t spin_limit, hipStream_t s) {
  const int64_t items = nbytes / MXG_PACK_BYTES * ranks;
  hipLaunchKernelGGL(collect_kernel<false>, dim3(blocks_for(items)), dim3(kThreads), 0, s,
                     slots, gen_stride, capacity, ranks, state, out, nbytes, spin_limit,
                     (const uint8_t*)nullptr, -1);
  return hipGetLastError();
}

hipError_t launch_mailbox_all_gather(uint8_t* slots, int64_t gen_stride, int64_t capacity,
                                     int ranks, int self, uint32_t* state, const uint8_t* src,
                                     uint8_t* out, int64_t nbytes, uint32_t spin_limit,
                                     hipStream_t s) {
  const int64_t items = nbytes / MXG_PACK_BYTES * ranks;
  hipLaunchKernelGGL(collect_kernel<true>, dim3(blocks_for(items)), dim3(kThreads), 0, s,
                     slots, gen_stride, capacity, ranks, state, out, nbytes, spin_limit, src,
                     self);
  return hipGetLastError();
}

hipError_t launch_mailbox_collect_sum(uint8_t* slots, int64_t gen_stride, int64_t capacity,
                                      int ranks, uint32_t* state, uint8_t* out, int64_t nbytes,
                                      uint32_t spin_limit, hipStream_t s) {
  const int64_t packs = nbytes / MXG_PACK_BYTES;
  hipLaunchKernelGGL(collect_sum_kernel, dim3(blocks_for(packs)), dim3(kThreads), 0, s, slots,
                     gen_stride, capacity, ranks, state, out, nbytes, spin_limit);
  return hipGetLastError();
}

}  // namespace mxg
