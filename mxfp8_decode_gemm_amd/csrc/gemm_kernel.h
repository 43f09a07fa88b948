// The low-batch MXFP8 GEMM with the Lamport publish in its epilogue, for
// gfx950 (MI355X).
//
// What it computes (publishing_gemm page = the API page of
// vllm.models.deepseek_v41.nvidia.specialized_decode.boundary.publishing_gemm;
// module docstring, "GEMM structure", and epilog_warp / publish_value):
//   C[t, n] = sum_k W[n, k] x[t, k] over e4m3fn data with one E8M0 scale per
//   32 K, FP32 accumulation, split-K over `split_k` workgroups that exchange
//   FP32 partials and each reduce a share of the tile, then BF16 rounding,
//   negative-zero clearing and one 16-byte store per eight consecutive
//   columns of one token into the mailbox slot of generation state[NEXT].
//
// How it is laid out on CDNA4 (not the pages' Blackwell design):
//   * Numerics. W is the MFMA A operand (16 output rows per instruction), x
//     the B operand (16 token columns; columns >= m repeat token 0 and are
//     never read, so no lane branches on its token). Each e4m3 byte
//     is turned, with its E8M0 scale, into the exact BF16 value
//     dec(byte) * 2^(scale-127) by v_cvt_scalef32_pk_bf16_fp8, and the
//     contraction runs on v_mfma_f32_16x16x32_bf16 with FP32 accumulation.
//     gfx950's scaled fp8 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4) was
//     measured on the device to drop the low bits of every product smaller
//     than about 2^-13 of the largest product in its 32-element scale block,
//     a biased truncation that grows with K and breaks the 1 BF16 ulp +
//     1e-6 sum|W x| acceptance bound; the BF16 instruction keeps products to
//     about 2^-25 of the largest in its 32-element K step. The path is HBM
//     bound, so the 4x MFMA count and the conversions cost well under a tenth
//     of the kernel's time.
//   * W never touches LDS: it is re-laid once (mxgemm_pack_weight) into 2 KiB
//     tiles of 16 rows x 128 K, so that each wave instruction reads 1 KiB of
//     contiguous HBM straight into VGPRs, `depth` K blocks ahead, as a raw
//     buffer load whose block offset is a scalar (no vector address math). Lane l holds
//     row l % 16 and K = 16*(l/16) + 0..15 and 64 + 16*(l/16) + 0..15 of the
//     block; the BF16 MFMA pairs A and B elements by lane group and position
//     (measured), so the B operand uses the same K split.
//   * x and its scales for the workgroup's K slice are staged once in LDS, in
//     the order the B operand reads them, and shared by every wave; their
//     loads go out before the W prologue and are waited for after it, or
//     after its first DX slots on the tiles that issue the rest later (XR
//     sets how many chunks each thread loads in that first round). With BF16 x
//     (QX) the stage quantizes it to e4m3 codes and E8M0 scales on the way
//     (quant_device.h). Variants built with X16 store the slice as its
//     exact BF16 values instead (each chunk converted with its scale byte on
//     the way into LDS), so the waves read the B operand without converting
//     it; the chooser takes them when the 2 m k_slice bytes fit.
//   * A workgroup's worker waves split its rows (WN) and its K slice (WK);
//     their partial tiles meet in LDS and are summed in ascending K order.
//   * Split-K across workgroups: in every token row of a tile, slice s owns
//     the contiguous pack columns [ceil(s P / S), ceil((s + 1) P / S)) (P packs
//     per row). The other slices store their partials of those columns as
//     (FP32 bits, epoch) 64-bit pairs with agent-scope stores, spread over
//     every worker wave; the owner's poll waves poll all of a column's pairs
//     in one batch until every tag equals this launch's epoch
//     (sync page = vllm.models.deepseek_v41.amd.mono.common.sync, Mailbox: one
//     round trip, no drain, no flag), then sum the slices in ascending K order.
//   * One lane per owned column rounds its sum to BF16; lane shuffles gather
//     eight consecutive columns of one token into one lane, which writes one
//     aligned 16-byte pack (and the raw pack to c_out when asked).
//   * With split-K a control wave runs beside the workers: it reads the
//     generation and the epoch, stores the epoch into this workgroup's word,
//     and in workgroup 0 stores the next epoch once every word holds the
//     current one, so no worker waits on those round trips.
//   * Without a mailbox (state null) the kernel is the plain GEMM into c_out,
//     the first half of the unfused publish path.
//
// This header holds the kernel template and its device helpers; each
// gemm_variants_*.hip file instantiates a share of the variant table (so the
// shares compile in parallel), and gemm_publish.hip holds the host side.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/mxgemm.h"
#include "mxgemm_internal.h"
#include "quant_device.h"

namespace mxg {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// 2^(s-127) as an FP32 multiplier: the biased exponent s in the exponent
// field; s == 0 is the subnormal 2^-127.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  // 2^-127 (an FP32 subnormal, kept: the library is built with FP32
  // denormals on) times 2^s, one instruction; s = 255 gives +inf.
  return __builtin_amdgcn_ldexpf(__uint_as_float(0x00400000u), (int)s);
}

// Eight e4m3fn bytes (two dwords, lowest byte first) times a power-of-two
// scale, as eight BF16 values. v_cvt_scalef32_pk_bf16_fp8 converts two bytes
// of a dword per instruction; an e4m3 value times 2^k is exact in BF16 for
// every scale the workloads use, and the instruction rounds to nearest even.
__device__ __forceinline__ v8bf fp8x8_to_bf16(uint32_t w0, uint32_t w1, float scale) {
  const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, false);
  const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, true);
  const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, false);
  const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, true);
  return v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// LDS header: [0] generation, [1] epoch, [2] the workspace's error word as
// read at the call's start, [4 + w] worker wave w's range flags (bit 0: an x
// scale byte of its staging outside the exact range, bit 1: a W scale byte
// of its rows outside it). 16 worker waves at most.
constexpr int kHeaderBytes = 80;
constexpr int kHdrFlags = 4;

// The E8M0 range in which e4m3 * 2^(s-127) is exact in BF16 for every code:
// an e4m3 value is a multiple of 2^-9, so after scaling a multiple of
// 2^(s-136), which BF16's smallest step 2^-133 divides for s >= 3; the
// largest, 448 * 2^(s-127) = 1.75 * 2^(s-119), stays below BF16's largest
// finite 1.9921875 * 2^127 for s <= 246. Inside this range the main loop
// converts each operand with its scale. A W row block whose scale bytes
// leave the range but span at most kScaleHi - kScaleLo binades stays in the
// main loop with all its scales moved into the range by one shift, undone
// on its partial sums after the loop. A workgroup that meets any other
// scale byte outside the range (an x scale byte, or a W row block spanning
// more) takes the exact path (products of the codes, each 32-wide block's
// sum scaled by 2^(sW + sX - 254) in FP32).
constexpr uint32_t kScaleLo = 3;
constexpr uint32_t kScaleHi = 246;

__device__ __forceinline__ bool scale_byte_out(uint32_t s) {
  return s < kScaleLo || s > kScaleHi;
}
__device__ __forceinline__ bool scale_word_out(uint32_t w) {
  return scale_byte_out(w & 0xFFu) || scale_byte_out((w >> 8) & 0xFFu) ||
         scale_byte_out((w >> 16) & 0xFFu) || scale_byte_out(w >> 24);
}

// Raw buffer descriptors (gfx9 family): the fourth word of a plain byte
// buffer, an offset no descriptor here reaches (1 GiB; offsets at or past a
// buffer's size read as zeros), and the cache policy of a streaming load.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kPastBuffer = 0x40000000;
constexpr int kLoadNontemporal = 2;

// A word that nothing writes while the kernel runs, read at a wave-uniform
// address through the constant address space: a scalar load, counted apart
// from the vector loads of the W stream, so a wait for it never waits for
// the stream (the dispatch's acquire makes earlier launches' stores visible).
__device__ __forceinline__ uint32_t ld_uniform_u32(const uint32_t* p) {
  return *(const __attribute__((address_space(4))) uint32_t*)(p);
}
// Lane i takes lane i + N of its 16-lane row (0 where that lies past the
// row): a DPP move on the vector unit instead of an LDS permute.
template <int N>
__device__ __forceinline__ uint32_t row_down(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x100 + N, 0xF, 0xF, true);
}
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

// BF16 bits of an FP32 value, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  const __bf16 a = (__bf16)lo;
  const __bf16 b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Each BF16 half equal to 0x8000 (negative zero) becomes 0x0000.
__device__ __forceinline__ uint32_t clear_negative_zero(uint32_t w) {
  const uint32_t lo = (w & 0xFFFFu) == 0x8000u ? 0u : (w & 0xFFFFu);
  const uint32_t hi = (w >> 16) == 0x8000u ? 0u : (w & 0xFFFF0000u);
  return lo | hi;
}

// Token row of index c in a slice of rows of d items each (c < 8 d: an
// activation has at most 8 rows): seven compares against multiples of the
// wave-uniform d instead of an integer division.
__device__ __forceinline__ int row_of(int c, int d) {
  int t = 0;
#pragma unroll
  for (int j = 1; j < 8; ++j) t += c >= j * d ? 1 : 0;
  return t;
}

// Copies x chunks (16 bytes) of the workgroup's K slice into LDS in the order
// the MFMA B operand reads them: chunk (kb, half, group, t) holds
// x[t][kb*128 + 64*half + 16*group .. +16).
// XR scales the round: 4 * XR chunks per thread, all loaded up front.
// X16: each chunk is stored as its sixteen exact BF16 values instead (two
// 16-byte pieces, dest16), converted with the scale byte loaded beside it.
template <int NT, int XR = 1, bool X16 = false>
struct XStage {
  static constexpr int kChunks = 4 * XR;  // chunks per thread per round
  static constexpr int kWords = 2;        // scale words per thread per round
  uint4 v[kChunks];
  int d[kChunks];
  uint32_t sc[X16 ? kChunks : 1];  // X16: the scale byte of each chunk
  uint32_t s0, s1;
  int e0, e1;

  __device__ __forceinline__ static int dest(int c, int cpr, int m) {
    const int t = row_of(c, cpr);
    const int q = c - t * cpr;
    const int kb = q >> 3, w8 = q & 7;
    return ((kb * 2 + (w8 >> 2)) * 4 + (w8 & 3)) * m + t;
  }
  // X16: the first of the two BF16 pieces of chunk c (the second is 4 m
  // further): piece ((kb * 4 + 2h + part) * 4 + grp) * m + t holds the eight
  // values MFMA step 2h + part of lane group grp reads in K block kb.
  __device__ __forceinline__ static int dest16(int c, int cpr, int m) {
    const int t = row_of(c, cpr);
    const int q = c - t * cpr;
    const int kb = q >> 3, w8 = q & 7;
    return ((kb * 4 + 2 * (w8 >> 2)) * 4 + (w8 & 3)) * m + t;
  }
  __device__ __forceinline__ static uint4 src(const uint8_t* x, int K, size_t k0, int c, int cpr) {
    const int t = row_of(c, cpr);
    const int q = c - t * cpr;
    return *reinterpret_cast<const uint4*>(x + (size_t)t * K + k0 + 16 * q);
  }
  // Loads are issued for every thread (an index past the slice re-reads the
  // last chunk), so each wave issues the same number of loads and the
  // compiler can wait for exactly these, not for the W loads issued later.
  __device__ __forceinline__ void load(const uint8_t* x, int K, size_t k0, int cpr, int xch,
                                       int c0, int tid) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = c0 + i * NT + tid;
      v[i] = src(x, K, k0, c < xch ? c : xch - 1, cpr);
    }
  }
  // The LDS places of the chunks (-1 past the slice): computed after the
  // loads are issued, so that the W prologue goes out right after them.
  __device__ __forceinline__ void dests(int m, int cpr, int xch, int c0, int tid) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = c0 + i * NT + tid;
      d[i] = c < xch ? (X16 ? dest16(c, cpr, m) : dest(c, cpr, m)) : -1;
    }
  }
  // X16: the E8M0 byte of each chunk's 32-value block (two chunks per block).
  __device__ __forceinline__ void load_chunk_scales(const uint8_t* xs, int K, size_t k0, int cpr,
                                                    int xch, int c0, int tid) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      int c = c0 + i * NT + tid;
      c = c < xch ? c : xch - 1;
      const int t = row_of(c, cpr);
      const int q = c - t * cpr;
      sc[i] = xs[(size_t)t * (K >> 5) + (k0 >> 5) + (q >> 1)];
    }
  }
  // Scale words: x_scale row t, word q of the slice -> LDS word t * wpr + q.
  __device__ __forceinline__ void load_scales(const uint8_t* xs, int K, size_t k0, int wpr,
                                              int nw, int c0, int tid) {
    const int c_0 = c0 + tid, c_1 = c0 + NT + tid;
    const int u0 = c_0 < nw ? c_0 : nw - 1, u1 = c_1 < nw ? c_1 : nw - 1;
    const int t0 = row_of(u0, wpr), t1 = row_of(u1, wpr);
    s0 = *reinterpret_cast<const uint32_t*>(xs + (size_t)t0 * (K >> 5) + (k0 >> 5) +
                                            4 * (u0 - t0 * wpr));
    s1 = *reinterpret_cast<const uint32_t*>(xs + (size_t)t1 * (K >> 5) + (k0 >> 5) +
                                            4 * (u1 - t1 * wpr));
    e0 = c_0 < nw ? c_0 : -1;
    e1 = c_1 < nw ? c_1 : -1;
  }
  __device__ __forceinline__ void store_scales(uint32_t* xsw) const {
    if (e0 >= 0) xsw[e0] = s0;
    if (e1 >= 0) xsw[e1] = s1;
  }
  // X16: keeps the scale conversion where it is called. Without it the
  // compiler decodes the scale bytes right after their loads, and so waits
  // for them before the W prologue is issued.
  __device__ __forceinline__ void pin_scales() {
    if constexpr (X16) {
#pragma unroll
      for (int i = 0; i < kChunks; ++i) asm volatile("" : "+v"(sc[i]));
    }
  }
  // Whether a scale byte this thread staged lies outside the exact range
  // (call after store: the scales are then already waited for).
  __device__ __forceinline__ bool scales_out() const {
    bool out = false;
    if constexpr (X16) {
      // A chunk of zero codes contributes zeros at any scale. The codes are
      // looked at only when some scale byte of the wave is out of range.
      bool sout = false;
#pragma unroll
      for (int i = 0; i < kChunks; ++i) sout |= d[i] >= 0 && scale_byte_out(sc[i]);
      if (__any(sout)) {
#pragma unroll
        for (int i = 0; i < kChunks; ++i)
          out |= d[i] >= 0 && scale_byte_out(sc[i]) &&
                 ((v[i].x | v[i].y | v[i].z | v[i].w) & 0x7F7F7F7Fu) != 0;
      }
    } else {
      out = (e0 >= 0 && scale_word_out(s0)) || (e1 >= 0 && scale_word_out(s1));
    }
    return out;
  }
  // FP8 chunks as they are, or (X16) as two pieces of exact BF16 values.
  __device__ __forceinline__ void store(uint4* xl, int m) const {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      if (d[i] < 0) continue;
      if constexpr (X16) {
        const float fs = e8m0_to_f32(sc[i]);
        xl[d[i]] = __builtin_bit_cast(uint4, fp8x8_to_bf16(v[i].x, v[i].y, fs));
        xl[d[i] + 4 * m] = __builtin_bit_cast(uint4, fp8x8_to_bf16(v[i].z, v[i].w, fs));
      } else {
        xl[d[i]] = v[i];
      }
    }
  }
};


// Quantizing activation stage: BF16 x of the workgroup's K slice becomes
// e4m3 codes and E8M0 scales in LDS, in the layout XStage writes (the codes
// of 16-value chunk (t, q) at XStage::dest, scale byte (t, b) at t*KS/32 + b).
// Each thread loads 16-byte chunks of 8 BF16 values; chunk c of the slice
// is row t = c / cpr8, values 8q .. 8q+7 with q = c % cpr8, so the 4 chunks
// of a 32-value block are 4 consecutive lanes (cpr8 and the round size are
// multiples of 4). Indices past the slice re-read the last chunk and are
// not stored; whole blocks lie on either side of that bound. A wave whose
// chunks of a round all lie past the slice skips them (loads and
// arithmetic); the test is on the wave's first chunk, so it is uniform. With
// q_out the codes and scales also go to [m, K] and [m, K/32] in global
// memory. X16: LDS gets the codes' exact BF16 values (XStage::dest16 pieces)
// instead of codes and scales.
template <int NT, bool X16 = false>
struct XQuant {
  static constexpr int kChunks = 8;  // chunks per thread per round
  uint4 v[kChunks];

  __device__ __forceinline__ void load(const uint16_t* xb, int K, size_t k0, int cpr8,
                                       int xch8, int c0, int tid) {
    const int wbase = tid & ~63;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      if (c0 + i * NT + wbase >= xch8) break;
      int c = c0 + i * NT + tid;
      c = c < xch8 ? c : xch8 - 1;
      const int t = row_of(c, cpr8);
      const int q = c - t * cpr8;
      v[i] = *reinterpret_cast<const uint4*>(xb + (size_t)t * K + k0 + 8 * q);
    }
  }
  // Returns whether a scale byte of this thread's chunks lies outside the
  // exact range.
  __device__ __forceinline__ bool store(uint8_t* xlb, uint8_t* xsl, int K, size_t k0, int m,
                                        int cpr8, int xch8, int c0, int tid, uint8_t* q_out,
                                        uint8_t* s_out) const {
    const int cpr = cpr8 >> 1;
    const int kspw = cpr8 >> 2;
    const int wbase = tid & ~63;
    bool out = false;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      if (c0 + i * NT + wbase >= xch8) break;
      const int c = c0 + i * NT + tid;
      const uint32_t sb = block_scale_byte(quad_max(chunk_amax(v[i])));
      const uint2 codes = chunk_codes(v[i], sb);
      if (c < xch8) {
        // Codes quantized from BF16 values times their scale are multiples
        // of 2^-133 (the grid of a BF16 input is never finer than e4m3's
        // at its magnitude) with 4 significant bits: BF16 values, except
        // where a code of 256 at scale byte 247 makes 2^128. Only the top
        // end of the range leaves BF16 here.
        out |= sb > kScaleHi;
        const int t = row_of(c, cpr8);
        const int q = c - t * cpr8;
        if constexpr (X16) {
          // The codes' exact BF16 values: one piece (see XStage::dest16).
          const int d = XStage<NT, 1, true>::dest16(t * cpr + (q >> 1), cpr, m) + 4 * m * (q & 1);
          reinterpret_cast<uint4*>(xlb)[d] =
              __builtin_bit_cast(uint4, fp8x8_to_bf16(codes.x, codes.y, e8m0_to_f32(sb)));
        } else {
          const int d = XStage<NT>::dest(t * cpr + (q >> 1), cpr, m);
          *reinterpret_cast<uint2*>(xlb + (size_t)d * 16 + 8 * (q & 1)) = codes;
          if ((q & 3) == 0) xsl[t * kspw + (q >> 2)] = (uint8_t)sb;
        }
        if (q_out) {
          *reinterpret_cast<uint2*>(q_out + (size_t)t * K + k0 + 8 * q) = codes;
          if ((q & 3) == 0) s_out[(size_t)t * (K >> 5) + (k0 >> 5) + (q >> 2)] = (uint8_t)sb;
        }
      }
    }
    return out;
  }
};

// The quantizing rounds from chunk c_first on (past the first round, see
// stage_rest; from 0 to re-stage the slice as FP8 for the exact path).
// Returns whether a scale byte lies outside the exact range.
template <int NT, bool X16>
__device__ __attribute__((noinline)) bool quant_rest(const uint16_t* xb, int K, size_t k0, int m,
                                                     int cpr8, int xch8, int tid, uint8_t* xlb,
                                                     uint8_t* xsl, uint8_t* q_out,
                                                     uint8_t* s_out, int c_first) {
  XQuant<NT, X16> st;
  bool out = false;
  for (int c0 = c_first; c0 < xch8; c0 += XQuant<NT>::kChunks * NT) {
    st.load(xb, K, k0, cpr8, xch8, c0, tid);
    out |= st.store(xlb, xsl, K, k0, m, cpr8, xch8, c0, tid, q_out, s_out);
  }
  return out;
}

// The rounds of x staging from chunk c_first and scale word w_first on:
// past the first round for slices larger than one (kept out of line: its
// loads would otherwise make the compiler wait for every W load in flight
// before the main loop of the common one-round case), or the whole slice as
// FP8 for the exact path. Returns whether a scale byte lies outside the
// exact range.
template <int NT, int XR, bool X16>
__device__ __attribute__((noinline)) bool stage_rest(const uint8_t* x, const uint8_t* xs, int K,
                                                     size_t k0, int m, int cpr, int xch, int wpr,
                                                     int nsw, int tid, uint4* xl, uint32_t* xsw,
                                                     int c_first, int w_first) {
  XStage<NT, XR, X16> st;
  bool out = false;
  for (int c0 = c_first; c0 < xch; c0 += XStage<NT, XR>::kChunks * NT) {
    st.load(x, K, k0, cpr, xch, c0, tid);
    if constexpr (X16) st.load_chunk_scales(xs, K, k0, cpr, xch, c0, tid);
    st.dests(m, cpr, xch, c0, tid);
    st.store(xl, m);
    if constexpr (X16) out |= st.scales_out();
  }
  if constexpr (X16) return out;  // the scales went into the BF16 values
  for (int c0 = w_first; c0 < nsw; c0 += XStage<NT, XR>::kWords * NT) {
    st.load_scales(xs, K, k0, wpr, nsw, c0, tid);
    st.store_scales(xsw);
    out |= st.scales_out();
  }
  return out;
}

// At least two waves per SIMD (<= 256 VGPRs): with split-K the grid must be
// resident at once, and a second wave hides the other's conversion work.
// With split-K one more wave, the control wave, runs beside the WN x WK
// worker waves and does the call's bookkeeping while they stream: it reads
// the generation and epoch, stores the epoch into this workgroup's word, and
// in workgroup 0 advances the epoch once every workgroup has read it. No
// worker wave waits for these round trips (loads and stores complete in
// order per wave, so one in flight would hold the worker's W loads).
// QX: x arrives as BF16 (a.xb) and is quantized in the activation stage.
// XR: MXFP8 x staged in rounds of 4 * XR chunks per thread (the first round's
// loads all go out before the W prologue).
// X16: the staged slice holds exact BF16 values (XStage::dest16 layout), not
// FP8 codes and scale bytes, and the main loop reads the B operand as is.
// Without a mailbox (a.state null) the kernel is a plain GEMM into c_out.
template <int RB, int WN, int WK, int D, int SK, bool QX, int XR = 1, bool X16 = false>
__global__ void __launch_bounds__(64 * (WN * WK + (SK > 1 ? 1 : 0)))
    __attribute__((amdgpu_waves_per_eu(2))) gemm_publish_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int NT = 64 * WN * WK;  // worker threads
  constexpr int RBT = RB * WN;    // 16-row blocks per tile
  constexpr int NTILE = 16 * RBT; // rows per tile

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Wave-uniform in a scalar register, so the W stream's base addresses and
  // the per-block selects stay on the scalar unit.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool ctl = SK > 1 && wave >= NT / 64;  // the control wave (split-K only)
  const int hand_tid = SK > 1 ? NT : 0; // reads the hand-off words
  const int wn = wave % WN;
  const int wk = wave / WN;
  const int r16 = lane & 15;  // A row / B column of this lane
  const int grp = lane >> 4;  // lane group: K pieces and scale block

  constexpr int S = SK;  // split-K slices (the launch's split_k)
  // Workgroups are handed to the 8 XCDs round-robin by index. When the
  // tiles divide evenly, the S slices of a tile get indices 8 apart, so they
  // run on one XCD and their pair exchange stays within its L2. Placement
  // only affects speed: the exchange is correct for any placement.
  int tile, slice;
  if (S > 1 && a.xcd_groups) {
    const int b = blockIdx.x, q = b >> 3;
    slice = q % S;
    tile = (q / S) * 8 + (b & 7);
  } else {
    tile = blockIdx.x / S;
    slice = blockIdx.x - tile * S;
  }
  const int m = a.m, N = a.n, K = a.k;
  const int KS = K / S;             // K slice of this workgroup
  const int NB = KS >> 7;           // 128-wide K blocks in the slice
  const int kb_lo = (wk * NB) / WK; // this wave's K blocks
  const int kb_hi = ((wk + 1) * NB) / WK;
  const int nbw = ctl ? 0 : kb_hi - kb_lo;  // the control wave streams nothing
  const int row0 = tile * NTILE;
  const size_t kslice0 = (size_t)slice * KS;

  uint32_t* hdr = reinterpret_cast<uint32_t*>(lds);
  uint4* xl = reinterpret_cast<uint4*>(lds + kHeaderBytes);
  uint8_t* xsl = lds + kHeaderBytes + (size_t)m * KS;

  // ---- call hand-off: generation and epoch ------------------------------
  // Read once per workgroup, before it counts itself (all_gather page,
  // _AllGatherKernel.kernel: the last CTA to arrive advances the state).
  // Without split-K every worker reads the generation with a scalar load
  // (nothing writes it during the call) and one thread stores it to LDS
  // after its x staging. With
  // split-K the control wave reads the generation, the epoch and the
  // workspace's error word (once a split-K poll has given up, its pairs can
  // no longer be told from this call's, so no later call publishes until
  // the workspace is armed again), stores them to LDS and stores its epoch
  // word, all before the first barrier: a load still in flight where the
  // control wave's path joins the workers' would make the workers wait for
  // their whole W prologue at the first register they reuse.
  uint32_t gen = 0, epoch = 0;
  if (S == 1 && a.state) gen = ld_uniform_u32(a.state + MXG_STATE_NEXT) % MXG_GENERATIONS;
  if (S > 1 && tid == hand_tid) {
    if (a.state) gen = ld_agent_u32(a.state + MXG_STATE_NEXT) % MXG_GENERATIONS;
    epoch = ld_agent_u32(a.ws_hdr + MXG_WS_EPOCH) + a.epoch_bias;
    const uint32_t wserr = ld_agent_u32(a.ws_hdr + MXG_WS_ERROR);
    hdr[0] = gen;
    hdr[1] = epoch;
    hdr[2] = wserr;
    // This workgroup has read the epoch (the stored word is the value
    // read, so the store is issued after the load returned).
    st_agent_u32(a.flags + blockIdx.x, epoch);
  }

  // ---- W scale range of this wave's rows --------------------------------
  // mxgemm_pack_weight leaves one word per 16-row block after the tiles: the
  // smallest and largest scale byte (bits 0-7, 8-15) of the block's 32-wide
  // blocks that hold a nonzero code (0xFF and 0 when none does: a block of
  // zero codes contributes zeros at any scale). Loaded first in the worker
  // region below, before the x loads, so waiting for x covers it.
  const int KBT = K >> 7;         // K blocks per row block
  const int rbn = (N + 15) >> 4;  // packed row blocks
  const uint32_t* wsum = reinterpret_cast<const uint32_t*>(a.ws + (size_t)rbn * KBT * 64);
  uint32_t wrange[RB];
  int wshift[RB];  // the scale shift of each row block (0 inside the exact range)
#pragma unroll
  for (int i = 0; i < RB; ++i) wshift[i] = 0;

  // ---- x slice, first round: loads issued before the W stream -----------
  const int cpr = KS >> 4;  // 16-byte chunks per x row in the slice
  const int xch = m * cpr;
  const int wpr = KS >> 7;  // x-scale words per token row in the slice
  const int nsw = m * wpr;
  const int cpr8 = KS >> 3;  // 8-value BF16 chunks per x row (quantizing stage)
  const int xch8 = m * cpr8;
  XStage<NT, XR, X16> xst;
  XQuant<NT, X16> xqs;
  bool xout = false;  // an x scale byte this thread stages lies outside the exact range

  // ---- W stream prologue (packed tiles, see mxgemm_pack_weight) ---------
  // Tile (rb, kb) is 2048 contiguous bytes: lane l's K pieces at 16 l and
  // 1024 + 16 l; its scales are 16 rows x 4 bytes. A wave streams the
  // contiguous tiles kb0 .. kb0 + nbw - 1 of each of its row blocks.
  const int kb0 = slice * NB + kb_lo;         // first absolute K block of this wave
  // Each of the wave's row blocks is read as a raw buffer over its nbw
  // contiguous tiles (scales: 64 bytes per tile), so the block offset goes
  // in a scalar register and the lane's offset stays fixed: no per-load
  // vector address arithmetic. Rows past N load the last row block (never
  // published).
  __amdgpu_buffer_rsrc_t wrs[RB], srs[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    int rb = (row0 >> 4) + wn * RB + i;
    rb = rb < rbn ? rb : rbn - 1;
    const size_t t0 = (size_t)rb * KBT + kb0;
    wrs[i] = __builtin_amdgcn_make_buffer_rsrc((void*)(a.w + t0 * 2048), (short)0, nbw * 2048,
                                               kBufferWord3);
    srs[i] = __builtin_amdgcn_make_buffer_rsrc((void*)(a.ws + t0 * 64), (short)0, nbw * 64,
                                               kBufferWord3);
  }
  v4u wlo[D][RB], whi[D][RB];
  uint32_t wsc[D][RB];
  // Block j of this wave (lane l's pieces at 16 l and 1024 + 16 l, its
  // scale word at 4 (l % 16)), or (j < 0) a dummy whose offset lies past the
  // buffer: the hardware returns zeros without a memory access. Every refill
  // slot issues its loads either way, so the count of loads in flight is the
  // same on every path.
  auto load_w = [&](int d, int j) __attribute__((always_inline)) {
    const int vo = j >= 0 ? 16 * lane : kPastBuffer;
    const int so = j >= 0 ? 4 * r16 : kPastBuffer;
    const int jo = j >= 0 ? j : 0;
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      wlo[d][i] = __builtin_amdgcn_raw_buffer_load_b128(wrs[i], vo, jo * 2048, kLoadNontemporal);
      whi[d][i] = __builtin_amdgcn_raw_buffer_load_b128(wrs[i], vo + 1024, jo * 2048,
                                                         kLoadNontemporal);
      wsc[d][i] = __builtin_amdgcn_raw_buffer_load_b32(srs[i], so, jo * 64, 0);
    }
  };
  constexpr int G = D > 16 ? D : 16;  // K blocks per straight-line group
  // Ring slots issued before the x stage (the rest follow it).
  constexpr int DX = SK == 1 ? (WN * WK >= 8 ? 1 : D) : (D > 3 && (QX || WN * WK <= 4) ? 3 : D);
  const int ng0 = nbw < G ? nbw : G;
  if (!ctl) {
    // The range words, x, then the W prologue, in one worker-only region: a
    // load left in flight where the control wave's path joins would have
    // the workers wait for their W prologue at the first register that load
    // wrote.
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int rb = (row0 >> 4) + wn * RB + i;
      wrange[i] = wsum[rb < rbn ? rb : rbn - 1];
    }
    if constexpr (QX) {
      xqs.load(a.xb, K, kslice0, cpr8, xch8, 0, tid);
    } else {
      xst.load(a.x, K, kslice0, cpr, xch, 0, tid);
      if constexpr (X16)
        xst.load_chunk_scales(a.xs, K, kslice0, cpr, xch, 0, tid);
      else
        xst.load_scales(a.xs, K, kslice0, wpr, nsw, 0, tid);
    }
    // The ring in slot order (the scheduler would otherwise reorder the
    // loads, and the in-order completion count would then make the first
    // steps wait for the last slots). Some tiles issue only DX slots here
    // and the rest after the x stage, so that x lands sooner; the W stream
    // still has slots in flight meanwhile. Interleaved A/B:
    //  * split-K, BF16 x and tiles of at most four worker waves, 3 slots:
    //    BF16 x N=7168/K=8192/m=8/S=4 15.5 -> 15.0 us, N=2048/K=8192/m=8/S=4
    //    10.5 -> 10.3 us; MXFP8 x on the 4-wave tile of N=2048/K=8192/m=8/S=4
    //    7.40 -> 7.08 us (mean of 9). The 7-wave tile of N=7168/K=8192/m=8/S=4
    //    and N=7168/K=4096/m=1/S=4 was level or 0.1 us slower;
    //  * without split-K, tiles of 8 or more waves (a whole-K x stage), 1
    //    slot: N=4096/K=16384 m=4 16.0 -> 15.3 us, m=8 17.2 -> 16.6 us, m=1
    //    and m=2 level (2 slots: bimodal, often slower); the 4-wave tile of
    //    N=7168/K=2048/m=4 was level or slower and keeps all its slots.
#pragma unroll
    for (int d = 0; d < DX; ++d) {
      load_w(d, d < ng0 ? d : -1);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- x and its scales into LDS -------------------------------------
    // The x loads were issued first, so waiting for them leaves the W
    // prologue in flight: the W stream starts at once and x lands in one
    // round trip.
    if constexpr (QX) {
      // The workgroups of tile 0 (one per K slice) also write the quantized
      // activation out when asked.
      uint8_t* qo = tile == 0 ? a.xq_out : nullptr;
      uint8_t* so = tile == 0 ? a.xs_out : nullptr;
      uint8_t* xlb = reinterpret_cast<uint8_t*>(xl);
      xout = xqs.store(xlb, xsl, K, kslice0, m, cpr8, xch8, 0, tid, qo, so);
      if (xch8 > XQuant<NT>::kChunks * NT)
        xout |= quant_rest<NT, X16>(a.xb, K, kslice0, m, cpr8, xch8, tid, xlb, xsl, qo, so,
                                    XQuant<NT>::kChunks * NT);
#pragma unroll
      for (int d = DX; d < D; ++d) {
        load_w(d, d < ng0 ? d : -1);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      uint32_t* xsw = reinterpret_cast<uint32_t*>(xsl);
      xst.dests(m, cpr, xch, 0, tid);
      xst.pin_scales();
      xst.store(xl, m);
      if constexpr (!X16) xst.store_scales(xsw);
      xout = xst.scales_out();
      if (xch > XStage<NT, XR>::kChunks * NT || (!X16 && nsw > XStage<NT, XR>::kWords * NT))
        xout |= stage_rest<NT, XR, X16>(a.x, a.xs, K, kslice0, m, cpr, xch, wpr, nsw, tid, xl,
                                        xsw, XStage<NT, XR>::kChunks * NT,
                                        XStage<NT, XR>::kWords * NT);
#pragma unroll
      for (int d = DX; d < D; ++d) {
        load_w(d, d < ng0 ? d : -1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // Range flags of this wave. The W summary is pinned here so that its
    // use, and so the wait for it, stays behind the W prologue. A row block
    // whose scale bytes reach outside the exact range but span at most
    // kScaleHi - kScaleLo binades keeps the main loop: its operands are
    // converted with every scale moved by one shift into the range (exact),
    // and its partial sums are scaled back by 2^-shift once, after the loop.
    // Only a wider span sends the workgroup to the exact path.
    bool wout = false;
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      asm volatile("" : "+v"(wrange[i]));
      // The same word in every lane: worked on by the scalar unit.
      wrange[i] = __builtin_amdgcn_readfirstlane(wrange[i]);
      const int lo = (int)(wrange[i] & 0xFFu), hi = (int)((wrange[i] >> 8) & 0xFFu);
      const int sh = lo < (int)kScaleLo ? (int)kScaleLo - lo
                                        : (hi > (int)kScaleHi ? (int)kScaleHi - hi : 0);
      wout |= sh != 0 && hi - lo > (int)(kScaleHi - kScaleLo);
      wshift[i] = sh;
    }
    const uint32_t fl = (__any(xout) ? 1u : 0u) | (wout ? 2u : 0u);
    if (lane == 0) hdr[kHdrFlags + wave] = fl;
  }
  if (S == 1 && tid == hand_tid) {
    hdr[0] = gen;
    hdr[1] = epoch;
    hdr[2] = 0;
  }
  __syncthreads();
  // A workgroup takes the exact path when any of its waves met a scale byte
  // outside the range the operand conversion keeps exact.
  uint32_t rflags = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) rflags |= hdr[kHdrFlags + w];
  const bool exact_path = rflags != 0;

  // ---- control wave: epoch bookkeeping while the workers stream ---------
  if (S > 1 && ctl) {
    if (blockIdx.x == 0) {
      // Every workgroup's word holding this call's epoch means every
      // workgroup has read it: only then may the next epoch be stored.
      const uint32_t e = __shfl(epoch, 0, 64);
      uint32_t polls = 0;
      bool ok = true;
      for (;;) {
        bool pending = false;
        for (int i = lane; i < (int)gridDim.x; i += 64) pending |= ld_agent_u32(a.flags + i) != e;
        if (!__any(pending)) break;
        if (++polls >= a.spin_limit) {
          ok = false;
          if (lane == 0)
            __hip_atomic_fetch_or(a.ws_hdr + MXG_WS_ERROR, MXG_ERR_SPLITK_SPIN, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      if (ok && lane == 0)
        st_agent_u32(a.ws_hdr + MXG_WS_EPOCH, (e + 1u == 0u ? 1u : e + 1u) - a.epoch_bias);
    }
  }

  // ---- exact path: x as FP8 codes in LDS -------------------------------
  // The BF16 stage holds x already scaled, which is not exact out of range:
  // the exact path stages the slice again as codes and scale bytes (the
  // FP8 stage's layout, over the same LDS). Workgroup-uniform branch.
  if constexpr (X16) {
    if (exact_path) {
      if (!ctl) {
        if constexpr (QX)
          quant_rest<NT, false>(a.xb, K, kslice0, m, cpr8, xch8, tid,
                                reinterpret_cast<uint8_t*>(xl), xsl, nullptr, nullptr, 0);
        else
          stage_rest<NT, 1, false>(a.x, a.xs, K, kslice0, m, cpr, xch, wpr, nsw, tid, xl,
                                   reinterpret_cast<uint32_t*>(xsl), 0, 0);
      }
      __syncthreads();
    }
  }

  // ---- main loop: K blocks of this wave ---------------------------------
  v4f acc[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
  // 2^(shift - 127) per row block: ldexp of it by a scale byte is the
  // shifted scale (a normal or subnormal FP32 value for shifts -9 .. 3).
  float wbase[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
    wbase[i] = __builtin_amdgcn_ldexpf(__uint_as_float(0x00400000u), wshift[i]);
  const bool tok = r16 < m;
  const int xrow = tok ? r16 : 0;  // x row this lane's B operand reads
  const uint4* xbp = xl + grp * m + xrow;  // X16: this lane's first BF16 piece
  const int kspw = KS >> 5;  // scale bytes per x row in the slice
  const int sb0 = grp >> 1;  // 32-block of this lane's first 16 K (its second is sb0 + 2)
  auto consume = [&](int d, int j) __attribute__((always_inline)) {
    const int kb = kb_lo + j;  // K block within the slice
    // B operand: x of this lane's token as exact BF16, four K steps.
    // Lanes past the last token convert token 0's values instead: the MFMA
    // columns they feed are never read, and no lane branches.
    v8bf bx[4];
    if constexpr (X16) {
      // Exact BF16 values staged by XStage / XQuant (dest16 layout).
#pragma unroll
      for (int q = 0; q < 4; ++q) bx[q] = __builtin_bit_cast(v8bf, xbp[(kb * 16 + q * 4) * m]);
    } else {
      const uint4 xlo = xl[((kb * 2 + 0) * 4 + grp) * m + xrow];
      const uint4 xhi = xl[((kb * 2 + 1) * 4 + grp) * m + xrow];
      const uint8_t* xsr = xsl + xrow * kspw + kb * 4;
      const float fs0 = e8m0_to_f32(xsr[sb0]);
      const float fs1 = e8m0_to_f32(xsr[sb0 + 2]);
      bx[0] = fp8x8_to_bf16(xlo.x, xlo.y, fs0);
      bx[1] = fp8x8_to_bf16(xlo.z, xlo.w, fs0);
      bx[2] = fp8x8_to_bf16(xhi.x, xhi.y, fs1);
      bx[3] = fp8x8_to_bf16(xhi.z, xhi.w, fs1);
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const float fa0 = __builtin_amdgcn_ldexpf(wbase[i], (int)((wsc[d][i] >> (8 * sb0)) & 0xFFu));
      const float fa1 =
          __builtin_amdgcn_ldexpf(wbase[i], (int)((wsc[d][i] >> (8 * (sb0 + 2))) & 0xFFu));
      const v8bf a0 = fp8x8_to_bf16(wlo[d][i].x, wlo[d][i].y, fa0);
      const v8bf a1 = fp8x8_to_bf16(wlo[d][i].z, wlo[d][i].w, fa0);
      const v8bf a2 = fp8x8_to_bf16(whi[d][i].x, whi[d][i].y, fa1);
      const v8bf a3 = fp8x8_to_bf16(whi[d][i].z, whi[d][i].w, fa1);
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bx[0], acc[i], 0, 0, 0);
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bx[1], acc[i], 0, 0, 0);
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2, bx[2], acc[i], 0, 0, 0);
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a3, bx[3], acc[i], 0, 0, 0);
    }
  };
  // Exact path, one K block: the MFMA runs on the codes themselves (every
  // e4m3 value is a BF16 value) one 32-wide scale block at a time, by
  // zeroing the B operand of the lane groups that hold the other block of
  // the same K step (groups 0-1 hold K 0-31 of a 64-wide half, groups 2-3 K
  // 32-63), and each block's sum is scaled by 2^(sW + sX - 254) with one
  // v_ldexp_f32 (FP32 subnormals kept) before it is added, blocks in
  // ascending K. Lane l's four results are rows 4 (l / 16) + r of the row
  // block and token l % 16; row r's scale word comes from lane 4 (l / 16) + r,
  // which loaded it. The W pieces come from the same ring as consume's.
  auto consume_exact = [&](const v4u (&ewl)[RB], const v4u (&ewh)[RB], const uint32_t (&ews)[RB],
                           int j) __attribute__((always_inline)) {
    const int kb = kb_lo + j;
    const uint4 xlo = xl[((kb * 2 + 0) * 4 + grp) * m + xrow];
    const uint4 xhi = xl[((kb * 2 + 1) * 4 + grp) * m + xrow];
    const uint32_t xsw = *reinterpret_cast<const uint32_t*>(xsl + xrow * kspw + kb * 4);
    const bool lo = grp < 2;
    const v8bf z = {};
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const uint32_t sw = ews[i];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const v4u wv = b < 2 ? ewl[i] : ewh[i];
        const uint4 xv = b < 2 ? xlo : xhi;
        const bool mine = (b & 1) ? !lo : lo;
        const v8bf a0 = fp8x8_to_bf16(wv.x, wv.y, 1.0f);
        const v8bf a1 = fp8x8_to_bf16(wv.z, wv.w, 1.0f);
        const v8bf x0 = fp8x8_to_bf16(xv.x, xv.y, 1.0f);
        const v8bf x1 = fp8x8_to_bf16(xv.z, xv.w, 1.0f);
        v4f t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, mine ? x0 : z, zero, 0, 0, 0);
        t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, mine ? x1 : z, t, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t swr = (uint32_t)__shfl((int)sw, 4 * grp + r, 64);
          const int e = (int)((swr >> (8 * b)) & 0xFFu) + (int)((xsw >> (8 * b)) & 0xFFu) - 254;
          acc[i][r] += __builtin_amdgcn_ldexpf(t[r], e);
        }
      }
    }
  };
  // Straight-line groups of G blocks with a D-deep ring of W registers: step
  // j consumes ring slot j % D and refills it with block j + D of the group
  // (or a dummy), so no register is carried across a loop edge and the wait
  // before each step is for exactly the loads D steps back. The first
  // group's ring was filled above; later groups (more than G blocks per
  // wave) refill it at their start. The exact path runs the same ring.
  auto stream = [&](auto&& step) __attribute__((always_inline)) {
    for (int g0 = 0; g0 < nbw; g0 += G) {
      const int ng = nbw - g0 < G ? nbw - g0 : G;
      if (g0 > 0) {
#pragma unroll
        for (int d = 0; d < D; ++d) load_w(d, d < ng ? g0 + d : -1);
      }
#pragma unroll
      for (int j = 0; j < G; ++j) {
        if (j < ng) step(j % D, g0 + j);
        if (j + D < G) load_w(j % D, j + D < ng ? g0 + j + D : -1);
      }
    }
  };
  if (exact_path) {
    // The prologue's ring is let land and dropped; the exact stream keeps
    // two blocks in flight in registers of its own.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    v4u el[2][RB], eh[2][RB];
    uint32_t es[2][RB];
    auto eload = [&](int d, int j) __attribute__((always_inline)) {
      const int vo = j >= 0 ? 16 * lane : kPastBuffer;
      const int so = j >= 0 ? 4 * r16 : kPastBuffer;
      const int jo = j >= 0 ? j : 0;
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        el[d][i] = __builtin_amdgcn_raw_buffer_load_b128(wrs[i], vo, jo * 2048, kLoadNontemporal);
        eh[d][i] = __builtin_amdgcn_raw_buffer_load_b128(wrs[i], vo + 1024, jo * 2048, kLoadNontemporal);
        es[d][i] = __builtin_amdgcn_raw_buffer_load_b32(srs[i], so, jo * 64, 0);
      }
    };
    eload(0, nbw > 0 ? 0 : -1);
    eload(1, nbw > 1 ? 1 : -1);
    for (int j0 = 0; j0 < nbw; j0 += 2) {
      consume_exact(el[0], eh[0], es[0], j0);
      eload(0, j0 + 2 < nbw ? j0 + 2 : -1);
      if (j0 + 1 < nbw) consume_exact(el[1], eh[1], es[1], j0 + 1);
      eload(1, j0 + 3 < nbw ? j0 + 3 : -1);
    }
    // No load of this path left in flight where it joins the main loop's:
    // the compiler would otherwise make the main loop wait for its own W
    // prologue before reusing those registers.
    __builtin_amdgcn_s_waitcnt(0x0F70);
  } else {
    stream(consume);
    // Undo the row blocks' scale shifts: one rounding, FP32 subnormals kept.
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][r] = __builtin_amdgcn_ldexpf(acc[i][r], -wshift[i]);
  }

  // ---- roles after the main loop ---------------------------------------
  // Each 16-byte pack (8 columns of one token) is reduced by one slice: in
  // every token row of the tile, slice s owns the pack columns
  // jc in [ceil(s * PPR / S), ceil((s + 1) * PPR / S)), a contiguous run.
  // With split-K every worker wave first sends its share of the partials the
  // other slices own; then the first PW waves handle the owned packs (poll,
  // reduce, publish), one lane per column. Loads and stores share one
  // in-order completion counter per wave, so a polling wave's first poll
  // also waits for its own sends; spreading the sends over every wave still
  // ends the send phase sooner than keeping the polling waves out of it
  // (measured). Without split-K every wave publishes.
  constexpr int NW = NT / 64;
  constexpr int PPR = NTILE / 8;  // packs per token row of the tile
  const int jlo = (slice * PPR + SK - 1) / SK;
  const int jhi = ((slice + 1) * PPR + SK - 1) / SK;
  const int cnt = jhi - jlo;           // owned packs per token row
  const int own_items = m * cnt * 8;   // one lane per owned (pack, column)
  int pw = NW;
  if (SK > 1 && NW > 1) {
    pw = (own_items + 63) >> 6;
    pw = pw < 1 ? 1 : (pw > NW - 1 ? NW - 1 : pw);
  }
  const bool poller = wave < pw;
  const bool sender = SK > 1 && !ctl;

  // ---- partial tile -> LDS [wk][t][row], summed over waves in K order ---
  __syncthreads();  // every wave is done with x in LDS
  float* red = reinterpret_cast<float*>(lds + kHeaderBytes);
  if (tok && !ctl) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int rl = (wn * RB + i) * 16 + 4 * grp;
      *reinterpret_cast<v4f*>(red + ((size_t)(wk * m + r16) * NTILE + rl)) = acc[i];
    }
  }
  __syncthreads();
  gen = hdr[0];
  epoch = hdr[1];
  // Set when an earlier call's split-K poll gave up: publish nothing, so the
  // consumer's collect times out and reports it instead of taking values
  // summed from pairs that may be stale.
  const bool ws_failed = hdr[2] != 0;
  uint8_t* slot = a.slot + (size_t)gen * a.gen_stride;
  const size_t ncols = (size_t)(N >> 3);
  // This workgroup's partial of tile row `row` (within the tile), token t.
  auto partial = [&](int t, int row) __attribute__((always_inline)) {
    float v = red[(size_t)t * NTILE + row];
#pragma unroll
    for (int w = 1; w < WK; ++w) v += red[(size_t)(w * m + t) * NTILE + row];
    return v;
  };

  // ---- sends: one (FP32 bits, epoch) pair per lane ----------------------
  // pairs[((slice * 8 + t) * (N / 8) + n / 8) * 8 + n % 8]; lanes take
  // consecutive columns of a token row, so a wave writes whole packs.
  if (sender) {
    const int s0 = tid;
    const int ns = NT;
    for (int q = s0; q < m * NTILE; q += ns) {
      const int t = q / NTILE;
      const int row = q - t * NTILE;
      const int jc = row >> 3;
      if (row0 + row >= N || (jc >= jlo && jc < jhi)) continue;
      st_agent_u64(a.pairs + ((size_t)slice * 8 + t) * ncols * 8 + row0 + row,
                   (uint64_t)__float_as_uint(partial(t, row)) | ((uint64_t)epoch << 32));
    }
  }

  // ---- owned packs: exchange, BF16, publish -----------------------------
  // Lane 8j + e of a wave takes column e of one owned pack; the eight lanes
  // of a pack stay together (every count below is a multiple of 8), so the
  // pack's BF16 values meet in its lane e = 0 for one 16-byte store.
  if (poller) {
    const int e = lane & 7;
    for (int i0 = wave * 64; i0 < own_items; i0 += pw * 64) {
      const int item = i0 + lane;
      const int pk = item >> 3;  // owned pack index: token row t, run position
      const int t = cnt > 0 ? pk / cnt : 0;
      const int jc = jlo + (pk - t * cnt);
      const int row = 8 * jc + e;
      const bool live = item < own_items && row0 + 8 * jc < N;
      float v = live ? partial(t, row) : 0.f;
      bool failed = false;  // this column's poll gave up
      if (SK > 1) {
        // Poll the other slices' pairs of this column in one batch.
        uint64_t pv[SK > 1 ? SK - 1 : 1];
        uint32_t polls = 0;
        for (;;) {
          bool pending = false;
          if (live) {
            // Device-scope loads: a peer's pair may sit in another XCD's
            // L2, and an L2-coherent load is not guaranteed to observe it.
#pragma unroll
            for (int o = 0; o < SK - 1; ++o) {
              const int src = o < slice ? o : o + 1;
              pv[o] = ld_agent_u64(a.pairs + ((size_t)src * 8 + t) * ncols * 8 + row0 + row);
            }
#pragma unroll
            for (int o = 0; o < SK - 1; ++o) pending |= (uint32_t)(pv[o] >> 32) != epoch;
          }
          if (!pending) break;
          if (++polls >= a.spin_limit) {
            __hip_atomic_fetch_or(a.ws_hdr + MXG_WS_ERROR, MXG_ERR_SPLITK_SPIN, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
            failed = true;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        // Sum the slices in ascending K order, this slice's partial in
        // place: pv[o] holds slice o below this slice and o + 1 above it.
        if (live) {
          float r = slice == 0 ? v : __uint_as_float((uint32_t)pv[0]);
#pragma unroll
          for (int o = 1; o < SK; ++o)
            r += o == slice ? v : __uint_as_float((uint32_t)pv[o < slice ? o : o - 1]);
          v = r;
        }
      }
      // BF16 (nearest even) of this column, then the pack's eight halves
      // gathered into lane e = 0: raw store, negative-zero clear, publish.
      const __bf16 hb = (__bf16)v;
      const uint32_t h = (uint32_t)__builtin_bit_cast(uint16_t, hb);
      // (Lane e = 0 of a pack reads lanes 1..7 of its own 8, inside its row.)
      const uint32_t pair = h | (row_down<1>(h) << 16);
      const uint32_t p1 = row_down<2>(pair);
      const uint32_t p2 = row_down<4>(pair);
      const uint32_t p3 = row_down<6>(pair);
      // A pack with a column whose poll gave up is not published.
      uint32_t fp = failed ? 1u : 0u;
      fp |= row_down<1>(fp);
      fp |= row_down<2>(fp);
      fp |= row_down<4>(fp);
      if (live && e == 0 && fp == 0 && !ws_failed) {
        const uint4 raw = {pair, p1, p2, p3};
        const size_t off = ((size_t)t * N + row0 + 8 * jc) * 2;
        if (a.c_out) *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(a.c_out) + off) = raw;
        if (a.slot) {
          uint4 clean;
          clean.x = clear_negative_zero(raw.x);
          clean.y = clear_negative_zero(raw.y);
          clean.z = clear_negative_zero(raw.z);
          clean.w = clear_negative_zero(raw.w);
          *reinterpret_cast<uint4*>(slot + off) = clean;
        }
      }
    }
  }

  // Hand the generation to the consumer once per grid (publishing_gemm page,
  // epilog_warp: block 0, one thread, sets the active stage word).
  if (a.state && blockIdx.x == 0 && tid == hand_tid) st_agent_u32(a.state + MXG_STATE_ACTIVE, gen);
}

}  // namespace

// ---- variant table --------------------------------------------------------
struct Variant {
  TileCfg cfg;
  int split_k;
  const void* fn;      // MXFP8 x
  const void* fn_q;    // BF16 x, quantized in the activation stage
  const void* fn16;    // MXFP8 x, staged as BF16 (null: not built)
  const void* fn16_q;  // BF16 x, quantized and staged as BF16 (null: not built)
};

#define MXG_FN(RB, WN, WK, D, SK, QX, XR, X16) \
  reinterpret_cast<const void*>(&gemm_publish_kernel<RB, WN, WK, D, SK, QX, XR, X16>)
#define MXG_V(RB, WN, WK, D, SK)                                                     \
  Variant{TileCfg{RB, WN, WK, D}, SK, MXG_FN(RB, WN, WK, D, SK, false, 1, false),    \
          MXG_FN(RB, WN, WK, D, SK, true, 1, false), nullptr, nullptr}
// Also built with x staged as BF16 (the tiles the chooser takes for the
// workload shapes).
#define MXG_V16(RB, WN, WK, D, SK)                                                   \
  Variant{TileCfg{RB, WN, WK, D}, SK, MXG_FN(RB, WN, WK, D, SK, false, 1, false),    \
          MXG_FN(RB, WN, WK, D, SK, true, 1, false),                                 \
          MXG_FN(RB, WN, WK, D, SK, false, 1, true), MXG_FN(RB, WN, WK, D, SK, true, 1, true)}
// The x stage with an 8-chunk first round (xr = 2: a slice of twice the
// size staged before the first barrier without a second, out-of-line round);
// BF16 x stages through XQuant either way.
// Not built with x staged as BF16: on N=4096/K=16384/m=8/split-K 4 that was
// 1 us slower.
#define MXG_V2(RB, WN, WK, D, SK)                                                    \
  Variant{TileCfg{RB, WN, WK, D, 2}, SK, MXG_FN(RB, WN, WK, D, SK, false, 2, false), \
          MXG_FN(RB, WN, WK, D, SK, true, 1, false), nullptr, nullptr}
#define MXG_VARIANT(RB, WN, WK, D) \
  MXG_V(RB, WN, WK, D, 1), MXG_V(RB, WN, WK, D, 2), MXG_V(RB, WN, WK, D, 4), \
      MXG_V(RB, WN, WK, D, 8)
#define MXG_VARIANT16(RB, WN, WK, D) \
  MXG_V16(RB, WN, WK, D, 1), MXG_V16(RB, WN, WK, D, 2), MXG_V16(RB, WN, WK, D, 4), \
      MXG_V16(RB, WN, WK, D, 8)

// The shares of the variant table, one per gemm_variants_*.hip file.
constexpr int kVariantParts = 6;
const Variant* gemm_variants_0(size_t* count);
const Variant* gemm_variants_1(size_t* count);
const Variant* gemm_variants_2(size_t* count);
const Variant* gemm_variants_3(size_t* count);
const Variant* gemm_variants_4(size_t* count);
const Variant* gemm_variants_5(size_t* count);

}  // namespace mxg
