// Internal declarations shared by the host API and the kernel files of the
// MXFP8 publishing GEMM library (gfx950). Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mxgemm.h"

namespace mxg {

// Everything one GEMM+publish launch needs, by value.
struct GemmArgs {
  const uint8_t* w;   // packed W tiles (mxgemm_pack_weight)
  const uint8_t* ws;  // packed scales
  const uint8_t* x;   // [m, k] e4m3fn (null when xb is given)
  const uint8_t* xs;  // [m, k/32] E8M0 (null when xb is given)
  const uint16_t* xb; // [m, k] BF16 to quantize in the kernel, or null
  uint8_t* xq_out;    // with xb: [m, k] codes as quantized, or null
  uint8_t* xs_out;    // with xb: [m, k/32] scales as quantized, or null
  uint8_t* slot;      // mailbox slots + rank * capacity (generation 0); null: no publish
  int64_t gen_stride; // bytes between generations: ranks * capacity
  uint32_t* state;    // mailbox state words; null: plain GEMM into c_out
  uint32_t* ws_hdr;   // split-K workspace header (null when split_k == 1)
  uint32_t* flags;    // split-K per-workgroup epoch words (null when split_k == 1)
  uint64_t* pairs;    // split-K (value, epoch) pairs (null when split_k == 1)
  int64_t pairs_bytes; // bytes of the pairs region
  uint16_t* c_out;    // raw BF16 output or null
  int32_t m, n, k, split_k;
  uint32_t spin_limit;
  int32_t xcd_groups; // set by the launcher: the slices of a tile share an XCD
  // Added to the workspace's stored EPOCH word on every read and taken off
  // on every write: 0 for a workspace armed by mxgemm_workspace_init (stored
  // EPOCH starts at 1), 1 for the library's zero-filled no-allocation
  // scratch (stored 0 means epoch 1). Epoch 0 is never live either way.
  uint32_t epoch_bias;
};

// A workgroup computes an output tile of n_tile = 16 * rb * wn rows for one
// K slice; its 64 * wn * wk threads form wn x wk waves (wn along rows, wk
// along K); each wave keeps `depth` K-blocks of W loads in flight.
// xr: rounds of 4 chunks per thread in the activation stage's first round.
// x16: the activation stage converts the x slice to its exact BF16 values on
// the way into LDS (B operand order), so the main loop reads the B operand
// without converting it; taken when the variant is built with it and its
// 2 m k_slice bytes of LDS fit.
struct TileCfg {
  int rb, wn, wk, depth;
  int xr = 1;
  int x16 = 0;
};

inline int tile_rows(const TileCfg& c) { return 16 * c.rb * c.wn; }
// Worker waves, plus the control wave of split-K launches.
inline int tile_threads(const TileCfg& c, int split_k) {
  return 64 * (c.wn * c.wk + (split_k > 1 ? 1 : 0));
}

// Dynamic LDS bytes of a launch (x slice and its scales, or its BF16 form when
// c.x16; the partial tile).
size_t gemm_lds_bytes(const TileCfg& c, int m, int k_slice);

// The tile for a problem. tile null: the default choice; "fp8": the default
// tile with x kept in FP8 in LDS; "rb,wn,wk,depth[,xr[,x16]]": exactly that
// variant (fails when it does not fit). Returns false when no variant fits.
bool choose_tile(int m, int n, int k, int split_k, const char* tile, TileCfg* out);

// Whether a variant is compiled in.
bool tile_available(const TileCfg& c);

// How many workgroups of this variant can be resident at once on the current
// device (CUs x blocks per CU); negative on a HIP error.
long gemm_resident_blocks(const TileCfg& c, int split_k, size_t lds_bytes);

// ev_start/ev_stop (may be null) are recorded around the kernel itself.
hipError_t launch_gemm_publish(const GemmArgs& a, const TileCfg& c, hipStream_t s,
                               hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

// Packs row-major W and scales into the GEMM's tile layout.
hipError_t launch_pack_weight(const uint8_t* w, const uint8_t* ws, int n, int k, uint8_t* wp,
                              uint8_t* wsp, hipStream_t s);

// Stand-alone activation quantizer: [rows, k] BF16 -> codes and scales.
hipError_t launch_quantize(const uint16_t* x, int rows, int k, uint8_t* xq, uint8_t* xs,
                           hipStream_t s);

// Plain read stream of `bytes` (a multiple of 16): one checksum word per
// MXG_STREAM_CHUNK_BYTES chunk into sink.
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s);

// The configurable read stream of mxg_stream_read_cfg (arguments checked by
// the caller).
hipError_t launch_stream_read_cfg(const void* src, size_t bytes, uint32_t* sink, int workgroups,
                                  int threads, int unroll, int kind, int interleave,
                                  hipStream_t s);

// One wave's 16 x 16 x k product with the block-scaled fp8 MFMA (scaled) or
// with the GEMM's BF16 conversion and BF16 MFMA (see mxg_probe_mfma).
hipError_t launch_mfma_probe(const uint8_t* a, const uint8_t* as, const uint8_t* b,
                             const uint8_t* bs, int k, int scaled, float* c, hipStream_t s);

// Mailbox kernels.
hipError_t launch_fill_u32(uint32_t* p, size_t words, uint32_t value, hipStream_t s);
hipError_t launch_state_init(uint32_t* state, hipStream_t s);
hipError_t launch_workspace_init(uint32_t* ws, size_t bytes, hipStream_t s);
hipError_t launch_mailbox_publish(uint8_t* slot, int64_t gen_stride, uint32_t* state,
                                  int peer, const uint8_t* src, int64_t nbytes, bool words,
                                  hipStream_t s);
hipError_t launch_mailbox_collect(uint8_t* slots, int64_t gen_stride, int64_t capacity,
                                  int ranks, uint32_t* state, uint8_t* out,
                                  int64_t nbytes, uint32_t spin_limit, hipStream_t s);
hipError_t launch_mailbox_collect_sum(uint8_t* slots, int64_t gen_stride, int64_t capacity,
                                      int ranks, uint32_t* state, uint8_t* out, int64_t nbytes,
                                      uint32_t spin_limit, hipStream_t s);

hipError_t launch_mailbox_all_gather(uint8_t* slots, int64_t gen_stride, int64_t capacity,
                                     int ranks, int self, uint32_t* state, const uint8_t* src,
                                     uint8_t* out, int64_t nbytes, uint32_t spin_limit,
                                     hipStream_t s);

// Poll limit of a call on mailbox mb (null: the default).
uint32_t spin_limit(const mxg_mailbox* mb);

// Host validation of a GEMM call from sizes and addresses alone, everything
// but the workspace: MXG_OK or the code gemm_call would return.
int gemm_validate(const mxg_mailbox* mb, const uint8_t* w, const uint8_t* w_scale,
                  const uint8_t* x, const uint8_t* x_scale, const uint16_t* xb, int32_t m,
                  int32_t n, int32_t k, int32_t split_k, uint16_t* c_out, uint8_t* xq_out,
                  uint8_t* xs_out);

// One GEMM launch after host validation (the body of mxgemm_publish and its
// siblings). mb null: plain GEMM into c_out. xb non-null: BF16 x quantized in
// the kernel. epoch_bias: see GemmArgs. Returns an MXG_* code.
int gemm_call(const mxg_mailbox* mb, const uint8_t* w, const uint8_t* w_scale, const uint8_t* x,
              const uint8_t* x_scale, const uint16_t* xb, int32_t m, int32_t n, int32_t k,
              int32_t split_k, void* workspace, size_t workspace_bytes, uint32_t epoch_bias,
              uint16_t* c_out, uint8_t* xq_out, uint8_t* xs_out, void* stream, void* ev_start,
              void* ev_stop, const char* tile = nullptr);

}  // namespace mxg
