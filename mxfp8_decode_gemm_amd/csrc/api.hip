// C ABI of the MXFP8 publishing GEMM library: host-side validation (from
// sizes and addresses only, before any HIP call), dispatch, graph helpers.
// The declarations, argument meanings and error rules are in
// include/mxgemm.h.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/mxgemm.h"
#include "mxgemm_internal.h"

namespace mxg {
namespace {
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool mailbox_ok(const mxg_mailbox* mb) {
  return mb && mb->slots && mb->state && mb->ranks >= 1 && mb->ranks <= MXG_MAX_RANKS &&
         mb->rank >= 0 && mb->rank < mb->ranks && mb->capacity_bytes > 0 &&
         mb->capacity_bytes % MXG_PACK_BYTES == 0;
}

int hip_code(hipError_t e) { return e == hipSuccess ? MXG_OK : MXG_EHIP; }
}  // namespace

uint32_t spin_limit(const mxg_mailbox* mb) {
  return mb && mb->spin_limit ? mb->spin_limit : MXG_DEFAULT_SPIN_LIMIT;
}
}  // namespace mxg

using namespace mxg;

extern "C" {

size_t mxg_mailbox_slots_bytes(int32_t ranks, int64_t capacity_bytes) {
  if (ranks < 1 || ranks > MXG_MAX_RANKS || capacity_bytes <= 0 ||
      capacity_bytes % MXG_PACK_BYTES)
    return 0;
  return (size_t)MXG_GENERATIONS * (size_t)ranks * (size_t)capacity_bytes;
}

int mailbox_init(mxg_mailbox* mb, void* slots, uint32_t* state, int32_t ranks, int32_t rank,
                 int64_t capacity_bytes, void* stream) {
  if (!mb || !slots || !state) return MXG_EINVAL;
  const size_t bytes = mxg_mailbox_slots_bytes(ranks, capacity_bytes);
  if (bytes == 0 || rank < 0 || rank >= ranks) return MXG_EINVAL;
  if (!aligned16(slots) || !aligned16(state)) return MXG_EALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_fill_u32(static_cast<uint32_t*>(slots), bytes / 4, MXG_SENTINEL, s);
  if (e == hipSuccess) e = launch_state_init(state, s);
  if (e != hipSuccess) return MXG_EHIP;
  mb->slots = slots;
  mb->state = state;
  mb->ranks = ranks;
  mb->rank = rank;
  mb->capacity_bytes = capacity_bytes;
  mb->spin_limit = 0;
  mb->reserved = 0;
  return MXG_OK;
}

size_t mxgemm_workspace_bytes(int32_t m, int32_t n, int32_t k, int32_t split_k) {
  (void)m;
  (void)k;
  if (split_k <= 1 || n <= 0) return 0;
  const size_t n8 = (size_t)((n + 7) / 8) * 8;
  // header, per-workgroup epoch words, pairs[split][token 0..7][n / 8][8] of 8 bytes
  return MXG_WS_HEADER_BYTES + MXG_WS_FLAG_BYTES + (size_t)split_k * 8 * n8 * 8;
}

size_t mxgemm_packed_weight_bytes(int32_t n, int32_t k) {
  if (n <= 0 || k <= 0 || k % 128) return 0;
  return (size_t)((n + 15) / 16) * 16 * (size_t)k;
}

size_t mxgemm_packed_scale_bytes(int32_t n, int32_t k) {
  if (n <= 0 || k <= 0 || k % 128) return 0;
  const size_t rbn = (size_t)((n + 15) / 16);
  // the scale tiles, then one range word per row block (rounded to 16 bytes)
  return rbn * 16 * (size_t)(k / 32) + (rbn * 4 + 15) / 16 * 16;
}

int mxgemm_pack_weight(const uint8_t* w, const uint8_t* w_scale, int32_t n, int32_t k,
                       uint8_t* w_packed, uint8_t* ws_packed, void* stream) {
  if (!w || !w_scale || !w_packed || !ws_packed) return MXG_EINVAL;
  if (n <= 0 || n % 8 || k <= 0 || k % 128) return MXG_EINVAL;
  if (!aligned16(w) || !aligned16(w_scale) || !aligned16(w_packed) || !aligned16(ws_packed))
    return MXG_EALIGN;
  return hip_code(launch_pack_weight(w, w_scale, n, k, w_packed, ws_packed,
                                     static_cast<hipStream_t>(stream)));
}

int mxgemm_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace || workspace_bytes < MXG_WS_HEADER_BYTES + MXG_WS_FLAG_BYTES ||
      workspace_bytes % 16)
    return MXG_EINVAL;
  if (!aligned16(workspace)) return MXG_EALIGN;
  return hip_code(launch_workspace_init(static_cast<uint32_t*>(workspace), workspace_bytes,
                                        static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace mxg {
int gemm_validate(const mxg_mailbox* mb, const uint8_t* w, const uint8_t* w_scale,
                  const uint8_t* x, const uint8_t* x_scale, const uint16_t* xb, int32_t m,
                  int32_t n, int32_t k, int32_t split_k, uint16_t* c_out, uint8_t* xq_out,
                  uint8_t* xs_out) {
  if (mb ? !mailbox_ok(mb) : !c_out) return MXG_EINVAL;
  if (!w || !w_scale) return MXG_EINVAL;
  if (xb ? (x || x_scale) : (!x || !x_scale || xq_out || xs_out)) return MXG_EINVAL;
  if (xb && (!xq_out) != (!xs_out)) return MXG_EINVAL;
  if (m < 1 || m > MXG_MAX_ROWS || n <= 0 || n % 8 || k <= 0 || k % 128) return MXG_EINVAL;
  if (split_k != 1 && split_k != 2 && split_k != 4 && split_k != 8) return MXG_EINVAL;
  if (k % (128 * split_k)) return MXG_EINVAL;
  if (!aligned16(w) || !aligned16(w_scale) || (x && !aligned16(x)) ||
      (x_scale && !aligned16(x_scale)) || (xb && !aligned16(xb)) ||
      (xq_out && !aligned16(xq_out)) || (c_out && !aligned16(c_out)))
    return MXG_EALIGN;
  if (mb && (!aligned16(mb->slots) || !aligned16(mb->state))) return MXG_EALIGN;
  if (mb && (int64_t)2 * m * n > mb->capacity_bytes) return MXG_ECAPACITY;
  return MXG_OK;
}

// One GEMM launch. mb null: plain GEMM into c_out (required). xb non-null:
// BF16 x quantized in the kernel (x and x_scale must be null), with the
// quantized activation optionally written to xq_out / xs_out.
int gemm_call(const mxg_mailbox* mb, const uint8_t* w, const uint8_t* w_scale,
              const uint8_t* x, const uint8_t* x_scale, const uint16_t* xb, int32_t m, int32_t n,
              int32_t k, int32_t split_k, void* workspace, size_t workspace_bytes,
              uint32_t epoch_bias, uint16_t* c_out, uint8_t* xq_out, uint8_t* xs_out,
              void* stream, void* ev_start, void* ev_stop, const char* tile) {
  const int rc =
      gemm_validate(mb, w, w_scale, x, x_scale, xb, m, n, k, split_k, c_out, xq_out, xs_out);
  if (rc != MXG_OK) return rc;
  if (split_k > 1) {
    if (!workspace || workspace_bytes < mxgemm_workspace_bytes(m, n, k, split_k))
      return MXG_EWORKSPACE;
    if (!aligned16(workspace)) return MXG_EALIGN;
  }
  // The tile choice also checks that a split-K grid can be resident at once:
  // the workgroups of one output tile wait for each other's partials.
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MXG_EHIP;
  TileCfg cfg;
  if (!choose_tile(m, n, k, split_k, tile, &cfg)) return MXG_EUNSUPPORTED;

  GemmArgs a;
  a.w = w;
  a.ws = w_scale;
  a.x = x;
  a.xs = x_scale;
  a.xb = xb;
  a.xq_out = xq_out;
  a.xs_out = xs_out;
  a.slot = mb ? static_cast<uint8_t*>(mb->slots) + (size_t)mb->rank * mb->capacity_bytes
              : nullptr;
  a.gen_stride = mb ? (int64_t)mb->ranks * mb->capacity_bytes : 0;
  a.state = mb ? mb->state : nullptr;
  a.ws_hdr = split_k > 1 ? static_cast<uint32_t*>(workspace) : nullptr;
  a.flags = split_k > 1 ? static_cast<uint32_t*>(workspace) + MXG_WS_HEADER_BYTES / 4 : nullptr;
  a.pairs = split_k > 1 ? reinterpret_cast<uint64_t*>(static_cast<uint8_t*>(workspace) +
                                                       MXG_WS_HEADER_BYTES + MXG_WS_FLAG_BYTES)
                        : nullptr;
  a.pairs_bytes = split_k > 1 ? (int64_t)(workspace_bytes - MXG_WS_HEADER_BYTES -
                                          MXG_WS_FLAG_BYTES)
                              : 0;
  a.xcd_groups = 0;
  a.c_out = c_out;
  a.m = m;
  a.n = n;
  a.k = k;
  a.split_k = split_k;
  a.spin_limit = spin_limit(mb);
  a.epoch_bias = epoch_bias;
  return hip_code(launch_gemm_publish(a, cfg, static_cast<hipStream_t>(stream),
                                      static_cast<hipEvent_t>(ev_start),
                                      static_cast<hipEvent_t>(ev_stop)));
}
}  // namespace mxg

extern "C" {

int mxgemm_publish(const mxg_mailbox* mb, const uint8_t* w, const uint8_t* w_scale,
                   const uint8_t* x, const uint8_t* x_scale, int32_t m, int32_t n, int32_t k,
                   int32_t split_k, void* workspace, size_t workspace_bytes, uint16_t* c_out,
                   void* stream) {
  if (!mb) return MXG_EINVAL;
  return gemm_call(mb, w, w_scale, x, x_scale, nullptr, m, n, k, split_k, workspace,
                   workspace_bytes, 0, c_out, nullptr, nullptr, stream, nullptr, nullptr);
}

int mxgemm_publish_timed(const mxg_mailbox* mb, const uint8_t* w, const uint8_t* w_scale,
                         const uint8_t* x, const uint8_t* x_scale, int32_t m, int32_t n,
                         int32_t k, int32_t split_k, void* workspace, size_t workspace_bytes,
                         uint16_t* c_out, void* stream, void* ev_start, void* ev_stop) {
  if (!mb || !ev_start || !ev_stop) return MXG_EINVAL;
  return gemm_call(mb, w, w_scale, x, x_scale, nullptr, m, n, k, split_k, workspace,
                   workspace_bytes, 0, c_out, nullptr, nullptr, stream, ev_start, ev_stop);
}

int mxgemm_publish_bf16(const mxg_mailbox* mb, const uint8_t* w, const uint8_t* w_scale,
                        const uint16_t* x, int32_t m, int32_t n, int32_t k, int32_t split_k,
                        void* workspace, size_t workspace_bytes, uint16_t* c_out,
                        uint8_t* x_q_out, uint8_t* x_scale_out, void* stream) {
  if (!mb || !x) return MXG_EINVAL;
  return gemm_call(mb, w, w_scale, nullptr, nullptr, x, m, n, k, split_k, workspace,
                   workspace_bytes, 0, c_out, x_q_out, x_scale_out, stream, nullptr, nullptr);
}

int mxgemm(const uint8_t* w, const uint8_t* w_scale, const uint8_t* x, const uint8_t* x_scale,
           int32_t m, int32_t n, int32_t k, int32_t split_k, void* workspace,
           size_t workspace_bytes, uint16_t* c_out, void* stream) {
  if (!c_out) return MXG_EINVAL;
  return gemm_call(nullptr, w, w_scale, x, x_scale, nullptr, m, n, k, split_k, workspace,
                   workspace_bytes, 0, c_out, nullptr, nullptr, stream, nullptr, nullptr);
}

int mxgemm_tile(const char* tile, const mxg_mailbox* mb, const uint8_t* w,
                const uint8_t* w_scale, const uint8_t* x, const uint8_t* x_scale,
                const uint16_t* x_bf16, int32_t m, int32_t n, int32_t k, int32_t split_k,
                void* workspace, size_t workspace_bytes, uint16_t* c_out, uint8_t* x_q_out,
                uint8_t* x_scale_out, void* stream) {
  if (!tile) return MXG_EINVAL;
  if (!mb && !c_out) return MXG_EINVAL;             // the plain GEMM needs c_out
  if (!mb && x_bf16) return MXG_EINVAL;             // BF16 x only with a publish
  if (x_bf16 && (x || x_scale)) return MXG_EINVAL;  // one activation form
  return gemm_call(mb, w, w_scale, x, x_scale, x_bf16, m, n, k, split_k, workspace,
                   workspace_bytes, 0, c_out, x_q_out, x_scale_out, stream, nullptr, nullptr,
                   tile);
}

int mxfp8_quantize(const uint16_t* x, int32_t rows, int32_t k, uint8_t* x_q, uint8_t* x_scale,
                   void* stream) {
  if (!x || !x_q || !x_scale || rows < 1 || k <= 0 || k % 32) return MXG_EINVAL;
  if (!aligned16(x) || !aligned16(x_q)) return MXG_EALIGN;
  return hip_code(launch_quantize(x, rows, k, x_q, x_scale, static_cast<hipStream_t>(stream)));
}

namespace {
int slot_publish_impl(const mxg_mailbox* mb, int32_t rank, const void* src, int64_t nbytes,
                      bool words, void* stream) {
  if (!mailbox_ok(mb) || !src || rank < 0 || rank >= mb->ranks) return MXG_EINVAL;
  if (!aligned16(src) || !aligned16(mb->slots) || !aligned16(mb->state)) return MXG_EALIGN;
  if (nbytes <= 0 || nbytes > mb->capacity_bytes || nbytes % MXG_PACK_BYTES)
    return MXG_ECAPACITY;
  uint8_t* slot = static_cast<uint8_t*>(mb->slots) + (size_t)rank * mb->capacity_bytes;
  return hip_code(launch_mailbox_publish(slot, (int64_t)mb->ranks * mb->capacity_bytes,
                                         mb->state, rank == mb->rank ? -1 : rank,
                                         static_cast<const uint8_t*>(src), nbytes,
                                         words, static_cast<hipStream_t>(stream)));
}
}  // namespace

int mailbox_publish(const mxg_mailbox* mb, int32_t rank, const void* src, int64_t nbytes,
                    void* stream) {
  return slot_publish_impl(mb, rank, src, nbytes, false, stream);
}

int mailbox_publish_words(const mxg_mailbox* mb, int32_t rank, const void* src, int64_t nbytes,
                          void* stream) {
  return slot_publish_impl(mb, rank, src, nbytes, true, stream);
}

int mailbox_all_gather(const mxg_mailbox* mb, const void* src, void* out, int64_t nbytes,
                       void* stream) {
  if (!mailbox_ok(mb) || !src || !out) return MXG_EINVAL;
  if (!aligned16(src) || !aligned16(out) || !aligned16(mb->slots) || !aligned16(mb->state))
    return MXG_EALIGN;
  if (nbytes <= 0 || nbytes > mb->capacity_bytes || nbytes % MXG_PACK_BYTES)
    return MXG_ECAPACITY;
  // src must not overlap out, except as exactly the caller's own output row.
  const uint8_t* s = static_cast<const uint8_t*>(src);
  const uint8_t* o = static_cast<const uint8_t*>(out);
  const uint8_t* own = o + (size_t)mb->rank * nbytes;
  if (s != own && s < o + (size_t)mb->ranks * nbytes && o < s + nbytes) return MXG_EINVAL;
  return hip_code(launch_mailbox_all_gather(
      static_cast<uint8_t*>(mb->slots), (int64_t)mb->ranks * mb->capacity_bytes,
      mb->capacity_bytes, mb->ranks, mb->rank, mb->state, s, static_cast<uint8_t*>(out),
      nbytes, spin_limit(mb), static_cast<hipStream_t>(stream)));
}

int mailbox_collect(const mxg_mailbox* mb, void* out, int64_t nbytes, void* stream) {
  if (!mailbox_ok(mb) || !out) return MXG_EINVAL;
  if (!aligned16(out) || !aligned16(mb->slots) || !aligned16(mb->state)) return MXG_EALIGN;
  if (nbytes <= 0 || nbytes > mb->capacity_bytes || nbytes % MXG_PACK_BYTES)
    return MXG_ECAPACITY;
  return hip_code(launch_mailbox_collect(
      static_cast<uint8_t*>(mb->slots), (int64_t)mb->ranks * mb->capacity_bytes,
      mb->capacity_bytes, mb->ranks, mb->state, static_cast<uint8_t*>(out), nbytes,
      spin_limit(mb), static_cast<hipStream_t>(stream)));
}

int mailbox_collect_sum(const mxg_mailbox* mb, void* out, int64_t nbytes, void* stream) {
  if (!mailbox_ok(mb) || !out) return MXG_EINVAL;
  if (!aligned16(out) || !aligned16(mb->slots) || !aligned16(mb->state)) return MXG_EALIGN;
  if (nbytes <= 0 || nbytes > mb->capacity_bytes || nbytes % MXG_PACK_BYTES)
    return MXG_ECAPACITY;
  return hip_code(launch_mailbox_collect_sum(
      static_cast<uint8_t*>(mb->slots), (int64_t)mb->ranks * mb->capacity_bytes,
      mb->capacity_bytes, mb->ranks, mb->state, static_cast<uint8_t*>(out), nbytes,
      spin_limit(mb), static_cast<hipStream_t>(stream)));
}

int mxg_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 || bytes > ((size_t)1 << 40)) return MXG_EINVAL;
  if (!aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return MXG_EALIGN;
  return hip_code(launch_stream_read(src, bytes, sink, static_cast<hipStream_t>(stream)));
}

int mxg_stream_read_cfg(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups,
                        int32_t threads, int32_t unroll, int32_t load_kind, int32_t interleave,
                        void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 || bytes > ((size_t)1 << 40)) return MXG_EINVAL;
  if (threads != 256 && threads != 512) return MXG_EINVAL;
  if (unroll != 4 && unroll != 8 && unroll != 16) return MXG_EINVAL;
  if (load_kind < 0 || load_kind > 4 || (interleave != 0 && interleave != 1)) return MXG_EINVAL;
  if (workgroups < 0 || workgroups > 65536 || (interleave && workgroups == 0)) return MXG_EINVAL;
  if ((load_kind == 2 || load_kind == 3) && bytes > (size_t)0x7FFF0000)
    return MXG_EINVAL;  // one raw buffer
  if (workgroups == 0 && (bytes + MXG_STREAM_CHUNK_BYTES - 1) / MXG_STREAM_CHUNK_BYTES > 0x7FFFFFFF)
    return MXG_EINVAL;
  if (!aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return MXG_EALIGN;
  return hip_code(launch_stream_read_cfg(src, bytes, sink, workgroups, threads, unroll, load_kind,
                                         interleave, static_cast<hipStream_t>(stream)));
}

int mxg_probe_mfma(const uint8_t* a, const uint8_t* a_scale, const uint8_t* b,
                   const uint8_t* b_scale, int32_t k, int32_t scaled, float* c, void* stream) {
  if (!a || !a_scale || !b || !b_scale || !c || k <= 0 || k % 128 || (scaled != 0 && scaled != 1))
    return MXG_EINVAL;
  if (!aligned16(a) || !aligned16(b) || !aligned16(c)) return MXG_EALIGN;
  return hip_code(launch_mfma_probe(a, a_scale, b, b_scale, k, scaled, c,
                                    static_cast<hipStream_t>(stream)));
}

int mxg_graph_begin(void* stream) {
  if (!stream) return MXG_EINVAL;  // the null stream cannot be captured
  return hip_code(
      hipStreamBeginCapture(static_cast<hipStream_t>(stream), hipStreamCaptureModeRelaxed));
}

int mxg_graph_end(void* stream, void** exec) {
  if (!stream || !exec) return MXG_EINVAL;
  hipGraph_t graph = nullptr;
  hipError_t e = hipStreamEndCapture(static_cast<hipStream_t>(stream), &graph);
  if (e != hipSuccess) return MXG_EHIP;
  hipGraphExec_t ge = nullptr;
  e = hipGraphInstantiate(&ge, graph, nullptr, nullptr, 0);
  (void)hipGraphDestroy(graph);
  if (e != hipSuccess) return MXG_EHIP;
  *exec = ge;
  return MXG_OK;
}

int mxg_graph_launch(void* exec, void* stream) {
  if (!exec) return MXG_EINVAL;
  return hip_code(
      hipGraphLaunch(static_cast<hipGraphExec_t>(exec), static_cast<hipStream_t>(stream)));
}

int mxg_graph_destroy(void* exec) {
  if (!exec) return MXG_EINVAL;
  return hip_code(hipGraphExecDestroy(static_cast<hipGraphExec_t>(exec)));
}

const char* mxg_strerror(int code) {
  switch (code) {
    case MXG_OK: return "ok";
    case MXG_EINVAL: return "invalid argument (null pointer, shape, rank or split_k)";
    case MXG_EALIGN: return "pointer not 16-byte aligned";
    case MXG_ECAPACITY: return "payload does not fit the mailbox slot";
    case MXG_EWORKSPACE: return "split-K workspace missing or too small";
    case MXG_EUNSUPPORTED: return "no kernel variant for these sizes on this device";
    case MXG_EHIP: return "HIP error";
    default: return "unknown error";
  }
}

}  // extern "C"
