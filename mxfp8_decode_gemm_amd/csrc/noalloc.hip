// mxgemm_publish_noalloc: the publishing GEMM for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc). The split-K workspace, the only device memory the GEMM
// needs beyond its inputs and outputs, is a library-held array instead of a
// caller's buffer.
//
// `scratch` below is that array, one copy per GPU, alive until the process
// ends. The code object's loader fills it with zeros on each device, which is
// an armed workspace under epoch bias 1 (stored EPOCH 0 is epoch 1; the zero
// epoch words and zero-tagged pairs are never live), so no call ever has to
// clear it. In host code the name `scratch` is a host-side stand-in, not a
// device address: the kernels get the address hipGetSymbolAddress returns for
// the current device, looked up once per device on the first call there.

#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/mxgemm.h"
#include "mxgemm_internal.h"

namespace {

constexpr size_t kScratchBytes =
    MXG_WS_HEADER_BYTES + MXG_WS_FLAG_BYTES + (size_t)MXG_NOALLOC_PAIR_BYTES;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch`, per device

// The current device's copy of `scratch`, or null (no device, a device index
// past kMaxDevices, or a failed symbol lookup).
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> g(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int mxgemm_publish_noalloc(const mxg_mailbox* mb, const uint8_t* w,
                                      const uint8_t* w_scale, const uint8_t* x,
                                      const uint8_t* x_scale, int32_t m, int32_t n, int32_t k,
                                      int32_t split_k, uint16_t* c_out, void* stream) {
  if (!mb) return MXG_EINVAL;
  const int rc = mxg::gemm_validate(mb, w, w_scale, x, x_scale, nullptr, m, n, k, split_k,
                                    c_out, nullptr, nullptr);
  if (rc != MXG_OK) return rc;
  if (split_k == 1)  // no workspace in use: exactly mxgemm_publish
    return mxg::gemm_call(mb, w, w_scale, x, x_scale, nullptr, m, n, k, split_k, nullptr, 0, 0,
                          c_out, nullptr, nullptr, stream, nullptr, nullptr);
  const size_t need = mxgemm_workspace_bytes(m, n, k, split_k);
  if (need > kScratchBytes) return MXG_EWORKSPACE;
  void* ws = device_scratch();
  if (!ws) return MXG_EHIP;
  return mxg::gemm_call(mb, w, w_scale, x, x_scale, nullptr, m, n, k, split_k, ws, need, 1,
                        c_out, nullptr, nullptr, stream, nullptr, nullptr);
}
