// Kernel variants of the publishing GEMM, share 0 of the table (the
// template is in gemm_kernel.h; the shares are separate files so that they
// compile in parallel).

#include "gemm_kernel.h"

namespace mxg {
namespace {
const Variant kPart[] = {
    MXG_VARIANT16(1, 1, 4, 4),
    MXG_VARIANT(1, 1, 8, 4),
    MXG_V(1, 1, 16, 4, 1),
};
}  // namespace

const Variant* gemm_variants_0(size_t* count) {
  *count = sizeof(kPart) / sizeof(kPart[0]);
  return kPart;
}

}  // namespace mxg
