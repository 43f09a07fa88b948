// Kernel variants of the publishing GEMM, share 4 of the table (the
// template is in gemm_kernel.h; the shares are separate files so that they
// compile in parallel).

#include "gemm_kernel.h"

namespace mxg {
namespace {
const Variant kPart[] = {
    MXG_VARIANT16(1, 2, 2, 5),
    MXG_VARIANT(1, 4, 2, 8),
    MXG_VARIANT(2, 1, 4, 4),
};
}  // namespace

const Variant* gemm_variants_4(size_t* count) {
  *count = sizeof(kPart) / sizeof(kPart[0]);
  return kPart;
}

}  // namespace mxg
