// Kernel variants of the publishing GEMM, share 5 of the table (the
// template is in gemm_kernel.h; the shares are separate files so that they
// compile in parallel).

#include "gemm_kernel.h"

namespace mxg {
namespace {
const Variant kPart[] = {
    MXG_VARIANT(1, 8, 1, 8),
    MXG_VARIANT(2, 2, 2, 4),
    MXG_V2(1, 4, 1, 3, 1),
    MXG_V2(1, 4, 1, 3, 2),
    MXG_V2(1, 4, 1, 3, 4),
    MXG_V2(1, 4, 1, 3, 8),
    MXG_V2(1, 1, 16, 4, 1),
};
}  // namespace

const Variant* gemm_variants_5(size_t* count) {
  *count = sizeof(kPart) / sizeof(kPart[0]);
  return kPart;
}

}  // namespace mxg
