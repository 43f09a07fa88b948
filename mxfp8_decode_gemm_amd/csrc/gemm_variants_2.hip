// Kernel variants of the publishing GEMM, share 2 of the table (the
// template is in gemm_kernel.h; the shares are separate files so that they
// compile in parallel).

#include "gemm_kernel.h"

namespace mxg {
namespace {
const Variant kPart[] = {
    MXG_VARIANT(1, 7, 1, 8),
    MXG_VARIANT(1, 7, 1, 4),
    MXG_VARIANT16(1, 7, 1, 3),
};
}  // namespace

const Variant* gemm_variants_2(size_t* count) {
  *count = sizeof(kPart) / sizeof(kPart[0]);
  return kPart;
}

}  // namespace mxg
