// Kernel variants of the publishing GEMM, share 1 of the table (the
// template is in gemm_kernel.h; the shares are separate files so that they
// compile in parallel).

#include "gemm_kernel.h"

namespace mxg {
namespace {
const Variant kPart[] = {
    MXG_VARIANT(1, 4, 1, 8),
    MXG_VARIANT16(1, 4, 1, 3),
};
}  // namespace

const Variant* gemm_variants_1(size_t* count) {
  *count = sizeof(kPart) / sizeof(kPart[0]);
  return kPart;
}

}  // namespace mxg
