// Kernel variants of the publishing GEMM, share 3 of the table (the
// template is in gemm_kernel.h; the shares are separate files so that they
// compile in parallel).

#include "gemm_kernel.h"

namespace mxg {
namespace {
const Variant kPart[] = {
    MXG_VARIANT16(1, 2, 2, 8),
    MXG_VARIANT16(1, 7, 1, 5),
};
}  // namespace

const Variant* gemm_variants_3(size_t* count) {
  *count = sizeof(kPart) / sizeof(kPart[0]);
  return kPart;
}

}  // namespace mxg
