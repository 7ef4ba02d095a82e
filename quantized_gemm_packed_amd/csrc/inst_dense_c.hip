// Dense GEMM instances (part 3): INT3 / UINT3 and MXFP6 (E2M3 / E3M2)
// weights x bf16.  The kernels are in gemm_kernels.h.
#include "gemm_kernels.h"

namespace hum {

static const Instance kDenseC[] = {
    HUM_DENSE_SET(F_INT3),
    HUM_DENSE_TILE32_SET(F_INT3),
    HUM_DENSE_SET(F_MXFP6_BF16),
    HUM_DENSE_SET(F_MXBF6_BF16),
};

HUM_TABLE(instances_dense_c, kDenseC)

}  // namespace hum
