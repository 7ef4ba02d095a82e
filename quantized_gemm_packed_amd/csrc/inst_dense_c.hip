// Dense GEMM instances (part 3): INT3 / UINT3 weights x bf16.  The kernels
// are in gemm_kernels.h.
#include "gemm_kernels.h"

namespace hum {

static const Instance kDenseC[] = {
    HUM_DENSE_SET(F_INT3),
    HUM_DENSE_TILE32_SET(F_INT3),
};

HUM_TABLE(instances_dense_c, kDenseC)

}  // namespace hum
