// Dense GEMM instances (part 4): INT2 / UINT2 and INT1 / UINT1 weights x
// bf16.  The kernels are in gemm_kernels.h.
#include "gemm_kernels.h"

namespace hum {

static const Instance kDenseD[] = {
    HUM_DENSE_SET(F_INT2),
    HUM_DENSE_TILE32_SET(F_INT2),
    HUM_DENSE_SET(F_INT1),
    HUM_DENSE_TILE32_SET(F_INT1),
};

HUM_TABLE(instances_dense_d, kDenseD)

}  // namespace hum
