// Dense GEMM instances (part 2): W8A16 (FP8 and INT8 weights), NVFP4 and
// MXINT4 weights x bf16.  The kernels are in gemm_kernels.h.
#include "gemm_kernels.h"

namespace hum {

static const Instance kDenseB[] = {
    HUM_DENSE_SET(F_FP8_BF16),
    HUM_DENSE_SET(F_INT8_BF16),
    HUM_DENSE_SET(F_NVFP4_BF16),
    HUM_DENSE_SET(F_MXINT4_BF16),
};

HUM_TABLE(instances_dense_b, kDenseB)

}  // namespace hum
