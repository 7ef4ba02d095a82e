// Dense GEMM instances (part 1): INT4 / UINT4, FP8 W8A8, MXFP4 x bf16,
// MXFP4 x MXFP8, W4A4 and block-scaled FP8.  The kernels are in
// gemm_kernels.h.
#include "gemm_kernels.h"

namespace hum {

static const Instance kDenseA[] = {
    HUM_DENSE_SET(F_INT),
    HUM_DENSE_SET(F_FP8),
    HUM_DENSE_SET(F_MXFP4_BF16),
    HUM_DENSE_SET(F_MXFP4_MXFP8),
    HUM_DENSE_TILE_SET(F_MXFP4_MXFP4),
    HUM_DENSE_SET(F_FP8_BLOCK),
    HUM_DENSE_TILE32_SET(F_INT),
    HUM_DENSE_TILE32_SET(F_MXFP4_BF16),
    HUM_TILE32_S(F_MXFP4_BF16, 8, 4, 2),
};

HUM_TABLE(instances_dense_a, kDenseA)

}  // namespace hum
