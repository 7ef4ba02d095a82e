// Stream-K variants of the dense tile kernels (the tile shapes the selector
// uses where the tile count leaves the chip's workgroup slots unevenly
// filled).  The kernels are in gemm_kernels.h.
#include "gemm_kernels.h"

namespace hum {

static const Instance kDenseSk[] = {
    HUM_TILE_SK(F_INT, 2, 2, 3, 16),
    HUM_TILE_SK(F_INT, 2, 4, 3, 16),
    HUM_TILE_SK(F_INT, 4, 2, 3, 32),
    HUM_TILE_SK(F_INT, 4, 4, 3, 32),
    HUM_TILE_SK(F_INT, 4, 4, 2, 32),
    HUM_TILE_SK(F_FP8, 2, 2, 3, 16),
    HUM_TILE_SK(F_FP8, 4, 4, 2, 16),
    HUM_TILE_SK(F_FP8, 8, 2, 2, 16),
    HUM_TILE_SK(F_MXFP4_BF16, 1, 2, 3, 16),
    HUM_TILE_SK(F_MXFP4_BF16, 2, 2, 3, 16),
    HUM_TILE_SK(F_MXFP4_BF16, 4, 4, 3, 32),
    HUM_TILE_SK(F_MXFP4_MXFP8, 2, 2, 3, 16),
    HUM_TILE_SK(F_MXFP4_MXFP8, 8, 2, 2, 16),
    HUM_TILE_SK(F_MXFP4_MXFP4, 2, 2, 3, 16),
    HUM_TILE_SK(F_MXFP4_MXFP4, 4, 4, 3, 16),
    HUM_TILE_SK(F_FP8_BLOCK, 2, 2, 3, 16),
    HUM_TILE_SK(F_FP8_BLOCK, 8, 2, 2, 16),
    HUM_TILE_SK(F_FP8_BF16, 2, 2, 3, 16),
    HUM_TILE_SK(F_INT8_BF16, 2, 2, 3, 16),
    HUM_TILE_SK(F_NVFP4_BF16, 2, 2, 3, 16),
    HUM_TILE_SK(F_MXINT4_BF16, 2, 2, 3, 16),
    HUM_TILE_SK(F_INT3, 2, 2, 3, 16),
    HUM_TILE_SK(F_INT2, 2, 2, 3, 16),
    HUM_TILE_SK(F_INT1, 2, 2, 3, 16),
    HUM_TILE_SK(F_MXFP6_BF16, 2, 2, 3, 16),
    HUM_TILE_SK(F_MXBF6_BF16, 2, 2, 3, 16),
};

HUM_TABLE(instances_dense_sk, kDenseSk)

}  // namespace hum
