// MoE GEMM instances (part 1): MXFP4 experts with bf16, MXFP8 and MXFP4
// activations.  The kernels are in gemm_kernels.h.
#include "gemm_kernels.h"

namespace hum {

static const Instance kMoeA[] = {
    HUM_STREAM(F_MXFP4_BF16, 2, 8, 4, A_GATHER, EPI_SWIGLU_BF16),
    HUM_STREAM(F_MXFP4_BF16, 2, 8, 4, A_DIRECT, EPI_SCATTER),
    HUM_STREAM(F_MXFP4_BF16, 2, 15, 4, A_GATHER, EPI_SWIGLU_BF16),
    HUM_STREAM(F_MXFP4_BF16, 2, 15, 4, A_DIRECT, EPI_SCATTER),
    HUM_MOE_SET(F_MXFP4_BF16, EPI_SWIGLU_BF16),
    HUM_MOE_SET(F_MXFP4_MXFP8, EPI_SWIGLU_MXFP8),
    HUM_MOE_TILE_SET(F_MXFP4_MXFP4, EPI_SWIGLU_MXFP4),
};

HUM_TABLE(instances_moe_a, kMoeA)

}  // namespace hum
