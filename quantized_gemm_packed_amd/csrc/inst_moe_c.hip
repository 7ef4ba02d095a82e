// MoE GEMM instances (part 3): NVFP4 and MXINT4 experts x bf16
// activations.  The kernels are in gemm_kernels.h.
#include "gemm_kernels.h"

namespace hum {

static const Instance kMoeC[] = {
    HUM_MOE_SET(F_NVFP4_BF16, EPI_SWIGLU_BF16),
    HUM_MOE_SET(F_MXINT4_BF16, EPI_SWIGLU_BF16),
};

HUM_TABLE(instances_moe_c, kMoeC)

}  // namespace hum
