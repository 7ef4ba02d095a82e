// MoE GEMM instances (part 2): FP8 experts -- per-token FP8 W8A8,
// block-scaled FP8 W8A8 (tiles only) and FP8 / INT8 weights with bf16
// activations (W8A16).  The SwiGLU output stays bf16; the layer quantizes
// it for the down GEMM where the activation format asks for it.  The
// kernels are in gemm_kernels.h.
#include "gemm_kernels.h"

namespace hum {

static const Instance kMoeB[] = {
    HUM_MOE_SET(F_FP8, EPI_SWIGLU_BF16),
    HUM_MOE_TILE_SET(F_FP8_BLOCK, EPI_SWIGLU_BF16),
    HUM_TILE_S(F_FP8_BLOCK, 1, 2, A_GATHER, EPI_SWIGLU_BF16, 3),
    HUM_TILE_S(F_FP8_BLOCK, 1, 2, A_DIRECT, EPI_SCATTER, 3),
    HUM_TILE_S(F_FP8_BLOCK, 1, 4, A_GATHER, EPI_SWIGLU_BF16, 3),
    HUM_TILE_S(F_FP8_BLOCK, 1, 4, A_DIRECT, EPI_SCATTER, 3),
    HUM_MOE_SET(F_FP8_BF16, EPI_SWIGLU_BF16),
    HUM_MOE_SET(F_INT8_BF16, EPI_SWIGLU_BF16),
};

HUM_TABLE(instances_moe_b, kMoeB)

}  // namespace hum
