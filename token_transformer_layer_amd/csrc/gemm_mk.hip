// Product kernels of one operand layout (input-gradient products computed
// transposed: A, the weight, M-contiguous; B, the output gradient,
// K-contiguous), split partial sums only.
#include "gemm_kernels.h"

namespace tpk {

hipError_t gemm_layout_mk_split(const GemmArgs &g, float *split_ws, int64_t ldc, Tile tile, hipStream_t st) {
    return launch<bf16, false, true>(g, EpiSplit{split_ws, ldc, (int64_t)g.M * ldc}, tile, st);
}

}  // namespace tpk
