// Product kernels of one operand layout (weight-gradient products: both operands M/N-contiguous).
#include "gemm_kernels.h"

namespace tpk {

hipError_t gemm_layout_tn(bool is_bf16, const GemmArgs &g, Epi kind, const EpiArgs &e, float *split_ws, Tile tile,
                          hipStream_t st) {
    if (is_bf16) return dispatch_epi<bf16, false, false>(g, kind, e, split_ws, tile, st);
    return dispatch_epi<float, false, false>(g, kind, e, nullptr, tile, st);
}

}  // namespace tpk
