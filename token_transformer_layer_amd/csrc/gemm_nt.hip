// Product kernels of one operand layout (forward products: both operands K-contiguous).
#include "gemm_kernels.h"

namespace tpk {

hipError_t gemm_layout_nt(bool is_bf16, const GemmArgs &g, Epi kind, const EpiArgs &e, float *split_ws, Tile tile,
                          hipStream_t st) {
    if (is_bf16) return dispatch_epi<bf16, true, true>(g, kind, e, split_ws, tile, st);
    return dispatch_epi<float, true, true>(g, kind, e, nullptr, tile, st);
}

}  // namespace tpk
