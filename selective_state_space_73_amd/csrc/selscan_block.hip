// Instantiations of the block's kernels: RMSNorm, conv + SiLU, conv history, conv step
// and the projections' GEMM.
#include "selscan_block.h"
#include "selscan_gemm.h"

namespace selscan {

hipError_t launch_block_op(const LaunchBlockOps& p) {
    return p.bf16 ? launch_block_kernels_t<uint16_t>(p) : launch_block_kernels_t<float>(p);
}

hipError_t launch_gemm(const LaunchGemm& p) {
    if (!p.bf16) return p.y_bf16 ? hipErrorInvalidValue : launch_gemm_t<float, float>(p);
    return p.y_bf16 ? launch_gemm_t<uint16_t, uint16_t>(p) : launch_gemm_t<uint16_t, float>(p);
}

}  // namespace selscan
