// Instantiations of the block's elementwise kernels (RMSNorm, conv + SiLU, conv history, conv step).
#include "selscan_block.h"

namespace selscan {

hipError_t launch_block_op(const LaunchBlockOps& p) {
    return p.bf16 ? launch_block_kernels_t<uint16_t>(p) : launch_block_kernels_t<float>(p);
}

}  // namespace selscan
