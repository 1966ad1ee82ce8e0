// Kernel instantiations of libselscan: fp32 I/O, Euler write term; backward (in a unit of
// its own so that it compiles in parallel with the forward).
#include "selscan_bwd.h"

namespace selscan {

hipError_t launch_bwd_f32_euler(const LaunchBwd& p) { return dispatch_bwd<float, false>(p); }

}  // namespace selscan
