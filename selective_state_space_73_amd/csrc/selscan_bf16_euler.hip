// Kernel instantiations of libselscan: bfloat16 I/O, Euler write term; forward and backward.
#include "selscan_device.h"
#include "selscan_bwd.h"

namespace selscan {

hipError_t launch_bf16_euler(const LaunchScan& p, bool step) { return dispatch_n<uint16_t, false>(p, step); }

hipError_t launch_bwd_bf16_euler(const LaunchBwd& p) { return dispatch_bwd<uint16_t, false>(p); }

}  // namespace selscan
