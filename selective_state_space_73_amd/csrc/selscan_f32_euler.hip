// Kernel instantiations of libselscan: fp32 I/O, Euler write term; forward and backward.
#include "selscan_device.h"
#include "selscan_bwd.h"

namespace selscan {

hipError_t launch_f32_euler(const LaunchScan& p, bool step) { return dispatch_n<float, false>(p, step); }

hipError_t launch_bwd_f32_euler(const LaunchBwd& p) { return dispatch_bwd<float, false>(p); }

}  // namespace selscan
