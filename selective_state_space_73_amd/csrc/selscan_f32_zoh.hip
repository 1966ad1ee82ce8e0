// Kernel instantiations of libselscan: fp32 I/O, zero-order-hold write term; forward and backward.
#include "selscan_device.h"
#include "selscan_bwd.h"

namespace selscan {

hipError_t launch_f32_zoh(const LaunchScan& p, bool step) { return dispatch_n<float, true>(p, step); }

hipError_t launch_bwd_f32_zoh(const LaunchBwd& p) { return dispatch_bwd<float, true>(p); }

}  // namespace selscan
