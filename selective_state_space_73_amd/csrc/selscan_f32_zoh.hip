// Kernel instantiations of libselscan: fp32 I/O, zero-order-hold write term; forward scan and decode step.
#include "selscan_device.h"

namespace selscan {

hipError_t launch_f32_zoh(const LaunchScan& p, bool step) { return dispatch_n<float, true>(p, step); }

}  // namespace selscan
