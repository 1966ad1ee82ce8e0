// Kernel instantiations of libselscan: fp32 I/O, Euler write term; forward scan and decode step.
#include "selscan_device.h"

namespace selscan {

hipError_t launch_f32_euler(const LaunchScan& p, bool step) { return dispatch_n<float, false>(p, step); }

}  // namespace selscan
