// Kernel instantiations of libselscan: bfloat16 I/O, Euler write term; forward scan and decode step.
#include "selscan_device.h"

namespace selscan {

hipError_t launch_bf16_euler(const LaunchScan& p, bool step) { return dispatch_n<uint16_t, false>(p, step); }

}  // namespace selscan
