// Kernel instantiations of libselscan: bfloat16 I/O, zero-order-hold write term; forward scan and decode step.
#include "selscan_device.h"

namespace selscan {

hipError_t launch_bf16_zoh(const LaunchScan& p, bool step) { return dispatch_n<uint16_t, true>(p, step); }

}  // namespace selscan
