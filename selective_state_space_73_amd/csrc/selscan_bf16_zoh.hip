// Kernel instantiations of libselscan: bfloat16 I/O, zero-order-hold write term; forward and backward.
#include "selscan_device.h"
#include "selscan_bwd.h"

namespace selscan {

hipError_t launch_bf16_zoh(const LaunchScan& p, bool step) { return dispatch_n<uint16_t, true>(p, step); }

hipError_t launch_bwd_bf16_zoh(const LaunchBwd& p) { return dispatch_bwd<uint16_t, true>(p); }

}  // namespace selscan
