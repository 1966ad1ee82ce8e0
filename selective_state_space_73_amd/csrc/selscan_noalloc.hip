// ss_conv_scan_fwd_noalloc: the full-sequence forward with its workspace (chunk
// aggregates, summed step sizes, copies of the initial states) in a fixed device
// array of this library instead of caller-supplied memory, for callers that cannot
// allocate device memory (code under graph capture, allocation-free serving loops).
//
// The array lives in device memory of every GPU the library runs on, from the first
// use until the process ends. Its device address is looked up once per device, with
// that device current; host code only ever passes that address on (the array's own
// name in host code is a host-side stand-in, not device memory). Nothing in the
// workspace needs to start at zero: the aggregate pass writes every entry the main
// pass reads, in stream order. Calls that overlap in time on one GPU (different
// streams, no ordering between them) share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "selscan.h"
#include "selscan_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[SS_NOALLOC_MAX_WORKSPACE];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's scratch array (looked up on first use).
ss_status scratch_ptr(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return selscan::set_error(SS_ERR_HIP, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return selscan::set_error(SS_ERR_UNSUPPORTED, "device index above 63");
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            return selscan::set_error(SS_ERR_HIP, e != hipSuccess ? hipGetErrorString(e)
                                                                  : "scratch array has no device address");
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return SS_OK;
}

}  // namespace

extern "C" ss_status ss_conv_scan_fwd_noalloc(const ss_dims* dims, const ss_args* args, void* stream) {
    // the dims are validated first so that an unusable size is reported as such
    const ss_status s = selscan::validate_dims(dims, false);
    if (s != SS_OK) {
        ss_time_next_call(nullptr, nullptr, nullptr, nullptr);
        return s;
    }
    const size_t need = ss_workspace_bytes(dims);
    if (need > (size_t)SS_NOALLOC_MAX_WORKSPACE) {
        ss_time_next_call(nullptr, nullptr, nullptr, nullptr);
        char msg[160];
        snprintf(msg, sizeof(msg), "these dims need %zu bytes of workspace, above the %zu of the built-in array",
                 need, (size_t)SS_NOALLOC_MAX_WORKSPACE);
        return selscan::set_error(SS_ERR_WORKSPACE, msg);
    }
    void* ws = nullptr;
    if (need > 0) {
        const ss_status sp = scratch_ptr(&ws);
        if (sp != SS_OK) {
            ss_time_next_call(nullptr, nullptr, nullptr, nullptr);
            return sp;
        }
    }
    return ss_conv_scan_fwd(dims, args, ws, need, stream);
}
