// libselscan_probes: calibration kernels of the benchmark (see include/selscan_probes.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "selscan_probes.h"

namespace {

typedef float vf4 __attribute__((ext_vector_type(4)));

constexpr int kRmwThreads = 256;
constexpr int kRmwPerLane = 4;             // 16-byte accesses per lane (64 bytes)

// Lane l of workgroup g owns vf4 elements g*1024 + k*256 + l, k = 0..3: each of a wave's
// four loads is one contiguous 1 KiB run. All loads are issued before any store.
__global__ void __launch_bounds__(kRmwThreads) k_rmw(vf4* __restrict__ p, int64_t n4) {
    const int64_t base = (int64_t)blockIdx.x * (kRmwThreads * kRmwPerLane) + threadIdx.x;
    vf4 v[kRmwPerLane];
#pragma unroll
    for (int k = 0; k < kRmwPerLane; ++k) {
        const int64_t i = base + (int64_t)k * kRmwThreads;
        v[k] = i < n4 ? __builtin_nontemporal_load(p + i) : vf4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int k = 0; k < kRmwPerLane; ++k) {
        const int64_t i = base + (int64_t)k * kRmwThreads;
        const vf4 r = v[k] * 0.5f + 1.0f;
        if (i < n4) __builtin_nontemporal_store(r, p + i);
    }
}

constexpr int kIssueGroups = 2048;
constexpr int kIssueThreads = 256;
constexpr int kChains = SSP_ISSUE_CHAINS;

// MODE 0: K fmas per chain and iteration; 1: one exponential; 2: one exponential and K fmas.
// The exponential is 2^-a (v_exp_f32 with a negated input), whose iterates stay near 0.64;
// the fma chain b <- b * 0.9999 + 1e-4 stays near 1.
template <int MODE, int K>
__global__ void __launch_bounds__(kIssueThreads) k_issue(float* __restrict__ out, int64_t iters) {
    float a[kChains], b[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) {
        a[j] = 0.5f + 0.01f * (float)j + 1e-4f * (float)(threadIdx.x & 63);
        b[j] = 1.0f - 0.01f * (float)j;
    }
    for (int64_t it = 0; it < iters; it += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int j = 0; j < kChains; ++j) {
                if constexpr (MODE >= 1) a[j] = __builtin_amdgcn_exp2f(-a[j]);
                if constexpr (MODE != 1) {
#pragma unroll
                    for (int k = 0; k < K; ++k) b[j] = __builtin_fmaf(b[j], 0.9999f, 1e-4f);
                }
            }
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kChains; ++j) s += a[j] + b[j];
    out[(int64_t)blockIdx.x * kIssueThreads + threadIdx.x] = s;
}

template <int MODE, int K>
hipError_t launch_issue(float* out, int64_t iters, hipStream_t st) {
    hipLaunchKernelGGL((k_issue<MODE, K>), dim3(kIssueGroups), dim3(kIssueThreads), 0, st, out, iters);
    return hipGetLastError();
}

template <int MODE>
hipError_t issue_k(float* out, int64_t iters, int kfma, hipStream_t st) {
    switch (kfma) {
        case 1: return launch_issue<MODE, 1>(out, iters, st);
        case 3: return launch_issue<MODE, 3>(out, iters, st);
        case 7: return launch_issue<MODE, 7>(out, iters, st);
        case 8: return launch_issue<MODE, 8>(out, iters, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

extern "C" int ssp_rmw(float* buf, size_t n_floats, void* stream) {
    if (!buf || n_floats == 0 || (n_floats % 16) != 0 || ((uintptr_t)buf & 15u)) return (int)hipErrorInvalidValue;
    const int64_t n4 = (int64_t)(n_floats / 4);
    const int64_t per_group = kRmwThreads * kRmwPerLane;
    const int64_t groups = (n4 + per_group - 1) / per_group;
    if (groups > INT32_MAX) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(k_rmw, dim3((unsigned)groups), dim3(kRmwThreads), 0, static_cast<hipStream_t>(stream),
                       reinterpret_cast<vf4*>(buf), n4);
    return (int)hipGetLastError();
}

extern "C" int ssp_issue(float* out, int64_t iters, int mode, int kfma, void* stream) {
    if (!out || iters < 4 || (iters % 4) != 0) return (int)hipErrorInvalidValue;
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (mode) {
        case 0: return (int)issue_k<0>(out, iters, kfma, st);
        case 1: return (int)launch_issue<1, 1>(out, iters, st);
        case 2: return (int)issue_k<2>(out, iters, kfma, st);
        default: return (int)hipErrorInvalidValue;
    }
}
