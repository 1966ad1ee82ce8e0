// Device kernels of the Mamba block around the scan (ss_block_fwd / ss_block_step):
// the RMSNorm in front of the block and the block's causal conv + SiLU, which is
// materialised here (as u) because the step-size, B and C projections read it
// (bembew.net "Overview of Mamba (SSM) Model", "How the Mamba Block Works";
// ozercemkelahmet.com "Mamba", "The block"). The projections are the GEMM of selscan_gemm.h and
// the scan is the library's own kernel, both launched from selscan_block.cpp. Every
// activation between the block's steps is fp32; only the block's input (read by the
// norm) has the I/O dtype.
#pragma once
#include "selscan_device.h"

namespace selscan {

// RMSNorm: out = x / sqrt(mean(x^2) + eps) * w, one wave per row of d_model values; x in
// the I/O dtype, out fp32.
template <typename T>
__global__ void __launch_bounds__(256)
k_rmsnorm(const T* __restrict__ x, const float* __restrict__ w, float* __restrict__ out, int64_t rows, int dm,
          float eps) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;                      // whole waves leave together
    const T* xr = x + row * dm;
    float ss = 0.0f;
    for (int i = lane; i < dm; i += 64) {
        const float v = IO<T>::ld(xr + i);
        ss = __builtin_fmaf(v, v, ss);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
    const float r = __builtin_amdgcn_rsqf(ss / (float)dm + eps);
    float* orow = out + row * dm;
    for (int i = lane; i < dm; i += 64) orow[i] = IO<T>::ld(xr + i) * r * w[i];
}

// Causal depthwise conv (width 4, tap 3 on the current token) + SiLU over a run of
// kBlockConvRun tokens per lane: u[b,t,d] = SiLU(cb + sum_k w_k xi[b,t-3+k,d]), with
// the initial history (oldest first) before token 0, or zeros. A lane loads its run and
// the three inputs before it at once (the runs overlap by three rows, re-read from
// cache), so short runs give the grid enough lanes to hide the load latency. Token runs
// beyond the grid's y extent are taken in a strided loop. Reads the history only;
// k_conv_history writes the new one afterwards.
constexpr int kBlockConvRun = 8;
constexpr int64_t kBlockConvMaxGridY = 65535;

__global__ void __launch_bounds__(256)
k_conv_silu(const float* __restrict__ xi, const float* __restrict__ conv_w, const float* __restrict__ conv_b,
            const float* __restrict__ hist, float* __restrict__ u, int64_t L, int D) {
    const int d = blockIdx.x * 256 + threadIdx.x;
    if (d >= D) return;
    const int b = blockIdx.z;
    const float w0 = conv_w[d * 4 + 0], w1 = conv_w[d * 4 + 1], w2 = conv_w[d * 4 + 2], w3 = conv_w[d * 4 + 3];
    const float cb = conv_b ? conv_b[d] : 0.0f;
    const int64_t bd = (int64_t)b * D + d;
    const float* xb = xi + (int64_t)b * L * D + d;
    float* ub = u + (int64_t)b * L * D + d;
    const int64_t nrun = (L + kBlockConvRun - 1) / kBlockConvRun;
    for (int64_t run = blockIdx.y; run < nrun; run += gridDim.y) {
        const int64_t t0 = run * kBlockConvRun;
        float xv[kBlockConvRun + 3];
#pragma unroll
        for (int j = 0; j < kBlockConvRun + 3; ++j) {
            const int64_t t = t0 - 3 + j;
            xv[j] = t >= L ? 0.0f : (t >= 0 ? xb[t * D] : (hist ? hist[bd * 3 + (3 + t)] : 0.0f));
        }
#pragma unroll
        for (int j = 0; j < kBlockConvRun; ++j) {
            const int64_t t = t0 + j;
            const float c = __builtin_fmaf(w3, xv[j + 3], __builtin_fmaf(w2, xv[j + 2],
                            __builtin_fmaf(w1, xv[j + 1], __builtin_fmaf(w0, xv[j], cb))));
            if (t < L) ub[t * D] = silu(c);
        }
    }
}

// New conv history [B,D,3] = the last three of (history, xi) for every (b, d).
__global__ void __launch_bounds__(256)
k_conv_history(const float* __restrict__ xi, float* __restrict__ hist, int64_t L, int D, int Bsz) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)Bsz * D) return;
    const int d = (int)(i % D);
    const int64_t b = i / D;
    const float h0 = hist[i * 3 + 0], h1 = hist[i * 3 + 1], h2 = hist[i * 3 + 2];
    float n[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int64_t t = L - 3 + k;                 // sequence position of new entry k
        // before the sequence: old entry 3 + t (selects, not an indexed private array)
        n[k] = t >= 0 ? xi[(b * L + t) * D + d] : (t == -1 ? h2 : (t == -2 ? h1 : h0));
    }
    hist[i * 3 + 0] = n[0]; hist[i * 3 + 1] = n[1]; hist[i * 3 + 2] = n[2];
}

// Decode: one token per stream; u = SiLU(conv over (history, x)), history shifted in place.
__global__ void __launch_bounds__(256)
k_conv_step(const float* __restrict__ xi, const float* __restrict__ conv_w, const float* __restrict__ conv_b,
            float* __restrict__ hist, float* __restrict__ u, int D, int S) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)S * D) return;
    const int d = (int)(i % D);
    const float xt = xi[i];
    const float h0 = hist[i * 3 + 0], h1 = hist[i * 3 + 1], h2 = hist[i * 3 + 2];
    const float cb = conv_b ? conv_b[d] : 0.0f;
    const float c = __builtin_fmaf(conv_w[d * 4 + 3], xt, __builtin_fmaf(conv_w[d * 4 + 2], h2,
                    __builtin_fmaf(conv_w[d * 4 + 1], h1, __builtin_fmaf(conv_w[d * 4 + 0], h0, cb))));
    u[i] = silu(c);
    hist[i * 3 + 0] = h1; hist[i * 3 + 1] = h2; hist[i * 3 + 2] = xt;
}

template <typename T>
static hipError_t launch_block_kernels_t(const LaunchBlockOps& p) {
    hipStream_t st = static_cast<hipStream_t>(p.stream);
    switch (p.op) {
        case LaunchBlockOps::kRmsNorm:
            hipLaunchKernelGGL((k_rmsnorm<T>), dim3((unsigned)((p.rows + 3) / 4)), dim3(256), 0, st,
                               static_cast<const T*>(p.in), p.w, static_cast<float*>(p.out), p.rows, p.cols, p.eps);
            break;
        case LaunchBlockOps::kConvSilu:
        {
            const int64_t runs = (p.L + kBlockConvRun - 1) / kBlockConvRun;
            hipLaunchKernelGGL(k_conv_silu, dim3((unsigned)((p.cols + 255) / 256),
                               (unsigned)(runs < kBlockConvMaxGridY ? runs : kBlockConvMaxGridY), (unsigned)p.batch),
                               dim3(256), 0, st, static_cast<const float*>(p.in), p.conv_w, p.conv_b, p.hist,
                               static_cast<float*>(p.out), p.L, p.cols);
        }
            break;
        case LaunchBlockOps::kConvHistory:
            hipLaunchKernelGGL(k_conv_history, dim3((unsigned)((p.batch * p.cols + 255) / 256)), dim3(256), 0, st,
                               static_cast<const float*>(p.in), p.hist, p.L, p.cols, (int)p.batch);
            break;
        case LaunchBlockOps::kConvStep:
            hipLaunchKernelGGL(k_conv_step, dim3((unsigned)((p.batch * p.cols + 255) / 256)), dim3(256), 0, st,
                               static_cast<const float*>(p.in), p.conv_w, p.conv_b, p.hist, static_cast<float*>(p.out),
                               p.cols, (int)p.batch);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace selscan
