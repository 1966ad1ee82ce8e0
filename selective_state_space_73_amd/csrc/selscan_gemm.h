// Dense projections of the Mamba block on the matrix cores: Y[M, Nout] = X[M, K] W[Nout, K]^T
// (+ R[M, Nout]), all row-major, fp32 accumulation (bembew.net "Overview of Mamba (SSM) Model",
// "How the Mamba Block Works": the input and output projections and the small step-size,
// B and C projections; ai360xpert.com "Mamba", "The selection mechanism").
//
// The activations X are fp32 (the block keeps every activation between its steps in
// fp32); the weights W have the block's I/O dtype. With bf16 weights each fp32 activation
// is split into two bf16 terms, x = hi + lo (hi = bf16(x), lo = bf16(x - hi), 16
// significant bits together), and both are multiplied by the bf16 weights on the matrix
// cores: the products are exact in fp32 and the projection carries the activation to
// about 2^-17 relative instead of the 2^-9 of one bf16 rounding, at twice the MFMA work.
// With fp32 weights X and W go to the fp32 MFMA directly.
//
// Both operands are contiguous along K, so a workgroup stages a TILE x BK tile of X and of W
// in LDS (16-byte row chunks, double buffered; X as its hi and lo bf16 tiles when W is
// bf16) and each of its four waves multiplies a TILE/2 x TILE/2 block of Y as MFMA tiles of
// 32 x 32 (2 x 2 of them for TILE = 128, one for TILE = 64, the size taken when the larger
// tiles would leave the GPU short of workgroups; the 64-wide tiles take twice the K depth
// per stage, so a short grid waits on half as many load round trips):
// v_mfma_f32_32x32x16_bf16 for bf16 (8 consecutive k per lane and half-wave) and
// v_mfma_f32_32x32x2_f32 for fp32. Lane l of a 32 x 32 result holds column l % 32 and rows
// 8 (v / 4) + 4 (l / 32) + v % 4, v = 0..15. Edges (M, Nout, K not multiples of the tile)
// are zero-filled on load and masked on store. Y (and the residual R) is fp32 or bf16 (TY).
//
// Output columns can be routed to up to three matrices (the block's fused projections:
// in_proj into the main branch and the gate, x_proj into the step-size rank, B and C).
// A grid short of workgroups splits K (gemm_plan): split s multiplies its K range and
// writes fp32 partials, and k_gemm_reduce sums the splits in order (deterministic), adds
// the residual and stores in TY.
#pragma once
#include "selscan_device.h"

namespace selscan {

constexpr int kGemmThreads = 256;

typedef __bf16 gemm_bf16x8 __attribute__((ext_vector_type(8)));
typedef float gemm_f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t gemm_u32x4 __attribute__((ext_vector_type(4)));
typedef float gemm_f32x4 __attribute__((ext_vector_type(4)));

template <typename TW, int TILE> struct GemmCfg;
template <int TILE> struct GemmCfg<uint16_t, TILE> {    // bf16 weights: 8 k per 16-byte chunk
    static constexpr int BK = TILE == 64 ? 64 : 32, KV = 8, PAD = 8;
};
template <int TILE> struct GemmCfg<float, TILE> {       // fp32: 4 k per 16-byte chunk
    static constexpr int BK = TILE == 64 ? 32 : 16, KV = 4, PAD = 4;
};

// Destination of output column n (< Nout) of row m: three row-major matrices side by side.
struct GemmOut {
    void* y0; void* y1; void* y2;
    int64_t c0, c1, c2;
};
template <typename T>
__device__ __forceinline__ T* gemm_dst(const GemmOut& o, int64_t m, int64_t n) {
    if (n < o.c0) return static_cast<T*>(o.y0) + m * o.c0 + n;
    n -= o.c0;
    if (n < o.c1) return static_cast<T*>(o.y1) + m * o.c1 + n;
    return static_cast<T*>(o.y2) + m * o.c2 + (n - o.c1);
}

// VEC: K is a multiple of KV and the row starts are 16-byte aligned, so whole chunks
// are loaded with 16-byte accesses (else element by element). PART: write the fp32
// partial of K split blockIdx.z (K range [z kper, (z + 1) kper)) to part[z, M, Nout].
template <typename TW, typename TY, bool RES, bool VEC, int TILE, bool PART>
__global__ void __launch_bounds__(kGemmThreads)
k_gemm(const float* __restrict__ X, const TW* __restrict__ W, const TY* Rsd, GemmOut out, float* __restrict__ part,
       int64_t M, int64_t Nout, int64_t K, int64_t kper) {
    constexpr bool SPLIT = sizeof(TW) == 2;                        // bf16 weights: X as hi + lo
    using C = GemmCfg<TW, TILE>;
    constexpr int BK = C::BK, KV = C::KV, LD = BK + C::PAD;       // LDS row stride in elements
    constexpr int CPR = BK / KV;                                   // chunks per tile row
    constexpr int CH = TILE * CPR / kGemmThreads;                  // chunks per thread per operand
    constexpr int NT = TILE / 64;                                  // 32 x 32 MFMA tiles per wave and dimension
    constexpr int HW = TILE / 2;                                   // rows and columns per wave
    static_assert((TILE == 64 || TILE == 128) && CH * kGemmThreads == TILE * CPR, "tile shape");
    __shared__ __attribute__((aligned(16))) TW sX[2][TILE][LD];            // X (fp32), or its hi terms
    __shared__ __attribute__((aligned(16))) TW sXl[SPLIT ? 2 : 1][SPLIT ? TILE : 1][SPLIT ? LD : 1];   // lo terms
    __shared__ __attribute__((aligned(16))) TW sW[2][TILE][LD];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;                       // this wave's HW x HW block
    const int64_t m0 = (int64_t)blockIdx.y * TILE, n0 = (int64_t)blockIdx.x * TILE;

    float rx[CH][KV];                                              // X chunks in flight (fp32)
    gemm_u32x4 rw[CH];                                             // W chunks in flight
    auto fetch_x = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int idx = tid + i * kGemmThreads;
            const int r = idx / CPR, kc = (idx % CPR) * KV;
            const int64_t gr = m0 + r, gk = k0 + kc;
            if (VEC) {
#pragma unroll
                for (int q = 0; q < KV / 4; ++q) {
                    const gemm_f32x4 v = (gr < M && gk < K) ? *reinterpret_cast<const gemm_f32x4*>(X + gr * K + gk + 4 * q)
                                                            : gemm_f32x4{0.f, 0.f, 0.f, 0.f};
                    rx[i][4 * q] = v.x; rx[i][4 * q + 1] = v.y; rx[i][4 * q + 2] = v.z; rx[i][4 * q + 3] = v.w;
                }
            } else {
#pragma unroll
                for (int j = 0; j < KV; ++j) rx[i][j] = (gr < M && gk + j < K) ? X[gr * K + gk + j] : 0.0f;
            }
        }
    };
    auto fetch_w = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int idx = tid + i * kGemmThreads;
            const int r = idx / CPR, kc = (idx % CPR) * KV;
            const int64_t gr = n0 + r, gk = k0 + kc;
            if (VEC) {
                rw[i] = (gr < Nout && gk < K) ? *reinterpret_cast<const gemm_u32x4*>(W + gr * K + gk)
                                              : gemm_u32x4{0u, 0u, 0u, 0u};
            } else {
                TW v[KV];
#pragma unroll
                for (int j = 0; j < KV; ++j) v[j] = (gr < Nout && gk + j < K) ? W[gr * K + gk + j] : TW(0);
                rw[i] = __builtin_bit_cast(gemm_u32x4, v);
            }
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int idx = tid + i * kGemmThreads;
            const int r = idx / CPR, kc = (idx % CPR) * KV;
            *reinterpret_cast<gemm_u32x4*>(&sW[buf][r][kc]) = rw[i];
            if constexpr (SPLIT) {
                uint16_t hi[KV], lo[KV];
#pragma unroll
                for (int j = 0; j < KV; ++j) {
                    hi[j] = IO<uint16_t>::bits(rx[i][j]);
                    lo[j] = IO<uint16_t>::bits(rx[i][j] - IO<uint16_t>::cvt(hi[j]));
                }
                *reinterpret_cast<gemm_u32x4*>(&sX[buf][r][kc]) = __builtin_bit_cast(gemm_u32x4, hi);
                *reinterpret_cast<gemm_u32x4*>(&sXl[buf][r][kc]) = __builtin_bit_cast(gemm_u32x4, lo);
            } else {
                *reinterpret_cast<gemm_u32x4*>(&sX[buf][r][kc]) = __builtin_bit_cast(gemm_u32x4, rx[i]);
            }
        }
    };

    gemm_f32x16 acc[NT][NT];
#pragma unroll
    for (int a = 0; a < NT; ++a)
#pragma unroll
        for (int b = 0; b < NT; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

    const int l32 = lane & 31, half = lane >> 5;
    // this workgroup's K stages: [kt0, kt1) (every split is non-empty: gemm_plan)
    const int64_t kall = (K + BK - 1) / BK;
    const int64_t kt0 = PART ? (int64_t)blockIdx.z * (kper / BK) : 0;
    const int64_t kt1 = PART ? (kt0 + kper / BK < kall ? kt0 + kper / BK : kall) : kall;
    fetch_x(kt0 * BK);
    fetch_w(kt0 * BK);
    stash(0);
    __syncthreads();
    for (int64_t kt = kt0; kt < kt1; ++kt) {
        const int buf = (int)((kt - kt0) & 1);
        const bool more = kt + 1 < kt1;
        if (more) {
            fetch_x((kt + 1) * BK);
            fetch_w((kt + 1) * BK);
        }
        if constexpr (SPLIT) {
#pragma unroll
            for (int ks = 0; ks < BK; ks += 16) {
                gemm_bf16x8 fh[NT], fl[NT], fb[NT];
#pragma unroll
                for (int a = 0; a < NT; ++a) {
                    fh[a] = *reinterpret_cast<const gemm_bf16x8*>(&sX[buf][wm * HW + a * 32 + l32][ks + 8 * half]);
                    fl[a] = *reinterpret_cast<const gemm_bf16x8*>(&sXl[buf][wm * HW + a * 32 + l32][ks + 8 * half]);
                }
#pragma unroll
                for (int b = 0; b < NT; ++b)
                    fb[b] = *reinterpret_cast<const gemm_bf16x8*>(&sW[buf][wn * HW + b * 32 + l32][ks + 8 * half]);
#pragma unroll
                for (int a = 0; a < NT; ++a)
#pragma unroll
                    for (int b = 0; b < NT; ++b) {
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fh[a], fb[b], acc[a][b], 0, 0, 0);
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fl[a], fb[b], acc[a][b], 0, 0, 0);
                    }
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < BK; ks += 2) {
                float fa[NT], fb[NT];
#pragma unroll
                for (int a = 0; a < NT; ++a) fa[a] = sX[buf][wm * HW + a * 32 + l32][ks + half];
#pragma unroll
                for (int b = 0; b < NT; ++b) fb[b] = sW[buf][wn * HW + b * 32 + l32][ks + half];
#pragma unroll
                for (int a = 0; a < NT; ++a)
#pragma unroll
                    for (int b = 0; b < NT; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[a], fb[b], acc[a][b], 0, 0, 0);
            }
        }
        if (more) stash(buf ^ 1);
        __syncthreads();
    }

    // epilogue: lane holds column l32 and rows 8 (v / 4) + 4 half + v % 4 of each 32 x 32 tile
#pragma unroll
    for (int a = 0; a < NT; ++a)
#pragma unroll
        for (int b = 0; b < NT; ++b) {
            const int64_t n = n0 + wn * HW + b * 32 + l32;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t m = m0 + wm * HW + a * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
                if (m < M && n < Nout) {
                    float val = acc[a][b][v];
                    if (PART) {
                        part[((int64_t)blockIdx.z * M + m) * Nout + n] = val;
                    } else {
                        if (RES) val += IO<TY>::ld(Rsd + m * Nout + n);
                        IO<TY>::st(gemm_dst<TY>(out, m, n), val);
                    }
                }
            }
        }
}

// Sum of the K splits' fp32 partials in split order (+ residual), stored as TY.
template <typename TY, bool RES>
__global__ void __launch_bounds__(256)
k_gemm_reduce(const float* __restrict__ part, int splits, const TY* Rsd, GemmOut out, int64_t M, int64_t Nout) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = M * Nout;
    if (i >= total) return;
    float v = part[i];
    for (int s = 1; s < splits; ++s) v += part[(int64_t)s * total + i];
    if (RES) v += IO<TY>::ld(Rsd + i);
    IO<TY>::st(gemm_dst<TY>(out, i / Nout, i % Nout), v);
}

template <typename TW, typename TY, int TILE, bool PART>
static void launch_gemm_tile(const LaunchGemm& p, const GemmPlan& g, bool vec, const GemmOut& o, hipStream_t st) {
    const dim3 grid((unsigned)((p.N + TILE - 1) / TILE), (unsigned)((p.M + TILE - 1) / TILE), (unsigned)g.splits);
    const float* X = static_cast<const float*>(p.X);
    const TW* W = static_cast<const TW*>(p.W);
    const TY* R = static_cast<const TY*>(p.R);
    // a split launch adds the residual in k_gemm_reduce
    const bool res = !PART && R != nullptr;
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, grid, dim3(kGemmThreads), 0, st, X, W, R, o, p.part, p.M, p.N, p.K, g.kper);
    };
    if constexpr (PART) {
        if (vec) go(k_gemm<TW, TY, false, true, TILE, true>);
        else go(k_gemm<TW, TY, false, false, TILE, true>);
    } else {
        if (vec) res ? go(k_gemm<TW, TY, true, true, TILE, false>) : go(k_gemm<TW, TY, false, true, TILE, false>);
        else res ? go(k_gemm<TW, TY, true, false, TILE, false>) : go(k_gemm<TW, TY, false, false, TILE, false>);
    }
}

template <typename TW, typename TY>
static hipError_t launch_gemm_t(const LaunchGemm& p) {
    hipStream_t st = static_cast<hipStream_t>(p.stream);
    const bool vec = p.K % GemmCfg<TW, 64>::KV == 0 && ((uintptr_t)p.X & 15u) == 0 && ((uintptr_t)p.W & 15u) == 0;
    const GemmPlan g = gemm_plan(p.M, p.N, p.K, sizeof(TW) == 2);
    if (g.bk != (g.tile == 64 ? GemmCfg<TW, 64>::BK : GemmCfg<TW, 128>::BK)) return hipErrorInvalidValue;
    if (g.splits > 1 && !p.part) return hipErrorInvalidValue;
    const GemmOut o{p.Y[0], p.Y[1], p.Y[2], p.cols[0], p.cols[1], p.N - p.cols[0] - p.cols[1]};
    if (g.splits > 1) {
        if (g.tile == 64) launch_gemm_tile<TW, TY, 64, true>(p, g, vec, o, st);
        else launch_gemm_tile<TW, TY, 128, true>(p, g, vec, o, st);
        const int64_t total = p.M * p.N;
        const dim3 rg((unsigned)((total + 255) / 256));
        const TY* R = static_cast<const TY*>(p.R);
        if (R) hipLaunchKernelGGL((k_gemm_reduce<TY, true>), rg, dim3(256), 0, st, p.part, g.splits, R, o, p.M, p.N);
        else hipLaunchKernelGGL((k_gemm_reduce<TY, false>), rg, dim3(256), 0, st, p.part, g.splits, R, o, p.M, p.N);
    } else {
        if (g.tile == 64) launch_gemm_tile<TW, TY, 64, false>(p, g, vec, o, st);
        else launch_gemm_tile<TW, TY, 128, false>(p, g, vec, o, st);
    }
    return hipGetLastError();
}

}  // namespace selscan
