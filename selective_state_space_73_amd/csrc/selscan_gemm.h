// Dense projections of the Mamba block on the matrix cores: Y[M, Nout] = X[M, K] W[Nout, K]^T
// (+ R[M, Nout]), all row-major, fp32 accumulation (bembew.net "Overview of Mamba (SSM) Model",
// "How the Mamba Block Works": the input and output projections and the small step-size,
// B and C projections; ai360xpert.com "Mamba", "The selection mechanism").
//
// Both operands are contiguous along K, so a workgroup stages a TILE x BK tile of X and of W
// in LDS (16-byte row chunks, double buffered) and each of its four waves multiplies a
// TILE/2 x TILE/2 block of Y as MFMA tiles of 32 x 32 (2 x 2 of them for TILE = 128, one for
// TILE = 64, the size taken when the larger tiles would leave the GPU short of workgroups):
// v_mfma_f32_32x32x16_bf16 for bf16 (8 consecutive k per lane and half-wave) and
// v_mfma_f32_32x32x2_f32 for fp32. Lane l of a 32 x 32 result holds column l % 32 and rows
// 8 (v / 4) + 4 (l / 32) + v % 4, v = 0..15. Edges (M, Nout, K not multiples of the tile)
// are zero-filled on load and masked on store.
#pragma once
#include "selscan_device.h"

namespace selscan {

constexpr int kGemmThreads = 256;
constexpr int kGemmFillGroups = 512;     // below this many 128-tiles, use 64-tiles

typedef __bf16 gemm_bf16x8 __attribute__((ext_vector_type(8)));
typedef float gemm_f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t gemm_u32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct GemmCfg;
template <> struct GemmCfg<uint16_t> {    // bf16: 32 k per tile, 8 per 16-byte chunk
    static constexpr int BK = 32, KV = 8, PAD = 8;
};
template <> struct GemmCfg<float> {       // fp32: 16 k per tile, 4 per 16-byte chunk
    static constexpr int BK = 16, KV = 4, PAD = 4;
};

// VEC: K is a multiple of KV and the row starts are 16-byte aligned, so whole chunks
// are loaded with one 16-byte access (else element by element).
template <typename T, bool RES, bool VEC, int TILE>
__global__ void __launch_bounds__(kGemmThreads)
k_gemm(const T* __restrict__ X, const T* __restrict__ W, const T* Rsd, T* Y, int64_t M, int64_t Nout, int64_t K) {
    using C = GemmCfg<T>;
    constexpr int BK = C::BK, KV = C::KV, LD = BK + C::PAD;       // LDS row stride in elements
    constexpr int CPR = BK / KV;                                   // 16-byte chunks per tile row
    constexpr int CH = TILE * CPR / kGemmThreads;                  // chunks per thread per operand
    constexpr int NT = TILE / 64;                                  // 32 x 32 MFMA tiles per wave and dimension
    constexpr int HW = TILE / 2;                                   // rows and columns per wave
    static_assert((TILE == 64 || TILE == 128) && CH * kGemmThreads == TILE * CPR, "tile shape");
    __shared__ __attribute__((aligned(16))) T sX[2][TILE][LD];
    __shared__ __attribute__((aligned(16))) T sW[2][TILE][LD];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;                       // this wave's HW x HW block
    const int64_t m0 = (int64_t)blockIdx.y * TILE, n0 = (int64_t)blockIdx.x * TILE;

    gemm_u32x4 rx[CH], rw[CH];                                     // one tile of each operand in flight
    auto fetch = [&](const T* P, int64_t r0, int64_t rows, int64_t k0, gemm_u32x4* reg) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int idx = tid + i * kGemmThreads;
            const int r = idx / CPR, kc = (idx % CPR) * KV;
            const int64_t gr = r0 + r, gk = k0 + kc;
            if (VEC) {
                reg[i] = (gr < rows && gk < K) ? *reinterpret_cast<const gemm_u32x4*>(P + gr * K + gk)
                                               : gemm_u32x4{0u, 0u, 0u, 0u};
            } else {
                T v[KV];
#pragma unroll
                for (int j = 0; j < KV; ++j) v[j] = (gr < rows && gk + j < K) ? P[gr * K + gk + j] : T(0);
                reg[i] = __builtin_bit_cast(gemm_u32x4, v);
            }
        }
    };
    auto stash = [&](T (*S)[LD], const gemm_u32x4* reg) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int idx = tid + i * kGemmThreads;
            *reinterpret_cast<gemm_u32x4*>(&S[idx / CPR][(idx % CPR) * KV]) = reg[i];
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
    const int64_t nk = (K + BK - 1) / BK;
    fetch(X, m0, M, 0, rx);
    fetch(W, n0, Nout, 0, rw);
    stash(sX[0], rx);
    stash(sW[0], rw);
    __syncthreads();
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int buf = (int)(kt & 1);
        const bool more = kt + 1 < nk;
        if (more) {
            fetch(X, m0, M, (kt + 1) * BK, rx);
            fetch(W, n0, Nout, (kt + 1) * BK, rw);
        }
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int ks = 0; ks < BK; ks += 16) {
                gemm_bf16x8 fa[NT], fb[NT];
#pragma unroll
                for (int a = 0; a < NT; ++a)
                    fa[a] = *reinterpret_cast<const gemm_bf16x8*>(&sX[buf][wm * HW + a * 32 + l32][ks + 8 * half]);
#pragma unroll
                for (int b = 0; b < NT; ++b)
                    fb[b] = *reinterpret_cast<const gemm_bf16x8*>(&sW[buf][wn * HW + b * 32 + l32][ks + 8 * half]);
#pragma unroll
                for (int a = 0; a < NT; ++a)
#pragma unroll
                    for (int b = 0; b < NT; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
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
        if (more) {
            stash(sX[buf ^ 1], rx);
            stash(sW[buf ^ 1], rw);
        }
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
                    if (RES) val += IO<T>::ld(Rsd + m * Nout + n);
                    IO<T>::st(Y + m * Nout + n, val);
                }
            }
        }
}

template <typename T, int TILE>
static void launch_gemm_tile(const LaunchGemm& p, bool vec, hipStream_t st) {
    const dim3 grid((unsigned)((p.N + TILE - 1) / TILE), (unsigned)((p.M + TILE - 1) / TILE));
    const T* X = static_cast<const T*>(p.X);
    const T* W = static_cast<const T*>(p.W);
    const T* R = static_cast<const T*>(p.R);
    T* Y = static_cast<T*>(p.Y);
    if (vec) {
        if (R) hipLaunchKernelGGL((k_gemm<T, true, true, TILE>), grid, dim3(kGemmThreads), 0, st, X, W, R, Y, p.M, p.N, p.K);
        else hipLaunchKernelGGL((k_gemm<T, false, true, TILE>), grid, dim3(kGemmThreads), 0, st, X, W, R, Y, p.M, p.N, p.K);
    } else {
        if (R) hipLaunchKernelGGL((k_gemm<T, true, false, TILE>), grid, dim3(kGemmThreads), 0, st, X, W, R, Y, p.M, p.N, p.K);
        else hipLaunchKernelGGL((k_gemm<T, false, false, TILE>), grid, dim3(kGemmThreads), 0, st, X, W, R, Y, p.M, p.N, p.K);
    }
}

template <typename T>
static hipError_t launch_gemm_t(const LaunchGemm& p) {
    hipStream_t st = static_cast<hipStream_t>(p.stream);
    const bool vec = p.K % GemmCfg<T>::KV == 0 && ((uintptr_t)p.X & 15u) == 0 && ((uintptr_t)p.W & 15u) == 0;
    const int64_t tiles128 = ((p.N + 127) / 128) * ((p.M + 127) / 128);
    if (tiles128 < kGemmFillGroups) launch_gemm_tile<T, 64>(p, vec, st);
    else launch_gemm_tile<T, 128>(p, vec, st);
    return hipGetLastError();
}

}  // namespace selscan
