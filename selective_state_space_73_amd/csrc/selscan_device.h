// Device code of libselscan for gfx950 (CDNA4, wave64): the kernel templates and
// their launchers. Included by the instantiation units selscan_<io>_<rule>.hip,
// one per I/O dtype and discretisation rule, which compile in parallel.
//
// The selective scan (S6) forward path: causal depthwise conv1d + SiLU,
// softplus step size, exp(Delta A) decay, write term, readout C.h + D u, SiLU(z)
// gate (ai360xpert.com "Mamba", "The selection mechanism"; ozercemkelahmet.com
// "Mamba", "A minimal selective scan in PyTorch"; bembew.net "Overview of Mamba
// (SSM) Model", "How the Mamba Block Works"). The write term is either the Euler
// form Delta B u or the zero-order-hold form (exp(Delta A) - 1) / A * B u
// (inferensys.com "Mamba", the discretization bullet; ai360xpert.com "Mamba",
// the simplified ZOH line of its code section), selected by the ZOH template flag.
//
// Mapping: one lane owns one (batch row, channel) pair and keeps its N state
// values in VGPRs for a run of consecutive tokens (a chunk). Loads of x, delta,
// z and stores of y are coalesced along d. B_t and C_t are the same for every
// channel: each workgroup stages them through LDS in fp32 tiles and every wave
// reads them back as broadcasts. Grids with too few channels for that mapping use
// a lane quad per channel instead (k_agg_q / k_scan_q, further down).
//
// Long sequences with few channels are split into chunks so the grid fills the
// GPU. The recurrence h_t = a_t h_{t-1} + b_t is associative in the pair (a, b)
// (ai360xpert.com "Mamba", "Why this breaks the parallel form": the scan exploits
// associativity; ozercemkelahmet.com "Deployment notes": chunks pass the state).
// A chunk's end state from zero, S_c, and its summed step size give its total
// decay exp(A * sum Delta), and the carry-ins fold from them. Chunks of at least
// kCorrMinChunk tokens of the plain forward run from zero in the main pass, which
// records S_c; k_fold folds the carries and k_corr adds their decaying part to the
// outputs afterwards. Otherwise (shorter chunks, the bidirectional and backward
// passes) an aggregate pass computes S_c first and the main pass folds it into its
// exact carry-in.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "selscan_internal.h"

namespace selscan {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Zero-order hold: states with |A| below this take the coefficient's A -> 0 limit
// Delta (exact to fp32 there, and it keeps 1/A finite)
constexpr float kZohZeroA = 0x1p-100f;
// (exp(x) - 1) / x = 1 + x/2 + x^2/6 + x^3/24 + O(x^4), written in t = x log2(e)
constexpr float kPhi1 = 0.34657359027997264f;     // ln2 / 2
constexpr float kPhi2 = 0.08007550231970024f;     // ln2^2 / 6
constexpr float kPhi3 = 0.013876027166205393f;    // ln2^3 / 24
constexpr float kZohSeriesT = 0.14426950408889634f;   // |t| below this (|x| < 0.1): series

// ---------------------------------------------------------------------------
// elementwise pieces (fp32)

// compile-time flag passed to generic lambdas
template <bool B> struct Tag { static constexpr bool value = B; };

__device__ __forceinline__ float exp2_fast(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ float log2_fast(float v) { return __builtin_amdgcn_logf(v); }
__device__ __forceinline__ float rcp_fast(float v) { return __builtin_amdgcn_rcpf(v); }

// SiLU(v) = v / (1 + e^-v)
__device__ __forceinline__ float silu(float v) {
    return v * rcp_fast(1.0f + exp2_fast(-kLog2e * v));
}

// softplus(v) = max(v,0) + log1p(e^-|v|). log1p(e) is taken as log(1+e) plus the
// rounding error of 1+e, which keeps relative accuracy when e is small.
__device__ __forceinline__ float softplus(float v) {
    const float e = exp2_fast(-kLog2e * __builtin_fabsf(v));
    const float s = 1.0f + e;
    const float corr = e - (s - 1.0f);
    const float lp = __builtin_fmaf(log2_fast(s), kLn2, corr);
    return __builtin_fmaxf(v, 0.0f) + lp;
}

// (exp(x) - 1) / x for x = t ln2: the series below |x| = 0.1 (truncation < 1e-6),
// otherwise (a - 1) / x with a = 2^t. Computing a - 1 from an fp32 a loses about
// 6e-8 / |x| relative near x = 0, which the series avoids; at x = 0 it is 1.
__device__ __forceinline__ float phi_series(float t) {
    return __builtin_fmaf(t, __builtin_fmaf(t, __builtin_fmaf(t, kPhi3, kPhi2), kPhi1), 1.0f);
}

// Zero-order-hold write coefficient (exp(Delta A) - 1) / A from the decay a = 2^t,
// t = Delta A log2(e), and iA = 1/A (0 for the A = 0 states, which take the series).
__device__ __forceinline__ float zoh_coef(float a, float t, float dt, float iA) {
    const float big = __builtin_fmaf(a, iA, -iA);
    const float small = dt * phi_series(t);
    return __builtin_fabsf(t) < kZohSeriesT ? small : big;
}

// Runtime-checked fast path for A[d, n] = (n + 1) * A[d, 0] (the A = -(1..N)
// initialisation of ozercemkelahmet.com "Mamba", "A minimal selective scan in PyTorch",
// and the benchmark workloads): then exp(Delta A[d, n]) = exp(Delta A[d, 0])^(n+1), so
// one exponential and N - 1 multiplies give every state's decay. a_n carries about
// n + 1 roundings of a_0 plus n of its own, so state n's accumulated rounding is
// about (n + 1) eps min(M_n, T) for a memory of M_n = 1 / |A_n Delta| tokens over a
// run of T: at most eps / |A_0 Delta|, the bound of state 0 on either path, but up to
// N times the exponentials' own error where the memory outlasts the run (small
// |A_0 Delta| over short sequences). So the identity must hold with A[d, 0] = 0 (no
// decay, the chain is exact) or A[d, 0] <= -1/2 (memories of at most 2 / Delta
// tokens); other channels take the general decays. The kernels that take it are
// launched twice, with POW = false and true; each workgroup votes on the identity over
// its channels and runs in exactly one of the two launches (the other returns at
// once).
constexpr int kPowMinN = 8;              // below this the saved exponentials do not pay for a second launch
constexpr int kPowLanes = 4;             // interleaved multiply chains of the scan's per-token decays

// a[n] = a0^(n+1): squares for even exponents, one more factor of a0 for odd ones
template <int N>
__device__ __forceinline__ void pow_chain(float a0, float* a) {
    a[0] = a0;
#pragma unroll
    for (int n = 1; n < N; ++n) {
        const int p = n + 1;
        a[n] = (p % 2 == 0) ? a[p / 2 - 1] * a[p / 2 - 1] : a[n - 1] * a0;
    }
}

// true on this lane when A[d, n] == (n + 1) * A[d, 0] holds exactly in fp32 for every n
// and A[d, 0] is 0 or at most -1/2 (its own loads, not merged with the kernel's later
// loads of A, so that these raw values are not kept live)
constexpr float kPowMaxA0 = -0.5f;
template <int N>
__device__ __forceinline__ bool pow_structured(const float* Arow) {
    const float a0 = __builtin_nontemporal_load(Arow);
    bool ok = a0 == 0.0f || a0 <= kPowMaxA0;
#pragma unroll
    for (int n = 1; n < N; ++n) ok = ok && (__builtin_nontemporal_load(Arow + n) == (float)(n + 1) * a0);
    return ok;
}

// Workgroup vote of the power fast path, taken at the start of a kernel launched once
// with POW = false and once with POW = true: returns true when this workgroup belongs
// to the other launch and must exit (uniformly, before any other barrier).
template <int N, bool POW>
__device__ __forceinline__ bool pow_skip(const float* Arow) {
    if constexpr (N < kPowMinN) {
        return POW;                                  // only the general launch exists
    } else {
        // one flag per wave in LDS, one barrier, then every lane reads all of them
        static_assert(kScanThreads % 64 == 0 && kScanThreads / 64 <= 32, "one vote bit per wave");
        __shared__ uint32_t votes;
        const bool mine = __all(pow_structured<N>(Arow));
        if (threadIdx.x == 0) votes = 0;
        __syncthreads();
        if ((threadIdx.x & 63) == 0 && !mine) atomicOr(&votes, 1u);
        __syncthreads();
        const bool all = votes == 0;
        return all != POW;
    }
}

typedef float vf4 __attribute__((ext_vector_type(4)));

template <typename T> struct IO;
template <> struct IO<float> {
    static __device__ __forceinline__ float cvt(float v) { return v; }
    static __device__ __forceinline__ float bits(float v) { return v; }
    static __device__ __forceinline__ float ld(const float* p) { return *p; }
    static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};
template <> struct IO<uint16_t> {   // bfloat16 bits
    static __device__ __forceinline__ float cvt(uint16_t v) {
        return __builtin_bit_cast(float, static_cast<uint32_t>(v) << 16);
    }
    static __device__ __forceinline__ float ld(const uint16_t* p) {
        return __builtin_bit_cast(float, static_cast<uint32_t>(*p) << 16);
    }
    static __device__ __forceinline__ void st(uint16_t* p, float v) { *p = bits(v); }
    static __device__ __forceinline__ uint16_t bits(float v) {
        return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));   // round to nearest even
    }
};

// Raw buffer access: a uniform base (SGPR resource), a 32-bit per-lane byte offset
// and a uniform byte offset, so the per-token addressing needs no 64-bit VALU
// arithmetic. Offsets stay below 2^32 (d_inner <= 2^26 is checked on the host).
constexpr int kBufDword3 = 0x00020000;            // raw buffer, 32-bit data format (gfx9 family)

template <typename T> struct Buf;
template <> struct Buf<uint16_t> {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ explicit Buf(const uint16_t* p)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), 0, -1, kBufDword3)) {}
    __device__ __forceinline__ uint16_t ld(unsigned voff, unsigned soff) const {
        return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
    }
    __device__ __forceinline__ void st(uint16_t v, unsigned voff, unsigned soff) const {
        __builtin_amdgcn_raw_buffer_store_b16(v, r, voff, soff, 0);
    }
};
template <> struct Buf<float> {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ explicit Buf(const float* p)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), 0, -1, kBufDword3)) {}
    __device__ __forceinline__ float ld(unsigned voff, unsigned soff) const {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
    }
    __device__ __forceinline__ void st(float v, unsigned voff, unsigned soff) const {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, voff, soff, 0);
    }
};

// ---------------------------------------------------------------------------
// The main pass: full forward over one chunk with outputs, from the chunk's exact
// initial state (the caller's state for chunk 0, else the carry folded from the
// aggregates of the earlier chunks). CK = true: checkpoint mode, no readout and no
// outputs, the state written every kCkptEvery tokens instead, states left untouched.

struct ScanArgs {
    int64_t L;            // sequence length
    int64_t chunk_len;    // tokens per chunk (a multiple of kScanTile when nchunks > 1)
    int D;                // channels
    int nchunks;
    int64_t nck;          // checkpoint slots per batch row (checkpoint mode): L / kCkptEvery
};

// Checkpoint mode of the main pass (used by the backward): the state after every
// kCkptEvery-th token is written to a [B, L / kCkptEvery, N/4, D, 4] buffer (four
// consecutive state entries per channel, channels consecutive, so each 16-byte
// store of a wave is contiguous), slot j holding the state after token
// kCkptEvery*j + kCkptEvery - 1.
constexpr int kCkptEvery = 4;

// Register budget of the scan kernel: three waves per SIMD (<= 168 VGPRs) for
// N <= 16, measured faster than the compiler's own choice (two waves at ~240
// VGPRs) because more resident waves hide the long per-token dependency chains;
// larger N needs the registers for the state and keeps one-wave-per-SIMD limits.
// (Without the conv the schedule under those caps spills, so it is left free; the
// zero-order hold's longer per-state chain with N more registers of 1/A, and the
// reversed pass's extra prefetched y, are held to two waves.)
template <int N, bool CONV, bool ZOH, bool CK, bool REV> constexpr int scan_waves_per_eu() {
    return (N > 16 || !CONV) ? 1 : (ZOH || CK || REV) ? 2 : 3;
}

// Zero-order hold: the write coefficient (exp(Delta A) - 1) / A comes from the decay
// already computed (zoh_coef: one fma, or a short series where Delta A is small).
// A bidirectional scan (ozercemkelahmet.com "Mamba", "Variants and extensions") runs
// two passes, neither with states in or out. PART: the forward pass, writing its
// gated output as fp32 to ypart [B, L, D] instead of y. REV: the same layer over the
// time-reversed sequence, so chunk-relative token r of chunk c is position
// L-1-(c*chunk_len + r); it adds its gated output to ypart's and writes the sum to y.
template <typename T, int N, bool CONV, bool GATE, bool ZOH, bool CK = false, bool REV = false, bool PART = false,
          bool POW = false, bool LOC = false>
__global__ void __launch_bounds__(kScanThreads) __attribute__((amdgpu_waves_per_eu(scan_waves_per_eu<N, CONV, ZOH, CK, REV>())))
k_scan(const T* __restrict__ x, const float* __restrict__ conv_w, const float* __restrict__ conv_b,
       const T* __restrict__ delta, const float* __restrict__ delta_bias, const float* __restrict__ A,
       const T* __restrict__ Bm, const T* __restrict__ Cm, const float* __restrict__ Dskip,
       const T* __restrict__ z, T* __restrict__ y,
       float* __restrict__ ssm_state,        // IN (nchunks == 1) and OUT (last chunk)
       float* __restrict__ conv_state,       // IN (nchunks == 1) and OUT (last chunk)
       float* __restrict__ ws_S,             // [B, nchunks-1, D, N] chunk end states (chunk 0 includes h0);
                                             // written by the plain forward as [B, nchunks, D, N]
       float* __restrict__ ws_sdt,           // [B, nchunks-1, D] summed step sizes (plain: written, [B, nchunks, D])
       const float* __restrict__ ws_h0,      // [B, D, N] copy of the initial state (nchunks > 1)
       const float* __restrict__ ws_c0,      // [B, D, K-1] copy of the initial conv history (nchunks > 1)
       float* __restrict__ ckpt,             // CK: [B, nck, N/4, D, 4] state checkpoints
       float* __restrict__ ypart,            // PART (written) / REV (read): [B, L, D] fp32 forward output
       ScanArgs sa) {
    static_assert(!(CK && GATE), "checkpoint mode has no gate");
    static_assert(!(CK && (REV || PART)) && !(REV && PART), "one mode per pass");
    // the plain forward with LOC: several chunks run from zero and k_corr adds their
    // carries; without LOC it takes the aggregate pass's carries as the other passes do
    constexpr bool PLAIN = !CK && !REV && !PART && LOC;
    static_assert(!LOC || (!CK && !REV && !PART), "LOC is a plain forward mode");
    static_assert(!POW || N >= kPowMinN, "power path only from kPowMinN states");
    const int D = sa.D;
    const int d_raw = blockIdx.x * kScanThreads + threadIdx.x;
    // lanes past the last channel work on the last channel: they compute and store
    // bit-identical values, so no store needs a branch
    const int d = d_raw < D ? d_raw : D - 1;
    if (pow_skip<N, POW>(A + (int64_t)d * N)) return;       // the workgroup runs in the other launch
    const unsigned du = (unsigned)d;              // zero-extended lane offset: uniform-base addressing
    const int c = blockIdx.y;
    const int b = blockIdx.z;
    const int64_t t0 = (int64_t)c * sa.chunk_len;
    const int64_t t1 = (t0 + sa.chunk_len < sa.L) ? t0 + sa.chunk_len : sa.L;
    const int nagg = sa.nchunks - 1;
    const bool multi = sa.nchunks > 1;
    // token v of the scan order sits at row prow(v) of [B, L, *]; consecutive tokens
    // are sD elements apart in [B, L, D] and sN in [B, L, N]
    auto prow = [&](int64_t v) -> int64_t { return (int64_t)b * sa.L + (REV ? sa.L - 1 - v : v); };
    const int64_t sD = REV ? -(int64_t)D : (int64_t)D;
    constexpr int sN = REV ? -N : N;

    // per-channel parameters
    float A2[N];
    float iA[ZOH ? N : 1];                        // ZOH: 1/A (0 for the A = 0 states)
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const float av = A[(int64_t)d * N + n];
        A2[n] = av * kLog2e;
        if (ZOH) {
            const bool zero = __builtin_fabsf(av) < kZohZeroA;
            iA[n] = zero ? 0.0f : 1.0f / av;
            if (zero) A2[n] = 0.0f;                   // an A = 0 state decays by exactly 1
        }
    }
    const float dbias = delta_bias ? delta_bias[d] : 0.0f;
    const float dsk = Dskip ? Dskip[d] : 0.0f;
    float w0 = 0.f, w1 = 0.f, w2 = 0.f, w3 = 1.f, cb = 0.f;
    if (CONV) {
        w0 = conv_w[d * 4 + 0]; w1 = conv_w[d * 4 + 1]; w2 = conv_w[d * 4 + 2]; w3 = conv_w[d * 4 + 3];
        cb = conv_b ? conv_b[d] : 0.0f;
    }

    // initial state of this chunk
    float h[N];
    const int64_t bd = (int64_t)b * D + d;
    if (c == 0) {
        // with several chunks, the checkpoint and bidirectional passes read the copy the
        // aggregate pass made, because their last chunk overwrites ssm_state (the plain
        // forward leaves it to k_corr)
        const float* src = REV ? nullptr : (ssm_state && multi && !PLAIN) ? ws_h0 : ssm_state;
#pragma unroll
        for (int n = 0; n < N; ++n) h[n] = src ? src[bd * N + n] : 0.0f;
    } else if (PLAIN) {
        // local run from a zero state; k_corr adds what the carry-in contributes
#pragma unroll
        for (int n = 0; n < N; ++n) h[n] = 0.0f;
    } else {
        // fold the aggregates of chunks 0..c-1 into the carry-in
#pragma unroll
        for (int n = 0; n < N; ++n) h[n] = 0.0f;
        for (int cc = 0; cc < c; ++cc) {
            const int64_t ai = ((int64_t)b * nagg + cc) * D + d;
            const float sdt = ws_sdt[ai];
            float dec[N];
            if constexpr (POW) {
                pow_chain<N>(exp2_fast(sdt * A2[0]), dec);
            } else {
#pragma unroll
                for (int n = 0; n < N; ++n) dec[n] = exp2_fast(sdt * A2[n]);
            }
#pragma unroll
            for (int n = 0; n < N; ++n) h[n] = __builtin_fmaf(dec[n], h[n], ws_S[ai * N + n]);
        }
    }

    // conv history x_{t0-3}, x_{t0-2}, x_{t0-1}: from x where t0-k >= 0, else from
    // the initial history (a multi-chunk call reads the copy the aggregate pass
    // made, because the last chunk overwrites conv_state)
    float x3 = 0.f, x2 = 0.f, x1 = 0.f;
    if (CONV) {
        const float* hsrc = (conv_state && !REV) ? ((multi && !PLAIN) ? ws_c0 : conv_state) : nullptr;
        float xh[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int64_t tt = t0 - 3 + j;
            xh[j] = tt >= 0 ? IO<T>::ld(x + prow(tt) * D + d)
                            : (hsrc ? hsrc[bd * 3 + (3 + tt)] : 0.0f);
        }
        x3 = xh[0]; x2 = xh[1]; x1 = xh[2];
    }

    // Token loop. B_t/C_t are staged through LDS in tiles of R tokens (double
    // buffered, one barrier per tile) and read back as wave-uniform broadcasts.
    // x/delta/z are prefetched one U-token group ahead as raw bits (two buffers
    // used alternately) and widened at use. Full tiles run without per-token
    // branches; only a chunk's last, partial tile goes token by token.
    constexpr int U = 4;
    constexpr int R = kScanTile;
    static_assert(R % (2 * U) == 0, "a tile holds whole pairs of groups");
    constexpr int NB = CK ? N : 2 * N;                  // staged values per token (B row, C row)
    __shared__ float sbc[2][R][NB];
    const int tid = threadIdx.x;
    __shared__ double srsum[PLAIN ? kScanThreads : 1];
    if constexpr (PLAIN) srsum[tid] = 0.0;
    const int nrows = (int)(t1 - t0);
    const unsigned voff = du * (unsigned)sizeof(T);               // lane byte offset within a token row
    const unsigned rowb = (unsigned)D * (unsigned)sizeof(T);      // bytes per token row
    const int64_t rowbase = prow(t0);                   // global row of the chunk's first token
    const T* xb = x + rowbase * D;
    const T* db = delta + rowbase * D;
    const T* zb = GATE ? z + rowbase * D : nullptr;
    T* yb = (CK || PART) ? nullptr : y + rowbase * D;
    float* ypb = (PART || REV) ? ypart + rowbase * D : nullptr;   // fp32 forward output of the chunk's first token
    const unsigned voff4 = du * 4u;                      // lane byte offset within an fp32 row
    const unsigned rowb4 = (unsigned)D * 4u;
    const T* Bb = Bm + rowbase * N;
    const T* Cb = CK ? nullptr : Cm + rowbase * N;

    // cooperative tile load: element e of the tile is (row e / N, state e % N)
    constexpr int TILE_ELEMS = R * N;
    constexpr int PER_THREAD = (TILE_ELEMS + kScanThreads - 1) / kScanThreads;
    T tb[PER_THREAD], tc[PER_THREAD];
    auto tile_fetch = [&](int r0) {
        // the tile's rows are contiguous in B and C: one uniform base, a 32-bit offset per element
        const int rlast = nrows - 1 - r0;
        const T* Bt = Bb + (int64_t)r0 * sN;
        const T* Ct = CK ? nullptr : Cb + (int64_t)r0 * sN;
#pragma unroll
        for (int k = 0; k < PER_THREAD; ++k) {
            const int e0 = tid + k * kScanThreads;
            const int e = e0 < TILE_ELEMS ? e0 : TILE_ELEMS - 1;
            const int r = e / N < rlast ? e / N : rlast;
            const int off = r * sN + e % N;
            tb[k] = Bt[off];
            if (!CK) tc[k] = Ct[off];
        }
    };
    // zero-order hold on the power path: B[n] is staged as B[n] / (n+1), the factor its
    // write coefficient takes from the geometric sum below (one rounding per value)
    auto tile_store = [&](int buf) {
#pragma unroll
        for (int k = 0; k < PER_THREAD; ++k) {
            const int e = tid + k * kScanThreads;
            if (e < TILE_ELEMS) {
                float bvs = IO<T>::cvt(tb[k]);
                if constexpr (ZOH && POW) bvs = bvs / (float)(e % N + 1);
                sbc[buf][e / N][e % N] = bvs;
                if (!CK) sbc[buf][e / N][N + e % N] = IO<T>::cvt(tc[k]);
            }
        }
    };

    // Per-token work in two phases. prologue(): the conv, SiLU, softplus and gate of
    // one token (a long dependent chain, run for a whole group of tokens first so the
    // chains of different tokens overlap). update(): the N-wide state update and
    // readout of one token, with its B/C row read from LDS up front.
    struct Pro { float u, dt, wv, g, yo; };
    auto prologue = [&](T xraw, T draw, T zraw, float yprev) -> Pro {
        Pro p;
        const float xt = IO<T>::cvt(xraw);
        if (CONV) {
            const float cv = __builtin_fmaf(w3, xt, __builtin_fmaf(w2, x1, __builtin_fmaf(w1, x2, __builtin_fmaf(w0, x3, cb))));
            x3 = x2; x2 = x1; x1 = xt;
            p.u = silu(cv);
        } else {
            p.u = xt;
        }
        p.dt = softplus(IO<T>::cvt(draw) + dbias);
        p.wv = p.dt * p.u;
        p.g = GATE ? silu(IO<T>::cvt(zraw)) : 1.0f;
        p.yo = REV ? yprev : 0.0f;                     // the forward pass's output at this position
        return p;
    };
    auto update = [&](const Pro& p, const float* bct, int r) {
        float bv[N], cv[N], a[N], t[N];
#pragma unroll
        for (int n = 0; n < N; ++n) bv[n] = bct[n];
        if constexpr (!CK) {
#pragma unroll
            for (int n = 0; n < N; ++n) cv[n] = bct[N + n];
        }
        if constexpr (POW) {
            // four interleaved power chains: a_0..a_3 (powers 1..4), then a_{n+4} = a_n a_3,
            // so the dependent multiplies are 3 + N/4 - 1 deep and each decay is used at
            // once (about five values live)
            float c[kPowLanes];
            c[0] = exp2_fast(p.dt * A2[0]);
            c[1] = c[0] * c[0];
            c[2] = c[1] * c[0];
            c[3] = c[1] * c[1];
            const float step = c[3];
            if constexpr (ZOH) {
                // (a_n - 1) / A_n = [(a_0 - 1) / A_0] G_n / (n+1) with A_n = (n+1) A_0 and
                // G_n = 1 + a_0 + ... + a_0^n: the coefficient of state 0 (with its series
                // near A_0 Delta = 0) once per token, G_n as four interleaved sums
                // G_{n+4} = G_n + a_n G_3 of positive terms (no cancellation for any n),
                // and 1/(n+1) already in the staged B
                const float cz = zoh_coef(c[0], p.dt * A2[0], p.dt, iA[0]) * p.u;
                float g[kPowLanes];
                g[0] = 1.0f;
                g[1] = 1.0f + c[0];
                g[2] = g[1] + c[1];
                g[3] = g[2] + c[2];
                const float q = g[3];
#pragma unroll
                for (int n = 0; n < N; ++n) {
                    const float an = c[n % kPowLanes];
                    const float gn = g[n % kPowLanes];
                    if (n + kPowLanes < N) {
                        c[n % kPowLanes] = an * step;
                        g[n % kPowLanes] = __builtin_fmaf(an, q, gn);
                    }
                    h[n] = __builtin_fmaf(an, h[n], (cz * gn) * bv[n]);
                }
            } else {
#pragma unroll
                for (int n = 0; n < N; ++n) {
                    const float an = c[n % kPowLanes];
                    if (n + kPowLanes < N) c[n % kPowLanes] = an * step;
                    h[n] = __builtin_fmaf(an, h[n], p.wv * bv[n]);
                }
            }
        } else {
#pragma unroll
            for (int n = 0; n < N; ++n) {
                t[n] = p.dt * A2[n];
                a[n] = exp2_fast(t[n]);
            }
            if constexpr (ZOH) {
#pragma unroll
                for (int n = 0; n < N; ++n)
                    h[n] = __builtin_fmaf(a[n], h[n], zoh_coef(a[n], t[n], p.dt, iA[n]) * (p.u * bv[n]));
            } else {
#pragma unroll
                for (int n = 0; n < N; ++n) h[n] = __builtin_fmaf(a[n], h[n], p.wv * bv[n]);
            }
        }
        if constexpr (!CK) {
            float ya = dsk * p.u, yc = 0.0f;
#pragma unroll
            for (int n = 0; n < N; n += 2) {
                ya = __builtin_fmaf(cv[n], h[n], ya);
                yc = __builtin_fmaf(cv[n + 1], h[n + 1], yc);
            }
            const float yv = REV ? __builtin_fmaf(ya + yc, p.g, p.yo) : (ya + yc) * p.g;
            // lanes past the last channel were clamped to it and store the same value
            if constexpr (PART) Buf<float>(ypb + (int64_t)r * sD).st(yv, voff4, 0u);
            else Buf<T>(yb + (int64_t)r * sD).st(IO<T>::bits(yv), voff, 0u);
        }
    };
    // checkpoint after chunk-relative row r (CK; the caller checks the spacing)
    auto store_ckpt = [&](int r) {
        const int64_t slot = (t0 + r + 1) / kCkptEvery - 1;
        vf4* dst = reinterpret_cast<vf4*>(ckpt) + ((int64_t)b * sa.nck + slot) * (N / 4) * D + d;
#pragma unroll
        for (int k = 0; k < N / 4; ++k) dst[(int64_t)k * D] = vf4{h[4 * k], h[4 * k + 1], h[4 * k + 2], h[4 * k + 3]};
    };
    // PLAIN: the chunk's summed step size, for its total decay exp(A * sum Delta) in
    // k_corr's fold: each group's fp32 sum is added (ds_add_f64, no return value) to an
    // fp64 total in the lane's own LDS slot, because a total kept in registers costs the
    // main pass a register spill at its three-waves-per-SIMD cap
    auto token = [&](T xraw, T draw, T zraw, float yprev, const float* bct, int r) {
        const Pro p = prologue(xraw, draw, zraw, yprev);
        if constexpr (PLAIN) atomicAdd(&srsum[tid], (double)p.dt);
        update(p, bct, r);
    };
    auto group = [&](const T* gx, const T* gd, const T* gz, const float* gy, const float* tile_rows, int r0) {
        Pro p[U];
#pragma unroll
        for (int i = 0; i < U; ++i) p[i] = prologue(gx[i], gd[i], gz[i], gy[i]);
        if constexpr (PLAIN) atomicAdd(&srsum[tid], (double)((p[0].dt + p[1].dt) + (p[2].dt + p[3].dt)));
#pragma unroll
        for (int i = 0; i < U; ++i) {
            update(p[i], tile_rows + i * NB, r0 + i);
            // power path: keep each token's chain of decays with its own update (hoisting
            // the next tokens' chains above it would hold N more values per token)
            if constexpr (POW) __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (CK) store_ckpt(r0 + U - 1);      // r0 + U is a multiple of kCkptEvery
    };
    T gx0[U], gd0[U], gz0[U], gx1[U], gd1[U], gz1[U];
    float gy0[U], gy1[U];
    auto load_group = [&](int r0, T* gx, T* gd, T* gz, float* gy) {
        // rows r0 .. r0+U-1 (clamped to the chunk's last row) at non-negative byte
        // offsets from the group's lowest-address row: the first row, or the last one
        // when the tokens run backward through memory (REV)
        const int rl = (r0 + U - 1 < nrows) ? r0 + U - 1 : nrows - 1;
        const int rb = REV ? rl : (r0 < nrows ? r0 : nrows - 1);
        const int64_t off = (int64_t)rb * sD;
        const Buf<T> bx(xb + off), bdl(db + off);
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int r = (r0 + i < nrows) ? r0 + i : nrows - 1;
            const unsigned so = (unsigned)(REV ? rb - r : r - rb) * rowb;
            gx[i] = bx.ld(voff, so);
            gd[i] = bdl.ld(voff, so);
            if (GATE) gz[i] = Buf<T>(zb + off).ld(voff, so);
            if (REV) gy[i] = Buf<float>(ypb + off).ld(voff4, (unsigned)(rb - r) * rowb4);
        }
    };

    int buf = 0;
    if (nrows > 0) {
        tile_fetch(0);
        tile_store(0);
        load_group(0, gx0, gd0, gz0, gy0);
    }
    __syncthreads();
    for (int tt = 0; tt < nrows; tt += R) {
        const bool more = tt + R < nrows;
        if (more) tile_fetch(tt + R);
        const float* tile = &sbc[buf][0][0];
        if (tt + R <= nrows) {
            for (int g = 0; g < R; g += 2 * U) {
                load_group(tt + g + U, gx1, gd1, gz1, gy1);
                group(gx0, gd0, gz0, gy0, tile + g * NB, tt + g);
                load_group(tt + g + 2 * U, gx0, gd0, gz0, gy0);
                group(gx1, gd1, gz1, gy1, tile + (g + U) * NB, tt + g + U);
            }
        } else {
            for (int r = tt; r < nrows; ++r) {
                const int64_t off = (int64_t)r * sD;
                token((xb + off)[du], (db + off)[du], GATE ? (zb + off)[du] : T(0), REV ? (ypb + off)[du] : 0.0f,
                      tile + (r - tt) * NB, r);
                if (CK && ((t0 + r + 1) % kCkptEvery) == 0) store_ckpt(r);
            }
        }
        if (more) tile_store(buf ^ 1);
        __syncthreads();
        buf ^= 1;
    }

    if constexpr (!CK && !REV && !PART && !LOC) {
        if (c == sa.nchunks - 1) {
            if (ssm_state) {
#pragma unroll
                for (int n = 0; n < N; ++n) ssm_state[bd * N + n] = h[n];
            }
            if (CONV && conv_state) {
                conv_state[bd * 3 + 0] = x3; conv_state[bd * 3 + 1] = x2; conv_state[bd * 3 + 2] = x1;
            }
        }
    }
    if constexpr (PLAIN) {
        if (!multi) {
            if (ssm_state) {
#pragma unroll
                for (int n = 0; n < N; ++n) ssm_state[bd * N + n] = h[n];
            }
            if (CONV && conv_state) {
                // a uniform base and a 32-bit lane offset (d < 2^26): no 64-bit offset kept
                // live across the token loop from the history read at the chunk start
                const Buf<float> cs(conv_state + (int64_t)b * D * 3);
                cs.st(x3, du * 12u, 0u); cs.st(x2, du * 12u, 4u); cs.st(x1, du * 12u, 8u);
            }
        } else {
            // the chunk's end state from its own start state and its summed step size
            // ([B, nchunks, D, N] and [B, nchunks, D]); k_corr writes the final states
            const int64_t ai = ((int64_t)b * sa.nchunks + c) * D + d;
#pragma unroll
            for (int n = 0; n < N; ++n) ws_S[ai * N + n] = h[n];
            ws_sdt[ai] = (float)srsum[tid];
        }
    }
}

// ---------------------------------------------------------------------------
// Chunk aggregates: for every chunk but the last, its end state S (from its
// initial state: zero, or the caller's state for chunk 0) and its summed step
// size. Written in the backward (Horner) form
//     S_n = sum_t exp(A_n * R_t) * Delta_t * u_t * B_t[n],   R_t = sum_{k>t} Delta_k,
// which is the unrolled recurrence. Under zero-order hold the write coefficient
// (exp(A_n Delta_t) - 1) / A_n times the decay exp(A_n R_t) telescopes to
// (E_t - E'_t) / A_n with E_t = exp(A_n (R_t + Delta_t)) and E'_t = exp(A_n R_t),
// and E'_t is the E of the token after t: one exponential per token and state, as
// for Euler. Where A_n Delta_t is small that difference cancels, and the term is
// taken as E'_t Delta_t phi(A_n Delta_t) with the series for phi instead.
// The sweep runs backward from the chunk end; a state index n is dropped
// (wave-uniformly) once exp(A_n * R) < 2^-kAggCutLog2 for every lane, because R
// only grows from there. Rows after every n is dropped only add Delta to the
// chunk's sum (needed exactly for its decay exp(A*sum)) and to a bound on what was
// dropped (both write coefficients are at most Delta for A <= 0):
//     |dropped part of S_n| <= 2^-kAggCutLog2 * M + umax * Mh,
//     M  = sum over the rows swept while some state is still active of
//          |Delta_t u_t| max_n |B_t[n]| (the rows that can hold a dropped term, and
//          the few before the first drop),
//     Mh = sum over rows after every state is dropped of exp(A_max R_t) Delta_t
//          max_n |B_t[n]|, A_max the least negative A (bounding every dropped weight),
// umax a bound on |u| over those rows (from their inputs, which need no SiLU).
// If it exceeds 2^-24 * max_n |S_n| (one unit roundoff of the aggregate) for any
// lane, the wave recomputes S exactly with the forward recurrence. R is
// accumulated in fp64.

// The cut sets how far back a state index is swept; the bound above must stay below
// one unit roundoff of the aggregate for the truncated sweep to stand. At 2^-36 the
// sweep is a tenth shorter, but on the long workload (steps log-uniform in
// [1e-3, 1e-1]) the zero-order-hold and adjoint aggregates then fail their bounds and
// take the exact fallback for most waves (3.6x and 1.8x slower); 2^-40 keeps them on
// the truncated sweep.
constexpr int kAggCutLog2 = 40;

// Rows per prefetched group of the aggregate pass: 8 up to d_state 16, 4 at 32 and 2 at 64,
// where the zero-order-hold form fills the register file with its four per-state arrays
// (with 8, that form kept its per-state arrays in scratch memory and once ended in a
// memory-aperture fault, though a host transcription of its index arithmetic finds
// every row, tile and LDS index in bounds, so it stays excluded).
template <int N> constexpr int agg_group_rows() { return N <= 16 ? 8 : (N <= 32 ? 4 : 2); }

// Whether the aggregate pass has a power launch: from kPowMinN states.
template <int N, bool ZOH> constexpr bool kAggPowLaunch = N >= kPowMinN;

// REV: the aggregates of the reversed scan order (see k_scan), no initial states.
// POW: the power fast path (launched twice, as k_scan): each row's decays
// exp(A_n R) = exp(A_0 R)^(n+1) from one exponential and a chain of multiplies. Under
// the identity A_n = (n+1) A_0 the drop order follows n (a block's least negative
// exponent falls with n, and every block is tested at the same R), so the active
// blocks are always a prefix and the chain stops at the first dropped one.
template <typename T, int N, bool CONV, bool ZOH, bool REV = false, bool POW = false>
__global__ void __launch_bounds__(kScanThreads)
k_agg(const T* __restrict__ x, const float* __restrict__ conv_w, const float* __restrict__ conv_b,
      const T* __restrict__ delta, const float* __restrict__ delta_bias, const float* __restrict__ A,
      const T* __restrict__ Bm, const float* __restrict__ ssm_state, const float* __restrict__ conv_state,
      float* __restrict__ ws_S, float* __restrict__ ws_sdt, float* __restrict__ ws_h0, float* __restrict__ ws_c0,
      ScanArgs sa) {
    const int D = sa.D;
    const int d_raw = blockIdx.x * kScanThreads + threadIdx.x;
    const int d = d_raw < D ? d_raw : D - 1;      // clamped lanes repeat the last channel
    // the vote only where launch_k_agg makes both launches
    if constexpr (kAggPowLaunch<N, ZOH>) {
        if (pow_skip<N, POW>(A + (int64_t)d * N)) return;   // the workgroup runs in the other launch
    }
    const unsigned du = (unsigned)d;              // zero-extended lane offset: uniform-base addressing
    const int c = blockIdx.y;                     // chunk, < nchunks - 1
    const int b = blockIdx.z;
    const int64_t t0 = (int64_t)c * sa.chunk_len;
    const int64_t t1 = t0 + sa.chunk_len;         // every chunk but the last is full
    const int nagg = sa.nchunks - 1;
    const int64_t row0 = (int64_t)b * sa.L;
    const int64_t bd = (int64_t)b * D + d;
    // token v of the scan order sits at row prow(v); consecutive tokens are sD / sN
    // elements apart (negative for the reversed order)
    auto prow = [&](int64_t v) -> int64_t { return row0 + (REV ? sa.L - 1 - v : v); };
    const int64_t sD = REV ? -(int64_t)D : (int64_t)D;
    constexpr int sN = REV ? -N : N;
    if (REV) { ssm_state = nullptr; conv_state = nullptr; }

    float A2[N];
    float iA[ZOH ? N : 1];                        // ZOH: 1/A (0 for the A = 0 states)
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const float av = A[(int64_t)d * N + n];
        const bool zero = ZOH && __builtin_fabsf(av) < kZohZeroA;
        A2[n] = zero ? 0.0f : av * kLog2e;            // ZOH: an A = 0 state decays by exactly 1
        if (ZOH) iA[n] = zero ? 0.0f : 1.0f / av;
    }
    const float dbias = delta_bias ? delta_bias[d] : 0.0f;
    float w0 = 0.f, w1 = 0.f, w2 = 0.f, w3 = 1.f, cb = 0.f;
    if (CONV) {
        w0 = conv_w[d * 4 + 0]; w1 = conv_w[d * 4 + 1]; w2 = conv_w[d * 4 + 2]; w3 = conv_w[d * 4 + 3];
        cb = conv_b ? conv_b[d] : 0.0f;
    }
    // the main pass of a multi-chunk call reads copies of the initial states,
    // because its last chunk overwrites them
    if (c == 0) {
        if (ssm_state) {
#pragma unroll
            for (int n = 0; n < N; ++n) ws_h0[bd * N + n] = ssm_state[bd * N + n];
        }
        if (CONV && conv_state) {
            ws_c0[bd * 3 + 0] = conv_state[bd * 3 + 0];
            ws_c0[bd * 3 + 1] = conv_state[bd * 3 + 1];
            ws_c0[bd * 3 + 2] = conv_state[bd * 3 + 2];
        }
    }
    constexpr int U = agg_group_rows<N>();
    static_assert(U <= 4 || N <= 16, "8-row groups only up to d_state 16");
    constexpr int R = kScanTile;
    static_assert(R % (2 * U) == 0, "tiles hold whole pairs of groups");
    constexpr int NB = N + 1;                     // B values and max_n |B| per token
    __shared__ float sB[2][R][NB];
    const int tid = threadIdx.x;
    constexpr int TILE_ELEMS = R * N;
    constexpr int PER_THREAD = (TILE_ELEMS + kScanThreads - 1) / kScanThreads;
    static_assert(kScanThreads % N == 0 && 64 % N == 0, "a token's N values sit in consecutive lanes of a wave");
    T tb[PER_THREAD];
    // tile with chunk-relative rows [rlo, rlo + R), rlo >= 0
    const T* Bc = Bm + prow(t0) * N;                      // uniform: B of the chunk's first token
    auto tile_fetch = [&](int rlo) {
#pragma unroll
        for (int k = 0; k < PER_THREAD; ++k) {
            const int e0 = tid + k * kScanThreads;
            const int e = e0 < TILE_ELEMS ? e0 : TILE_ELEMS - 1;
            tb[k] = Bc[(rlo + e / N) * sN + e % N];
        }
    };
    auto tile_store = [&](int buf) {
#pragma unroll
        for (int k = 0; k < PER_THREAD; ++k) {
            const int e = tid + k * kScanThreads;
            const float v = IO<T>::cvt(tb[k]);
            float m = __builtin_fabsf(v);
#pragma unroll
            for (int o = 1; o < N; o <<= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o, N));
            if (e < TILE_ELEMS) {
                // zero-order hold on the power path: B[n] / (n+1), the factor its write
                // coefficient takes from the geometric sum (the bound keeps max |B|)
                sB[buf][e / N][e % N] = (ZOH && POW) ? v / (float)(e % N + 1) : v;
                if (e % N == 0) sB[buf][e / N][N] = m;
            }
        }
    };

    float S[N];
    float Ep[ZOH ? N : 1];                        // ZOH: exp(A_n R) at the previous (later) token
#pragma unroll
    for (int n = 0; n < N; ++n) S[n] = 0.0f;
#pragma unroll
    for (int n = 0; n < (ZOH ? N : 1); ++n) Ep[n] = 1.0f;
    double Rsum = 0.0;                            // sum of Delta over the tokens swept so far
    float M = 0.0f;                               // sum |Delta u| max|B| over swept rows (full mode)
    float Mh = 0.0f;                              // sum Delta max|B| over rows swept after every n was dropped
    float xmax = 0.0f;                            // max |x| feeding those rows
    // state indices are dropped in blocks of BS (pairs up to d_state 32: single states
    // save some exponentials but cost a branch and a register copy per state and group,
    // measured slower); a block goes once its least negative exponent A2 * R is below
    // the cut on every lane
    constexpr int BS = N <= 32 ? 2 : N / 16;
    constexpr int NBLK = N / BS;
    static_assert(NBLK <= 32, "one mask bit per block");
    float A2blk[NBLK];
#pragma unroll
    for (int j = 0; j < NBLK; ++j) {
        float m = A2[BS * j];
#pragma unroll
        for (int q = 1; q < BS; ++q) m = __builtin_fmaxf(m, A2[BS * j + q]);
        A2blk[j] = m;
    }
    const uint32_t full = NBLK == 32 ? 0xffffffffu : (1u << NBLK) - 1u;
    uint32_t act = full;
    const float cut = -(float)kAggCutLog2;
    // the least negative exponent of all states: once every state is dropped (all of
    // them negative then), exp2(A2max * R) bounds each dropped state's weight at R
    float A2max = A2blk[0];
#pragma unroll
    for (int j = 1; j < NBLK; ++j) A2max = __builtin_fmaxf(A2max, A2blk[j]);

    // initial conv history (x_{-3}, x_{-2}, x_{-1}) in registers
    float hist0 = 0.f, hist1 = 0.f, hist2 = 0.f;
    if (CONV && conv_state) { hist0 = conv_state[bd * 3 + 0]; hist1 = conv_state[bd * 3 + 1]; hist2 = conv_state[bd * 3 + 2]; }

    // Token indices below are relative to the chunk start (int32). Every chunk this
    // kernel sweeps is full and a whole number of B tiles long (the host's chunking),
    // so no row is padding. x before the chunk start is the previous chunk's, except in
    // chunk 0, whose rows 0..2 take x_{-3..-1} from the initial history.
    const int clen = (int)(t1 - t0);
    const bool first = t0 == 0;
    // lowest chunk-relative row of x the sweep loads: x_{r-3} of rows down to -U (the
    // prefetch past the chunk start); t0 >= kScanTile > 3 + U when it is not chunk 0
    const int xlo = first ? 0 : -(3 + U);
    const T* xrow0 = x + prow(t0) * D;                    // uniform: token t0 of this batch row
    const T* drow0 = delta + prow(t0) * D;
    const unsigned voff = du * (unsigned)sizeof(T);       // lane byte offset within a token row
    const unsigned rowb = (unsigned)D * (unsigned)sizeof(T);
    auto hist_x = [&](int r) -> float { return r == -1 ? hist2 : (r == -2 ? hist1 : hist0); };   // r in -3..-1
    auto xmem = [&](int r) -> float { return IO<T>::ld(xrow0 + (int64_t)r * sD + d); };
    // conv window for the token about to be processed (r): xa = x_r, xb = x_{r-1}, xc = x_{r-2}
    // (clen >= kScanTile, so these rows are the chunk's own)
    float xa = xmem(clen - 1), xb = xmem(clen - 2), xc = xmem(clen - 3);
    // rows top, top-1, .., top-U+1 (each clamped to >= lo) of a [., D] tensor whose
    // chunk-relative row 0 is at p0: one uniform base at the group's lowest address and
    // uniform byte offsets from it
    auto load_rows = [&](const T* p0, int top, int lo, T* out) {
        const int hi = top > lo ? top : lo;
        const int bot = top - (U - 1) > lo ? top - (U - 1) : lo;
        const Buf<T> bf(p0 + (int64_t)(REV ? hi : bot) * sD);
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int r = top - i > lo ? top - i : lo;
            out[i] = bf.ld(voff, (unsigned)(REV ? hi - r : r - bot) * rowb);
        }
    };
    // prefetch of a group (rows gr-1 .. gr-U): delta of those rows, x of rows gr-4 .. gr-U-3;
    // two buffers used alternately
    T pd0[U], px0[U], pd1[U], px1[U];
    auto load_group = [&](int gr, T* pd, T* px) {
        load_rows(drow0, gr - 1, 0, pd);
        load_rows(xrow0, gr - 4, xlo, px);
    };
    bool cut_seen = false;                                // the window at the switch enters xmax once

    // one group of U rows (gr-1 .. gr-U); rowref is the staged row group_row(gr). Up to
    // d_state 16 that is row gr-U and the B row of gr-1-i (and its max |B|) is read at
    // rowref + (U-1-i) * NB, so every LDS read is one base register plus a non-negative
    // immediate offset (a negative one cannot be encoded and costs an address move per
    // read). Larger d_state passes row gr-1 and reads downward from it: with the cheaper
    // reads the compiler keeps more of them in flight, which the zero-order-hold kernel
    // at d_state 64 has no registers for. EDGE: chunk 0's last group (gr = U), whose rows
    // 0..2 take their oldest conv input from the initial history.
    // Up to d_state 16 (8-row groups) that group is a separate copy of the code; above,
    // the history enters through a few selects under a uniform branch (a second copy of
    // the larger kernels' group would not fit their registers), in the last group or, with
    // 2-row groups, the last two.
    constexpr bool PEEL = N <= 16;
    auto group = [&](auto edge, int gr, const T* cd, const T* cx, const float* rowref) {
        constexpr bool EDGE = decltype(edge)::value;
        auto brow = [&](int i) -> const float* { return N <= 16 ? rowref + (U - 1 - i) * NB : rowref - i * NB; };
        float xd[U];                                      // x_{r-3} of each row r = gr-1-i
#pragma unroll
        for (int i = 0; i < U; ++i) xd[i] = (EDGE && U - 4 - i < 0) ? hist_x(U - 4 - i) : IO<T>::cvt(cx[i]);
        if (!PEEL && first && gr - U < 3) {
            // the group of rows U-1..0, and with 2-row groups also rows 3..2 (row 2 takes x_{-1})
            if (gr == U) {
#pragma unroll
                for (int i = 0; i < U; ++i) {
                    if (U - 4 - i < 0) xd[i] = hist_x(U - 4 - i);
                }
            } else if (U < 3 && gr == 2 * U) {
#pragma unroll
                for (int i = 0; i < U; ++i) {
                    if (2 * U - 4 - i < 0) xd[i] = hist_x(2 * U - 4 - i);
                }
            }
        }
        if (act) {
            float dt[U], wv[U], uu[U];
#pragma unroll
            for (int i = 0; i < U; ++i) {
                float u;
                if (CONV) {
                    const float cv = __builtin_fmaf(w3, xa, __builtin_fmaf(w2, xb, __builtin_fmaf(w1, xc, __builtin_fmaf(w0, xd[i], cb))));
                    u = silu(cv);
                } else {
                    u = xa;
                }
                xa = xb; xb = xc; xc = xd[i];
                dt[i] = softplus(IO<T>::cvt(cd[i]) + dbias);
                wv[i] = dt[i] * u;
                uu[i] = u;
            }
            // suffix sums: fp64 running total, fp32 within the group. Rf excludes the
            // row's own Delta (Euler decay), Ri includes it (ZOH telescoping)
            const float rbase = (float)Rsum;
            float Rf[U], Ri[U], part = 0.0f;
#pragma unroll
            for (int i = 0; i < U; ++i) { Rf[i] = rbase + part; part += dt[i]; Ri[i] = rbase + part; }
            Rsum += (double)part;
            // every row swept while a state is active enters M (a superset of the rows
            // after the first drop, which loosens the bound only slightly)
#pragma unroll
            for (int i = 0; i < U; ++i) M = __builtin_fmaf(__builtin_fabsf(wv[i]), brow(i)[N], M);
            if constexpr (POW) {
                // running power e0^(BS j) of each row's base decay, advanced through the
                // active prefix of blocks. Zero-order hold: the row's term for state n is
                // exp(A_n R) (a_n - 1) / A_n u B[n] (R without the row's own step, a_n its
                // decay), with (a_n - 1) / A_n = [(a_0 - 1) / A_0] G_n / (n+1) and
                // G_n = 1 + a_0 + ... + a_0^n carried beside the running power; 1/(n+1)
                // is in the staged B.
                float e0[U], pw[U], a0[U], pa[U], gs[U], cz[U];
#pragma unroll
                for (int i = 0; i < U; ++i) {
                    e0[i] = exp2_fast(A2[0] * Rf[i]);
                    pw[i] = 1.0f;
                    if constexpr (ZOH) {
                        const float t0 = dt[i] * A2[0];
                        a0[i] = exp2_fast(t0);
                        pa[i] = 1.0f;
                        gs[i] = 0.0f;
                        cz[i] = zoh_coef(a0[i], t0, dt[i], iA[0]) * uu[i];
                    }
                }
#pragma unroll
                for (int j = 0; j < NBLK; ++j) {
                    if ((act >> j) & 1u) {                // then so is every block before it
                        // the block's staged B values of every row of the group are read
                        // first, so their LDS latency is not waited on row by row
                        float bb[U][BS];
#pragma unroll
                        for (int i = 0; i < U; ++i) {
#pragma unroll
                            for (int q = 0; q < BS; ++q) bb[i][q] = brow(i)[BS * j + q];
                        }
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int i = 0; i < U; ++i) {
#pragma unroll
                            for (int q = 0; q < BS; ++q) {
                                pw[i] *= e0[i];
                                if constexpr (ZOH) {
                                    gs[i] += pa[i];
                                    pa[i] *= a0[i];
                                    S[BS * j + q] = __builtin_fmaf(pw[i], (cz[i] * gs[i]) * bb[i][q], S[BS * j + q]);
                                } else {
                                    S[BS * j + q] = __builtin_fmaf(pw[i], wv[i] * bb[i][q], S[BS * j + q]);
                                }
                            }
                        }
                        if (!__any(A2blk[j] * (float)Rsum > cut)) act &= ~(1u << j);
                    }
                }
            } else {
#pragma unroll
            for (int j = 0; j < NBLK; ++j) {
                if ((act >> j) & 1u) {
                    if constexpr (ZOH) {
#pragma unroll
                        for (int i = 0; i < U; ++i) {
#pragma unroll
                            for (int q = 0; q < BS; ++q) {
                                const int n = BS * j + q;
                                const float e = exp2_fast(A2[n] * Ri[i]);
                                const float ts = dt[i] * A2[n];
                                const float big = (e - Ep[n]) * iA[n];                 // (E - E') / A
                                const float small = Ep[n] * (dt[i] * phi_series(ts));   // E' Delta phi
                                const float cf = __builtin_fabsf(ts) < kZohSeriesT ? small : big;
                                S[n] = __builtin_fmaf(cf, uu[i] * brow(i)[n], S[n]);
                                Ep[n] = e;
                            }
                        }
                    } else {
                        // the block's staged B values of every row are read first and its
                        // U * BS weights computed next, so the exponentials cover the LDS
                        // latency instead of each row waiting on its own read
                        float bb[U][BS], ee[U][BS];
#pragma unroll
                        for (int i = 0; i < U; ++i) {
#pragma unroll
                            for (int q = 0; q < BS; ++q) bb[i][q] = brow(i)[BS * j + q];
                        }
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int i = 0; i < U; ++i) {
#pragma unroll
                            for (int q = 0; q < BS; ++q) ee[i][q] = exp2_fast(A2[BS * j + q] * Rf[i]);
                        }
#pragma unroll
                        for (int i = 0; i < U; ++i) {
#pragma unroll
                            for (int q = 0; q < BS; ++q)
                                S[BS * j + q] = __builtin_fmaf(ee[i][q], wv[i] * bb[i][q], S[BS * j + q]);
                        }
                    }
                    // weights only shrink further back: drop the block once every lane is below the cut
                    if (!__any(A2blk[j] * (float)Rsum > cut)) act &= ~(1u << j);
                }
            }
            }
        } else {
            if (!cut_seen) {
                // the window entering the first row after the cut
                xmax = __builtin_fmaxf(__builtin_fabsf(xa), __builtin_fmaxf(__builtin_fabsf(xb), __builtin_fabsf(xc)));
                cut_seen = true;
            }
            // every row of the group has weight at most exp2(A2max * R) at the group's
            // first R, since R only grows (one exponential per group)
            const float wt = exp2_fast(A2max * (float)Rsum);
            float part = 0.0f, mg = 0.0f;
#pragma unroll
            for (int i = 0; i < U; ++i) {
                // each x enters the bound once, as the newest input of the row that loads it
                xmax = __builtin_fmaxf(xmax, __builtin_fabsf(xd[i]));
                const float dtv = softplus(IO<T>::cvt(cd[i]) + dbias);
                part += dtv;
                mg = __builtin_fmaf(dtv, brow(i)[N], mg);
            }
            Mh = __builtin_fmaf(wt, mg, Mh);
            Rsum += (double)part;
        }
    };

    auto group_row = [](int gr) { return N <= 16 ? gr - U : gr - 1; };
    const int ntiles = clen / R;
    tile_fetch(clen - R);
    tile_store(0);
    load_group(clen, pd0, px0);
    __syncthreads();
    int buf = 0;
    for (int k = 0; k < ntiles; ++k) {
        const int rhi = clen - k * R;                     // tile rows [rhi - R, rhi)
        if (k + 1 < ntiles) tile_fetch(rhi - 2 * R);
        const float* tbase = &sB[buf][0][0] - (int64_t)(rhi - R) * NB;   // row r of this tile at tbase + r*NB
        const bool edge = first && k + 1 == ntiles;      // the tile holding chunk 0's rows 0..2
        for (int gr = rhi; gr > rhi - R; gr -= 2 * U) {
            load_group(gr - U, pd1, px1);
            group(Tag<false>{}, gr, pd0, px0, tbase + group_row(gr) * NB);
            load_group(gr - 2 * U, pd0, px0);
            if (PEEL && edge && gr - U == U) group(Tag<PEEL>{}, U, pd1, px1, tbase + group_row(U) * NB);
            else group(Tag<false>{}, gr - U, pd1, px1, tbase + group_row(gr - U) * NB);
        }
        if (k + 1 < ntiles) tile_store(buf ^ 1);
        __syncthreads();
        buf ^= 1;
    }
    xmax = cut_seen ? xmax : 0.0f;
    // rows swept after the cut: |u| <= |c| <= |cb| + sum_k |w_k| max|x| (SiLU(c) shrinks |c|)
    const float umax = CONV ? __builtin_fabsf(cb) + (__builtin_fabsf(w0) + __builtin_fabsf(w1) + __builtin_fabsf(w2) +
                                                    __builtin_fabsf(w3)) * xmax
                            : xmax;
    const float Rtot = (float)Rsum;
    if (c == 0 && ssm_state) {
#pragma unroll
        for (int n = 0; n < N; ++n) S[n] = __builtin_fmaf(exp2_fast(A2[n] * Rtot), ssm_state[bd * N + n], S[n]);
    }
    float smax = 0.0f;
#pragma unroll
    for (int n = 0; n < N; ++n) smax = __builtin_fmaxf(smax, __builtin_fabsf(S[n]));
    const float bound = __builtin_ldexpf(M, -kAggCutLog2) + umax * Mh;
    const bool bad = !(bound <= smax * 0x1p-24f);
    if (__any(bad)) {
        // exact forward recurrence over the chunk (rare: the dropped part was not negligible)
        float h[N];
        const float* src = (c == 0) ? ssm_state : nullptr;
#pragma unroll
        for (int n = 0; n < N; ++n) h[n] = src ? src[bd * N + n] : 0.0f;
        // x_{-3..-1}: the history in chunk 0, else the previous chunk's last rows (the
        // loads read row 0 in chunk 0 and the value is selected afterwards)
        const float m3 = xmem(first ? 0 : -3), m2 = xmem(first ? 0 : -2), m1 = xmem(first ? 0 : -1);
        float x3 = first ? hist0 : m3, x2 = first ? hist1 : m2, x1 = first ? hist2 : m1;
        double sd = 0.0;
        for (int64_t t = t0; t < t1; ++t) {
            const float xt = IO<T>::ld(x + prow(t) * D + d);
            float u = xt;
            if (CONV) {
                const float cv = __builtin_fmaf(w3, xt, __builtin_fmaf(w2, x1, __builtin_fmaf(w1, x2, __builtin_fmaf(w0, x3, cb))));
                x3 = x2; x2 = x1; x1 = xt;
                u = silu(cv);
            }
            const float dtv = softplus(IO<T>::ld(delta + prow(t) * D + d) + dbias);
            sd += (double)dtv;
            const float w = dtv * u;
            const T* Bt = Bm + prow(t) * N;
#pragma unroll
            for (int n = 0; n < N; ++n) {
                const float tn = dtv * A2[n];
                const float a = exp2_fast(tn);
                if constexpr (ZOH) {
                    h[n] = __builtin_fmaf(a, h[n], zoh_coef(a, tn, dtv, iA[n]) * (u * IO<T>::cvt(Bt[n])));
                } else {
                    h[n] = __builtin_fmaf(a, h[n], w * IO<T>::cvt(Bt[n]));
                }
            }
        }
#pragma unroll
        for (int n = 0; n < N; ++n) S[n] = h[n];
        Rsum = sd;
    }
    const int64_t ai = ((int64_t)b * nagg + c) * D + d;
    ws_sdt[ai] = (float)Rsum;
#pragma unroll
    for (int n = 0; n < N; ++n) ws_S[ai * N + n] = S[n];
}

// ---------------------------------------------------------------------------
// Carry correction of the plain forward over several chunks. The main pass runs
// every chunk but the first from a zero state and writes each chunk's end state
// S_c and summed step size; k_fold (below) turns them into the carry-ins
//     H_1 = S_0,   H_{c+1} = exp(A_n * sum Delta_c) H_c + S_c.
// By linearity of the recurrence the true state at chunk-relative row r of chunk
// c >= 1 is the local one plus E_r[n] H_c[n], E_r[n] = exp(A_n R_r) with R_r the
// step sizes of rows 0..r summed (the decay alone carries the state; the write
// term, Euler or zero-order hold, does not enter). So the output misses
//     sum_n C_r[n] E_r[n] H_c[n]   (times SiLU(z_r) with the gate),
// which k_corr adds to y. Where A_n <= 0, E only shrinks as r grows: a state index
// is dropped (wave-uniformly, in blocks as in k_agg) once exp(A_n R) <= 2^-kCorrCutLog2
// on every lane whose carry is not exactly zero, and that leaves every later state of
// the chunk off by at most 2^-kCorrCutLog2 |H_c[n]| (one fp32 unit roundoff of the
// carry, the rounding H_c itself already holds). A workgroup stops once its waves have
// dropped every index, so the pass reads
// delta, z and y only over each chunk's head; channels whose states barely decay
// (A_n > 0 or tiny steps) keep theirs to the chunk end.
// POW: decays from exp(A_0 R)^(n+1); the per-row sum is then a polynomial in
// exp(A_0 R), evaluated by Horner's rule over the states up to the highest one still
// active (the drop order follows n, so dropped states below it add zero terms only
// where their carry is exactly zero).
constexpr int kCorrCutLog2 = 24;
constexpr int kCorrDepth = 8;                 // prefetched 4-row groups of delta, z and y

// The fold of the plain forward's chunk end states, one thread per (batch row,
// channel, state): H_1 = S_0, H_{c+1} = exp(A sum Delta_c) H_c + S_c, each carry H_c
// written over slot c-1 of the end states (already read by then), the final state
// exp(A sum Delta_last) H_last + S_last to ssm_state and the conv history (the last
// three inputs) to conv_state. Loads are issued kFoldBatch chunks at a time, so a
// thread waits on about nchunks / kFoldBatch memory round trips rather than nchunks.
constexpr int kFoldBatch = 16;
template <typename T, int N>
__global__ void __launch_bounds__(kScanThreads)
k_fold(const T* __restrict__ x, const float* __restrict__ A, float* __restrict__ ssm_state,
       float* __restrict__ conv_state, float* __restrict__ ws_S, const float* __restrict__ ws_sdt,
       int64_t batch, ScanArgs sa) {
    const int64_t D = sa.D;
    const int64_t i = (int64_t)blockIdx.x * kScanThreads + threadIdx.x;   // (b, d, n)
    if (i >= batch * D * N) return;                 // no barriers in this kernel
    const int n = (int)(i % N);
    const int64_t bd = i / N;
    const int64_t b = bd / D, d = bd % D;
    const float av = A[d * N + n];
    const float a2 = __builtin_fabsf(av) < kZohZeroA ? 0.0f : av * kLog2e;
    const int nc = sa.nchunks;
    float* Sb = ws_S + (b * nc * D + d) * N + n;     // slot c at Sb[c * D * N]
    const float* tb = ws_sdt + b * nc * D + d;       // slot c at tb[c * D]
    float H = 0.0f;
    for (int c0 = 0; c0 < nc; c0 += kFoldBatch) {
        float sv[kFoldBatch], tv[kFoldBatch];
#pragma unroll
        for (int k = 0; k < kFoldBatch; ++k) {
            const int c = c0 + k < nc ? c0 + k : nc - 1;
            sv[k] = Sb[(int64_t)c * D * N];
            tv[k] = tb[(int64_t)c * D];
        }
#pragma unroll
        for (int k = 0; k < kFoldBatch; ++k) {
            const int c = c0 + k;
            if (c < nc) {
                if (c > 0) Sb[(int64_t)(c - 1) * D * N] = H;     // carry into chunk c
                H = __builtin_fmaf(exp2_fast(a2 * tv[k]), H, sv[k]);
            }
        }
    }
    if (ssm_state) ssm_state[bd * N + n] = H;
    if (conv_state && n < 3) {
        // the chunking keeps the last chunk at least one tile long, so L > 3
        conv_state[bd * 3 + n] = IO<T>::cvt(x[(b * sa.L + sa.L - 3 + n) * D + d]);
    }
}

template <typename T, int N, bool GATE, bool POW>
__global__ void __launch_bounds__(kScanThreads)
k_corr(const T* __restrict__ delta, const float* __restrict__ delta_bias, const float* __restrict__ A,
       const T* __restrict__ Cm, const T* __restrict__ z, T* __restrict__ y, const float* __restrict__ ws_H,
       ScanArgs sa) {
    const int D = sa.D;
    const int d_raw = blockIdx.x * kScanThreads + threadIdx.x;
    const int d = d_raw < D ? d_raw : D - 1;      // clamped lanes repeat the last channel
    // y is read, corrected and written back, so only the channel's own lane may store
    // (the clamped lanes of the main pass write identical values; here each would add
    // its correction again)
    const bool owner = d_raw < D;
    if (pow_skip<N, POW>(A + (int64_t)d * N)) return;   // the workgroup runs in the other launch
    const unsigned du = (unsigned)d;
    const int nc = sa.nchunks;
    const int c = blockIdx.y + 1;                 // chunks 1 .. nchunks-1
    const int b = blockIdx.z;
    const int64_t t0 = (int64_t)c * sa.chunk_len;
    const int64_t t1 = (t0 + sa.chunk_len < sa.L) ? t0 + sa.chunk_len : sa.L;

    float A2[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const float av = A[(int64_t)d * N + n];
        A2[n] = __builtin_fabsf(av) < kZohZeroA ? 0.0f : av * kLog2e;   // decays by exactly 1
    }
    const float dbias = delta_bias ? delta_bias[d] : 0.0f;
    // carry-in of chunk c, written by k_fold over slot c-1 of the end states
    float H[N];
    const float* hc = ws_H + ((((int64_t)b * nc + (c - 1)) * D) + d) * N;
#pragma unroll
    for (int n = 0; n < N; ++n) H[n] = hc[n];

    // state blocks and the drop rule
    constexpr int BS = N <= 32 ? 2 : N / 16;
    constexpr int NBLK = N / BS;
    static_assert(NBLK <= 32, "one mask bit per block");
    float A2blk[NBLK];
    uint32_t live = 0;                            // blocks with a nonzero carry on this lane
#pragma unroll
    for (int j = 0; j < NBLK; ++j) {
        float m = A2[BS * j];
        bool nz = H[BS * j] != 0.0f;
#pragma unroll
        for (int q = 1; q < BS; ++q) { m = __builtin_fmaxf(m, A2[BS * j + q]); nz = nz || H[BS * j + q] != 0.0f; }
        A2blk[j] = m;
        live |= nz ? (1u << j) : 0u;
    }
    const float cut = -(float)kCorrCutLog2;
    uint32_t act = 0;
#pragma unroll
    for (int j = 0; j < NBLK; ++j) act |= __any((live >> j) & 1u) ? (1u << j) : 0u;

    // workgroup-uniform exit: one flag word per wave, double-buffered by tile parity so
    // that a wave writing the next tile's word never races a wave still reading this one
    constexpr int NW = kScanThreads / 64;
    __shared__ uint32_t wact[2][NW];
    const int wave = threadIdx.x >> 6;
    auto all_done = [&](int parity) -> bool {
        if ((threadIdx.x & 63) == 0) wact[parity][wave] = act;
        __syncthreads();
        uint32_t any = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) any |= wact[parity][w];
        return any == 0;
    };
    if (all_done(1)) return;

    // C tiles through LDS (as k_scan's B/C), delta, z and y one U-row group ahead
    constexpr int U = 4;
    constexpr int R = kScanTile;
    static_assert(R % (2 * U) == 0, "a tile holds whole pairs of groups");
    __shared__ float sC[2][R][N];
    const int tid = threadIdx.x;
    const int nrows = (int)(t1 - t0);
    const unsigned voff = du * (unsigned)sizeof(T);
    const unsigned rowb = (unsigned)D * (unsigned)sizeof(T);
    const int64_t rowbase = (int64_t)b * sa.L + t0;
    const T* db = delta + rowbase * D;
    const T* zb = GATE ? z + rowbase * D : nullptr;
    T* yb = y + rowbase * D;
    const T* Cb = Cm + rowbase * N;
    constexpr int TILE_ELEMS = R * N;
    constexpr int PER_THREAD = (TILE_ELEMS + kScanThreads - 1) / kScanThreads;
    T tc[PER_THREAD];
    auto tile_fetch = [&](int r0) {
        const int rlast = nrows - 1 - r0;
        const T* Ct = Cb + (int64_t)r0 * N;
#pragma unroll
        for (int k = 0; k < PER_THREAD; ++k) {
            const int e0 = tid + k * kScanThreads;
            const int e = e0 < TILE_ELEMS ? e0 : TILE_ELEMS - 1;
            const int r = e / N < rlast ? e / N : rlast;
            tc[k] = Ct[r * N + e % N];
        }
    };
    auto tile_store = [&](int buf) {
#pragma unroll
        for (int k = 0; k < PER_THREAD; ++k) {
            const int e = tid + k * kScanThreads;
            if (e < TILE_ELEMS) sC[buf][e / N][e % N] = IO<T>::cvt(tc[k]);
        }
    };
    // delta, z and y of kCorrDepth groups in flight: the grid gives a SIMD about two
    // waves and a group's work is short, so one group ahead would leave each wave
    // waiting on HBM latency
    T gd[kCorrDepth][U], gz[kCorrDepth][U], gy[kCorrDepth][U];
    auto load_group = [&](int r0, T* gd, T* gz, T* gy) {
        const int rb = r0 < nrows ? r0 : nrows - 1;
        const int64_t off = (int64_t)rb * D;
        const Buf<T> bdl(db + off), by(yb + off);
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int r = (r0 + i < nrows) ? r0 + i : nrows - 1;
            const unsigned so = (unsigned)(r - rb) * rowb;
            gd[i] = bdl.ld(voff, so);
            if (GATE) gz[i] = Buf<T>(zb + off).ld(voff, so);
            gy[i] = by.ld(voff, so);
        }
    };

    double rsum = 0.0;                            // step sizes of the rows swept so far
    auto group = [&](const T* gd, const T* gz, const T* gy, const float* crow, int r0) {
        float Rr[U], g[U], corr[U];
        float part = 0.0f;
        const float rbase = (float)rsum;
#pragma unroll
        for (int i = 0; i < U; ++i) {
            // rows past the chunk end (the last chunk's final group) add no step
            const float dt = r0 + i < nrows ? softplus(IO<T>::cvt(gd[i]) + dbias) : 0.0f;
            part += dt;
            Rr[i] = rbase + part;                     // R of row r0+i, its own step included
            g[i] = GATE ? silu(IO<T>::cvt(gz[i])) : 1.0f;
            corr[i] = 0.0f;
        }
        rsum += (double)part;
        if constexpr (POW) {
            float e0[U];
#pragma unroll
            for (int i = 0; i < U; ++i) e0[i] = exp2_fast(A2[0] * Rr[i]);
            // Horner from the highest active state down: acc = sum_n C[n] H[n] e0^n, times e0
#pragma unroll
            for (int j = NBLK - 1; j >= 0; --j) {
                if ((act >> j) != 0u) {               // block j is at or below the highest active one
#pragma unroll
                    for (int q = BS - 1; q >= 0; --q) {
                        const int n = BS * j + q;
#pragma unroll
                        for (int i = 0; i < U; ++i)
                            corr[i] = __builtin_fmaf(corr[i], e0[i], crow[i * N + n] * H[n]);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < U; ++i) corr[i] *= e0[i];
        } else {
#pragma unroll
            for (int j = 0; j < NBLK; ++j) {
                if ((act >> j) & 1u) {
#pragma unroll
                    for (int q = 0; q < BS; ++q) {
                        const int n = BS * j + q;
#pragma unroll
                        for (int i = 0; i < U; ++i) {
                            const float e = exp2_fast(A2[n] * Rr[i]);
                            corr[i] = __builtin_fmaf(crow[i * N + n], H[n] * e, corr[i]);
                        }
                    }
                }
            }
        }
        const int64_t off = (int64_t)r0 * D;
        const Buf<T> by(yb + off);
#pragma unroll
        for (int i = 0; i < U; ++i) {
            if (r0 + i < nrows && owner) {
                const float yv = __builtin_fmaf(corr[i], g[i], IO<T>::cvt(gy[i]));
                by.st(IO<T>::bits(yv), voff, (unsigned)i * rowb);
            }
        }
        // drop blocks whose decay is below the cut on every lane that carries them
        const float rl = Rr[U - 1];
#pragma unroll
        for (int j = 0; j < NBLK; ++j) {
            if ((act >> j) & 1u) {
                if (!__any(((live >> j) & 1u) && A2blk[j] * rl > cut)) act &= ~(1u << j);
            }
        }
    };

    int buf = 0;
    tile_fetch(0);
    tile_store(0);
#pragma unroll
    for (int q = 0; q < kCorrDepth; ++q) load_group(q * U, gd[q], gz[q], gy[q]);
    __syncthreads();
    constexpr int GPT = R / U;                    // groups per tile
    static_assert(GPT % kCorrDepth == 0, "the in-flight slots cycle within a tile");
    for (int tt = 0; tt < nrows; tt += R) {
        const bool more = tt + R < nrows;
        if (more) tile_fetch(tt + R);
        const float* tile = &sC[buf][0][0];
        // group k of the tile sits in slot k % kCorrDepth; once it is done the slot takes
        // the group kCorrDepth further on (rows past the chunk end are clamped loads)
#pragma unroll
        for (int k = 0; k < GPT; ++k) {
            const int q = k % kCorrDepth;
            const int r0 = tt + k * U;
            if (act && r0 < nrows) group(gd[q], gz[q], gy[q], tile + k * U * N, r0);
            load_group(r0 + kCorrDepth * U, gd[q], gz[q], gy[q]);
        }
        if (more) tile_store(buf ^ 1);
        const int parity = (tt / R) & 1;
        if (all_done(parity)) return;             // (includes the barrier of the tile swap)
        buf ^= 1;
    }
}

// ---------------------------------------------------------------------------
// Decode step. Four lanes (a quad) per (stream, channel): lane q holds state
// entries [q*N/4, (q+1)*N/4), so every state load and store of a wave is one
// contiguous, nontemporal vector access. The conv taps and the readout are
// summed across the quad with DPP; lane q < 3 holds conv history entry q and
// lane 3 the new input, so the shifted history is one quad rotation away.

// DPP quad permutations: xor-1, xor-2 and "take lane q+1" (lane 3 keeps its own)
constexpr int kQuadXor1 = 1 | (0 << 2) | (3 << 4) | (2 << 6);
constexpr int kQuadXor2 = 2 | (3 << 2) | (0 << 4) | (1 << 6);
constexpr int kQuadNext = 1 | (2 << 2) | (3 << 4) | (3 << 6);

template <int CTRL>
__device__ __forceinline__ float quad_dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_sum(float v) {
    v += quad_dpp<kQuadXor1>(v);
    return v + quad_dpp<kQuadXor2>(v);
}

template <int NQ>
__device__ __forceinline__ void ld_nt(const float* p, float* v) {
    if constexpr (NQ % 4 == 0) {
#pragma unroll
        for (int k = 0; k < NQ / 4; ++k) {
            const vf4 t = __builtin_nontemporal_load(reinterpret_cast<const vf4*>(p) + k);
            v[4 * k] = t.x; v[4 * k + 1] = t.y; v[4 * k + 2] = t.z; v[4 * k + 3] = t.w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < NQ; ++k) v[k] = __builtin_nontemporal_load(p + k);
    }
}
template <int NQ>
__device__ __forceinline__ void st_nt(float* p, const float* v) {
    if constexpr (NQ % 4 == 0) {
#pragma unroll
        for (int k = 0; k < NQ / 4; ++k) {
            const vf4 t = {v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]};
            __builtin_nontemporal_store(t, reinterpret_cast<vf4*>(p) + k);
        }
    } else {
#pragma unroll
        for (int k = 0; k < NQ; ++k) __builtin_nontemporal_store(v[k], p + k);
    }
}

template <typename T, int N, bool CONV, bool GATE, bool ZOH>
__global__ void __launch_bounds__(kStepThreads)
k_step(const T* __restrict__ x, const float* __restrict__ conv_w, const float* __restrict__ conv_b,
       const T* __restrict__ delta, const float* __restrict__ delta_bias, const float* __restrict__ A,
       const T* __restrict__ Bm, const T* __restrict__ Cm, const float* __restrict__ Dskip,
       const T* __restrict__ z, T* __restrict__ y, float* __restrict__ ssm_state,
       float* __restrict__ conv_state, int D, int S) {
    constexpr int NQ = N / 4;
    constexpr int SPT = kStepStreams;         // streams handled by each quad (same channel)
    const int q = threadIdx.x & 3;
    const int d = blockIdx.x * (kStepThreads / 4) + (threadIdx.x >> 2);
    const int s0 = blockIdx.y * SPT;
    if (d >= D) return;                       // whole quads leave together

    // channel parameters, shared by the SPT streams
    float aq[NQ], iaq[ZOH ? NQ : 1];
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
        const float av = A[(int64_t)d * N + q * NQ + k];
        const bool zero = ZOH && __builtin_fabsf(av) < kZohZeroA;
        aq[k] = zero ? 0.0f : av * kLog2e;
        if (ZOH) iaq[k] = zero ? 0.0f : 1.0f / av;
    }
    const float wq = CONV ? conv_w[d * 4 + q] : 0.0f;
    const float cb = (CONV && conv_b) ? conv_b[d] : 0.0f;
    const float dbias = delta_bias ? delta_bias[d] : 0.0f;
    const float dsk = Dskip ? Dskip[d] : 0.0f;

    // every stream's loads first (streams past S are clamped to the last one and skipped below)
    float hq[SPT][NQ], hist[SPT];
    T braw[SPT][NQ], craw[SPT][NQ], xraw[SPT], draw[SPT], zraw[SPT];
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
        const int s = (s0 + j < S) ? s0 + j : S - 1;
        const int64_t sd = (int64_t)s * D + d;
        ld_nt<NQ>(ssm_state + sd * N + q * NQ, hq[j]);
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
            braw[j][k] = Bm[(int64_t)s * N + q * NQ + k];
            craw[j][k] = Cm[(int64_t)s * N + q * NQ + k];
        }
        xraw[j] = x[sd];
        draw[j] = delta[sd];
        zraw[j] = GATE ? z[sd] : T(0);
        hist[j] = (CONV && q < 3) ? __builtin_nontemporal_load(conv_state + sd * 3 + q) : 0.0f;
    }

#pragma unroll
    for (int j = 0; j < SPT; ++j) {
        if (s0 + j >= S) break;                // uniform across the workgroup
        const int64_t sd = (int64_t)(s0 + j) * D + d;
        const float xt = IO<T>::cvt(xraw[j]);
        float u;
        if (CONV) {
            // lane q contributes w[q] * (history q, or the new input on lane 3)
            const float v = q < 3 ? hist[j] : xt;
            u = silu(quad_sum(wq * v) + cb);
            // shifted history (x_{t-2}, x_{t-1}, x_t): lane q takes lane q+1's value
            const float nh = quad_dpp<kQuadNext>(v);
            if (q < 3) __builtin_nontemporal_store(nh, conv_state + sd * 3 + q);
        } else {
            u = xt;
        }
        const float dt = softplus(IO<T>::cvt(draw[j]) + dbias);
        const float wv = dt * u;
        float yp = 0.0f;
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
            const float tk = dt * aq[k];
            const float a = exp2_fast(tk);
            if constexpr (ZOH) {
                hq[j][k] = __builtin_fmaf(a, hq[j][k], zoh_coef(a, tk, dt, iaq[k]) * (u * IO<T>::cvt(braw[j][k])));
            } else {
                hq[j][k] = __builtin_fmaf(a, hq[j][k], wv * IO<T>::cvt(braw[j][k]));
            }
            yp = __builtin_fmaf(IO<T>::cvt(craw[j][k]), hq[j][k], yp);
        }
        st_nt<NQ>(ssm_state + sd * N + q * NQ, hq[j]);
        float yv = quad_sum(yp) + dsk * u;
        if (GATE) yv *= silu(IO<T>::cvt(zraw[j]));
        if (q == 0) IO<T>::st(y + sd, yv);
    }
}

// ---------------------------------------------------------------------------
// Forward scan on grids that one lane per channel cannot fill (few batch rows x
// channels, and sequences too short for enough chunks of at least one B/C tile):
// four lanes (a quad) per (batch row, channel), lane q holding state entries
// [q N/4, (q+1) N/4) as in the decode step, so the chip holds four times as many
// waves; the readout is summed over the quad with DPP. The aggregates and their
// workspace are those of k_agg / k_scan and the carry-in is the same fold, with the
// aggregates of 8 chunks loaded before any is folded; chunks need not be whole B/C
// tiles (nothing is staged in LDS), so the forward chunks these grids more finely. A
// chunk's aggregate is its end state by the forward recurrence, exactly (the chunks
// here are short, where the truncated backward sweep would drop little).
// Tokens go in groups of kQuadGroup = 4, loaded one group ahead (two register buffers
// used alternately). The per-token work that does not depend on the state index
// (conv + SiLU, softplus, SiLU(z)) is split over the quad: lane q loads x, delta and z
// of token q of the group only, takes the earlier inputs of its conv window from the
// lanes before it (DPP shifts within the quad, the carried window where the shift
// would reach before the group), computes that token's terms and DPP broadcasts them
// to the other lanes. Every lane loads the B and C quarter-rows of all four tokens.
// Lanes past the last channel repeat it but store nothing: with no barrier between
// the waves of a workgroup, such a lane could otherwise read an in-place state after
// its owner has written it.
constexpr int kQuadGroup = 4;              // one token of a group per lane of the quad
constexpr int kQuadFold = 8;               // aggregates loaded per step of the carry fold

// lane i's value on every lane of its quad
template <int I>
__device__ __forceinline__ float quad_bcast(float v) {
    return quad_dpp<I | (I << 2) | (I << 4) | (I << 6)>(v);
}
// lane q takes lane q-1's value (quad_perm 0,0,1,2) and lane q-2's (quad_perm 0,0,0,1);
// lanes without such a predecessor get lane 0's, which the caller replaces
constexpr int kQuadPrev1 = 0 | (0 << 2) | (1 << 4) | (2 << 6);
constexpr int kQuadPrev2 = 0 | (0 << 2) | (0 << 4) | (1 << 6);

template <typename T, int NQ, bool GATE, bool CB>
struct QuadGroup {
    T x, dl, z;                                  // token q of the group (lane q)
    T b[kQuadGroup][NQ], c[CB ? kQuadGroup : 1][CB ? NQ : 1];
};

// Loads of rows r0 .. r0 + kQuadGroup - 1 of the chunk (clamped to its last row): x,
// delta and z of row r0 + q on lane q, the B and C quarter-rows of all four rows.
template <typename T, int N, bool GATE, bool CB>
__device__ __forceinline__ void quad_load(QuadGroup<T, N / 4, GATE, CB>& g, int r0, int nrows, const T* xb,
                                          const T* db, const T* zb, const T* Bb, const T* Cb, int64_t D, int q) {
    constexpr int NQ = N / 4;
    const int64_t rq = r0 + q < nrows ? r0 + q : nrows - 1;
    g.x = xb[rq * D];
    g.dl = db[rq * D];
    if constexpr (GATE) g.z = zb[rq * D];
#pragma unroll
    for (int i = 0; i < kQuadGroup; ++i) {
        const int64_t r = r0 + i < nrows ? r0 + i : nrows - 1;
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
            g.b[i][k] = Bb[r * N + q * NQ + k];
            if constexpr (CB) g.c[i][k] = Cb[r * N + q * NQ + k];
        }
    }
}

// Per-channel parameters and the conv window of a quad lane.
template <int NQ, bool CONV, bool ZOH>
struct QuadChannel {
    float A2[NQ], iA[ZOH ? NQ : 1];
    float dbias, w0, w1, w2, w3, cb;
    float x3, x2, x1;                            // x_{t-3}, x_{t-2}, x_{t-1}
    __device__ __forceinline__ void init(const float* A, const float* delta_bias, const float* conv_w,
                                         const float* conv_b, int d, int q) {
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
            const float av = A[(int64_t)d * (4 * NQ) + q * NQ + k];
            const bool zero = ZOH && __builtin_fabsf(av) < kZohZeroA;
            A2[k] = zero ? 0.0f : av * kLog2e;            // ZOH: an A = 0 state decays by exactly 1
            if (ZOH) iA[k] = zero ? 0.0f : 1.0f / av;
        }
        dbias = delta_bias ? delta_bias[d] : 0.0f;
        w0 = w1 = w2 = cb = 0.0f; w3 = 1.0f;
        if (CONV) {
            w0 = conv_w[d * 4 + 0]; w1 = conv_w[d * 4 + 1]; w2 = conv_w[d * 4 + 2]; w3 = conv_w[d * 4 + 3];
            cb = conv_b ? conv_b[d] : 0.0f;
        }
        x3 = x2 = x1 = 0.0f;
    }
    // Input u (conv + SiLU, or x itself), step size and gate factor SiLU(z) of the
    // group's tokens 0..3: lane q computes those of token q, then every lane gets all
    // four by broadcast. The window advances by the m (1..4) valid tokens.
    template <typename T, bool GATE, typename G>
    __device__ __forceinline__ void group_prologue(const G& g, int q, int m, float* u, float* dt, float* gz) {
        static_assert(kQuadGroup == 4, "one token per lane of the quad");
        const float xq = IO<T>::cvt(g.x);            // x of token q
        float uq;
        if constexpr (CONV) {
            // token q's window x_{t-3}, x_{t-2}, x_{t-1}: earlier tokens of the group from
            // the lanes before q, the rest from the window carried into the group
            const float s1 = quad_dpp<kQuadPrev1>(xq), s2 = quad_dpp<kQuadPrev2>(xq), s3 = quad_bcast<0>(xq);
            const float p1 = q >= 1 ? s1 : x1;
            const float p2 = q >= 2 ? s2 : (q == 1 ? x1 : x2);
            const float p3 = q == 3 ? s3 : (q == 2 ? x1 : (q == 1 ? x2 : x3));
            uq = silu(__builtin_fmaf(w3, xq, __builtin_fmaf(w2, p1, __builtin_fmaf(w1, p2, __builtin_fmaf(w0, p3, cb)))));
            // the window after the group's m valid tokens
            const float l0 = s3, l1 = quad_bcast<1>(xq), l2 = quad_bcast<2>(xq), l3 = quad_bcast<3>(xq);
            const float o1 = x1, o2 = x2;
            if (m == 4) { x3 = l1; x2 = l2; x1 = l3; }
            else if (m == 3) { x3 = l0; x2 = l1; x1 = l2; }
            else if (m == 2) { x3 = o1; x2 = l0; x1 = l1; }
            else { x3 = o2; x2 = o1; x1 = l0; }
        } else {
            uq = xq;
        }
        const float dq = softplus(IO<T>::cvt(g.dl) + dbias);
        u[0] = quad_bcast<0>(uq); u[1] = quad_bcast<1>(uq); u[2] = quad_bcast<2>(uq); u[3] = quad_bcast<3>(uq);
        dt[0] = quad_bcast<0>(dq); dt[1] = quad_bcast<1>(dq); dt[2] = quad_bcast<2>(dq); dt[3] = quad_bcast<3>(dq);
        if constexpr (GATE) {
            const float gq = silu(IO<T>::cvt(g.z));
            gz[0] = quad_bcast<0>(gq); gz[1] = quad_bcast<1>(gq); gz[2] = quad_bcast<2>(gq); gz[3] = quad_bcast<3>(gq);
        }
    }
    // state update with step dt, input u and B row values braw; returns sum_k C_k h_k
    template <typename T, bool READ>
    __device__ __forceinline__ float update(float* h, float dt, float u, const T* braw, const T* craw) {
        const float wv = dt * u;
        float yp = 0.0f;
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
            const float tk = dt * A2[k];
            const float a = exp2_fast(tk);
            const float coef = ZOH ? zoh_coef(a, tk, dt, iA[ZOH ? k : 0]) * u : wv;
            h[k] = __builtin_fmaf(a, h[k], coef * IO<T>::cvt(braw[k]));
            if (READ) yp = __builtin_fmaf(IO<T>::cvt(craw[k]), h[k], yp);
        }
        return yp;
    }
};

// The conv window x_{t0-3}, x_{t0-2}, x_{t0-1} of a chunk starting at t0.
template <typename T>
__device__ __forceinline__ void quad_window(float& x3, float& x2, float& x1, const T* xcol, int64_t t0, int64_t D,
                                            const float* hist, int64_t bd) {
    float xh[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int64_t tt = t0 - 3 + j;
        xh[j] = tt >= 0 ? IO<T>::ld(xcol + tt * D) : (hist ? hist[bd * 3 + (3 + tt)] : 0.0f);
    }
    x3 = xh[0]; x2 = xh[1]; x1 = xh[2];
}

// Aggregates of every chunk but the last: its end state from its initial state (zero,
// or the caller's state for chunk 0) and its summed step size (accumulated in fp64);
// chunk 0 also copies the initial states for the main pass, whose last chunk
// overwrites them.
template <typename T, int N, bool CONV, bool ZOH>
__global__ void __launch_bounds__(kScanThreads)
k_agg_q(const T* __restrict__ x, const float* __restrict__ conv_w, const float* __restrict__ conv_b,
        const T* __restrict__ delta, const float* __restrict__ delta_bias, const float* __restrict__ A,
        const T* __restrict__ Bm, const float* __restrict__ ssm_state, const float* __restrict__ conv_state,
        float* __restrict__ ws_S, float* __restrict__ ws_sdt, float* __restrict__ ws_h0, float* __restrict__ ws_c0,
        ScanArgs sa) {
    constexpr int NQ = N / 4;
    const int D = sa.D;
    const int q = threadIdx.x & 3;
    const int d_raw = (blockIdx.x * kScanThreads + threadIdx.x) >> 2;
    const bool live = d_raw < D;
    const int d = live ? d_raw : D - 1;
    const int c = blockIdx.y, b = blockIdx.z;
    const int64_t t0 = (int64_t)c * sa.chunk_len;
    const int nrows = (int)sa.chunk_len;         // every chunk but the last is full
    const int64_t bd = (int64_t)b * D + d;
    QuadChannel<NQ, CONV, ZOH> ch;
    ch.init(A, delta_bias, conv_w, conv_b, d, q);
    float h[NQ];
#pragma unroll
    for (int k = 0; k < NQ; ++k) h[k] = (c == 0 && ssm_state) ? ssm_state[bd * N + q * NQ + k] : 0.0f;
    if (c == 0 && live) {
#pragma unroll
        for (int k = 0; k < NQ; ++k)
            if (ssm_state) ws_h0[bd * N + q * NQ + k] = h[k];
        if (CONV && conv_state && q == 0) {
            ws_c0[bd * 3 + 0] = conv_state[bd * 3 + 0];
            ws_c0[bd * 3 + 1] = conv_state[bd * 3 + 1];
            ws_c0[bd * 3 + 2] = conv_state[bd * 3 + 2];
        }
    }
    const T* xcol = x + (int64_t)b * sa.L * D + d;              // channel d of batch row b, token 0
    if (CONV) quad_window<T>(ch.x3, ch.x2, ch.x1, xcol, t0, D, conv_state, bd);
    const T* xb = xcol + t0 * D;
    const T* db = delta + ((int64_t)b * sa.L + t0) * D + d;
    const T* Bb = Bm + ((int64_t)b * sa.L + t0) * N;
    double sdt = 0.0;
    QuadGroup<T, NQ, false, false> g0, g1;
    auto group = [&](const QuadGroup<T, NQ, false, false>& g, int r0) {
        if (r0 >= nrows) return;                                   // uniform
        const int m = nrows - r0 < kQuadGroup ? nrows - r0 : kQuadGroup;
        float u[kQuadGroup], dt[kQuadGroup];
        ch.template group_prologue<T, false>(g, q, m, u, dt, nullptr);
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < kQuadGroup; ++i) {
            if (i >= m) break;                                     // uniform
            part += dt[i];
            ch.template update<T, false>(h, dt[i], u[i], g.b[i], nullptr);
        }
        sdt += (double)part;
    };
    quad_load<T, N, false, false>(g0, 0, nrows, xb, db, nullptr, Bb, nullptr, D, q);
    for (int r = 0; r < nrows; r += 2 * kQuadGroup) {
        quad_load<T, N, false, false>(g1, r + kQuadGroup, nrows, xb, db, nullptr, Bb, nullptr, D, q);
        group(g0, r);
        quad_load<T, N, false, false>(g0, r + 2 * kQuadGroup, nrows, xb, db, nullptr, Bb, nullptr, D, q);
        group(g1, r + kQuadGroup);
    }
    if (live) {
        const int64_t ai = ((int64_t)b * (sa.nchunks - 1) + c) * D + d;
        if (q == 0) ws_sdt[ai] = (float)sdt;
#pragma unroll
        for (int k = 0; k < NQ; ++k) ws_S[ai * N + q * NQ + k] = h[k];
    }
}

template <typename T, int N, bool CONV, bool GATE, bool ZOH>
__global__ void __launch_bounds__(kScanThreads)
k_scan_q(const T* __restrict__ x, const float* __restrict__ conv_w, const float* __restrict__ conv_b,
         const T* __restrict__ delta, const float* __restrict__ delta_bias, const float* __restrict__ A,
         const T* __restrict__ Bm, const T* __restrict__ Cm, const float* __restrict__ Dskip,
         const T* __restrict__ z, T* __restrict__ y, float* __restrict__ ssm_state, float* __restrict__ conv_state,
         const float* __restrict__ ws_S, const float* __restrict__ ws_sdt, const float* __restrict__ ws_h0,
         const float* __restrict__ ws_c0, ScanArgs sa) {
    constexpr int NQ = N / 4;
    const int D = sa.D;
    const int q = threadIdx.x & 3;
    const int d_raw = (blockIdx.x * kScanThreads + threadIdx.x) >> 2;
    const bool live = d_raw < D;
    const int d = live ? d_raw : D - 1;
    const int c = blockIdx.y, b = blockIdx.z;
    const int64_t t0 = (int64_t)c * sa.chunk_len;
    const int64_t t1 = (t0 + sa.chunk_len < sa.L) ? t0 + sa.chunk_len : sa.L;
    const int nrows = (int)(t1 - t0);
    const int nagg = sa.nchunks - 1;
    const bool multi = sa.nchunks > 1;
    const int64_t bd = (int64_t)b * D + d;
    QuadChannel<NQ, CONV, ZOH> ch;
    ch.init(A, delta_bias, conv_w, conv_b, d, q);
    const float dsk = Dskip ? Dskip[d] : 0.0f;

    // initial state: the caller's (or its copy) for chunk 0, else the fold of the
    // aggregates of chunks 0 .. c-1
    float h[NQ];
    if (c == 0) {
        const float* src = (ssm_state && multi) ? ws_h0 : ssm_state;
#pragma unroll
        for (int k = 0; k < NQ; ++k) h[k] = src ? src[bd * N + q * NQ + k] : 0.0f;
    } else {
#pragma unroll
        for (int k = 0; k < NQ; ++k) h[k] = 0.0f;
        for (int c0 = 0; c0 < c; c0 += kQuadFold) {
            float sd[kQuadFold], sv[kQuadFold][NQ];
#pragma unroll
            for (int j = 0; j < kQuadFold; ++j) {
                const int cc = c0 + j < c ? c0 + j : c - 1;      // past c: a repeated load, unused
                const int64_t ai = ((int64_t)b * nagg + cc) * D + d;
                sd[j] = ws_sdt[ai];
#pragma unroll
                for (int k = 0; k < NQ; ++k) sv[j][k] = ws_S[ai * N + q * NQ + k];
            }
#pragma unroll
            for (int j = 0; j < kQuadFold; ++j) {
                if (c0 + j < c) {                                 // uniform
#pragma unroll
                    for (int k = 0; k < NQ; ++k) h[k] = __builtin_fmaf(exp2_fast(sd[j] * ch.A2[k]), h[k], sv[j][k]);
                }
            }
        }
    }
    const T* xcol = x + (int64_t)b * sa.L * D + d;
    if (CONV) quad_window<T>(ch.x3, ch.x2, ch.x1, xcol, t0, D, conv_state ? (multi ? ws_c0 : conv_state) : nullptr, bd);
    const int64_t row0 = (int64_t)b * sa.L + t0;
    const T* xb = xcol + t0 * D;
    const T* db = delta + row0 * D + d;
    const T* zb = GATE ? z + row0 * D + d : nullptr;
    T* yb = y + row0 * D + d;
    const T* Bb = Bm + row0 * N;
    const T* Cb = Cm + row0 * N;
    QuadGroup<T, NQ, GATE, true> g0, g1;
    auto group = [&](const QuadGroup<T, NQ, GATE, true>& g, int r0) {
        if (r0 >= nrows) return;                                   // uniform
        const int m = nrows - r0 < kQuadGroup ? nrows - r0 : kQuadGroup;
        float u[kQuadGroup], dt[kQuadGroup], gz[kQuadGroup];
        ch.template group_prologue<T, GATE>(g, q, m, u, dt, gz);
#pragma unroll
        for (int i = 0; i < kQuadGroup; ++i) {
            if (i >= m) break;                                     // uniform
            const float yp = ch.template update<T, true>(h, dt[i], u[i], g.b[i], g.c[i]);
            float yv = quad_sum(yp) + dsk * u[i];
            if constexpr (GATE) yv *= gz[i];
            if (live && q == 0) IO<T>::st(yb + (int64_t)(r0 + i) * D, yv);
        }
    };
    quad_load<T, N, GATE, true>(g0, 0, nrows, xb, db, zb, Bb, Cb, D, q);
    for (int r = 0; r < nrows; r += 2 * kQuadGroup) {
        quad_load<T, N, GATE, true>(g1, r + kQuadGroup, nrows, xb, db, zb, Bb, Cb, D, q);
        group(g0, r);
        quad_load<T, N, GATE, true>(g0, r + 2 * kQuadGroup, nrows, xb, db, zb, Bb, Cb, D, q);
        group(g1, r + kQuadGroup);
    }
    if (live && c == sa.nchunks - 1) {
        if (ssm_state) {
#pragma unroll
            for (int k = 0; k < NQ; ++k) ssm_state[bd * N + q * NQ + k] = h[k];
        }
        if (CONV && conv_state && q == 0) {
            conv_state[bd * 3 + 0] = ch.x3; conv_state[bd * 3 + 1] = ch.x2; conv_state[bd * 3 + 2] = ch.x1;
        }
    }
}

// ---------------------------------------------------------------------------
// launchers (templates; each instantiation unit calls dispatch_n for its dtype and rule)

// k_scan over `grid`: once with the general decays and, from kPowMinN states on, once
// more with the power chain (each workgroup runs in one of the two, by its vote). The
// optional start event is recorded before the first launch, the stop event after the last.
template <typename T, int N, bool CONV, bool GATE, bool ZOH, bool CK, bool REV, bool PART, bool LOC = false,
          typename... Args>
static void launch_k_scan(dim3 grid, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1, Args... args) {
    if constexpr (N >= kPowMinN) {
        hipExtLaunchKernelGGL((k_scan<T, N, CONV, GATE, ZOH, CK, REV, PART, false, LOC>), grid, dim3(kScanThreads), 0,
                              st, ev0, nullptr, 0, args...);
        hipExtLaunchKernelGGL((k_scan<T, N, CONV, GATE, ZOH, CK, REV, PART, true, LOC>), grid, dim3(kScanThreads), 0,
                              st, nullptr, ev1, 0, args...);
    } else {
        hipExtLaunchKernelGGL((k_scan<T, N, CONV, GATE, ZOH, CK, REV, PART, false, LOC>), grid, dim3(kScanThreads), 0,
                              st, ev0, ev1, 0, args...);
    }
}

// The aggregate pass: as k_scan, general and power launches for the Euler form from
// kPowMinN states.
template <typename T, int N, bool CONV, bool ZOH, bool REV, typename... Args>
static void launch_k_agg(dim3 grid, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1, Args... args) {
    if constexpr (kAggPowLaunch<N, ZOH>) {
        hipExtLaunchKernelGGL((k_agg<T, N, CONV, ZOH, REV, false>), grid, dim3(kScanThreads), 0, st, ev0, nullptr, 0,
                              args...);
        hipExtLaunchKernelGGL((k_agg<T, N, CONV, ZOH, REV, true>), grid, dim3(kScanThreads), 0, st, nullptr, ev1, 0,
                              args...);
    } else {
        hipExtLaunchKernelGGL((k_agg<T, N, CONV, ZOH, REV, false>), grid, dim3(kScanThreads), 0, st, ev0, ev1, 0,
                              args...);
    }
}

// The carry correction: general and, from kPowMinN states, power launches.
template <typename T, int N, bool GATE, typename... Args>
static void launch_k_corr(dim3 grid, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1, Args... args) {
    if constexpr (N >= kPowMinN) {
        hipExtLaunchKernelGGL((k_corr<T, N, GATE, false>), grid, dim3(kScanThreads), 0, st, ev0, nullptr, 0, args...);
        hipExtLaunchKernelGGL((k_corr<T, N, GATE, true>), grid, dim3(kScanThreads), 0, st, nullptr, ev1, 0, args...);
    } else {
        hipExtLaunchKernelGGL((k_corr<T, N, GATE, false>), grid, dim3(kScanThreads), 0, st, ev0, ev1, 0, args...);
    }
}

template <typename T, int N, bool CONV, bool GATE, bool ZOH, bool REV = false, bool PART = false>
static hipError_t launch_scan_t(const LaunchScan& p) {
    const T* x = static_cast<const T*>(p.x);
    const T* dl = static_cast<const T*>(p.delta);
    const T* z = static_cast<const T*>(p.z);
    T* y = static_cast<T*>(p.y);
    hipStream_t st = static_cast<hipStream_t>(p.stream);
    ScanArgs sa{p.L, p.chunk_len, (int)p.D, p.nchunks, 0};
    const unsigned gx = (unsigned)((p.D + kScanThreads - 1) / kScanThreads);
    if constexpr (!REV && !PART && N <= 16) {
        if (p.quad) {
            // few channels: a lane quad per channel (k_agg_q / k_scan_q)
            const unsigned gq = (unsigned)((4 * p.D + kScanThreads - 1) / kScanThreads);
            if (p.nchunks > 1) {
                hipExtLaunchKernelGGL((k_agg_q<T, N, CONV, ZOH>), dim3(gq, p.nchunks - 1, (unsigned)p.batch),
                                      dim3(kScanThreads), 0, st, static_cast<hipEvent_t>(p.ev_agg[0]),
                                      static_cast<hipEvent_t>(p.ev_agg[1]), 0, x, p.conv_w, p.conv_b, dl,
                                      p.delta_bias, p.A, static_cast<const T*>(p.B), p.ssm_state, p.conv_state,
                                      p.ws_S, p.ws_sdt, p.ws_h0, p.ws_c0, sa);
            }
            hipExtLaunchKernelGGL((k_scan_q<T, N, CONV, GATE, ZOH>), dim3(gq, p.nchunks, (unsigned)p.batch),
                                  dim3(kScanThreads), 0, st, static_cast<hipEvent_t>(p.ev_main[0]),
                                  static_cast<hipEvent_t>(p.ev_main[1]), 0, x, p.conv_w, p.conv_b, dl, p.delta_bias,
                                  p.A, static_cast<const T*>(p.B), static_cast<const T*>(p.C), p.Dskip, z, y,
                                  p.ssm_state, p.conv_state, p.ws_S, p.ws_sdt, p.ws_h0, p.ws_c0, sa);
            return hipGetLastError();
        }
    }
    // the aggregate and correction passes take whole B/C tiles of full chunks (no padding
    // rows) before the last chunk
    if (p.nchunks > 1 && (p.chunk_len % kScanTile != 0 || p.chunk_len < kScanTile)) return hipErrorInvalidValue;
    if constexpr (!REV && !PART) {
        if (p.nchunks > 1 && p.chunk_len >= kCorrMinChunk) {
            // plain forward: every chunk in one pass (all but the first from zero), the
            // fold of their end states into carries, then the carries added over each
            // chunk's head
            launch_k_scan<T, N, CONV, GATE, ZOH, false, false, false, true>(
                dim3(gx, p.nchunks, (unsigned)p.batch), st, static_cast<hipEvent_t>(p.ev_main[0]),
                static_cast<hipEvent_t>(p.ev_main[1]), x, p.conv_w, p.conv_b, dl, p.delta_bias, p.A,
                static_cast<const T*>(p.B), static_cast<const T*>(p.C), p.Dskip, z, y, p.ssm_state, p.conv_state,
                p.ws_S, p.ws_sdt, p.ws_h0, p.ws_c0, static_cast<float*>(nullptr), p.ypart, sa);
            // one thread per (batch row, channel, state): chunking only happens with fewer
            // than 256 x 256 channels in all, so the grid stays small
            const int64_t nfold = p.batch * p.D * N;
            hipExtLaunchKernelGGL((k_fold<T, N>), dim3((unsigned)((nfold + kScanThreads - 1) / kScanThreads)),
                                  dim3(kScanThreads), 0, st, static_cast<hipEvent_t>(p.ev_agg[0]), nullptr, 0, x,
                                  p.A, p.ssm_state, CONV ? p.conv_state : static_cast<float*>(nullptr), p.ws_S,
                                  static_cast<const float*>(p.ws_sdt), p.batch, sa);
            launch_k_corr<T, N, GATE>(dim3(gx, p.nchunks - 1, (unsigned)p.batch), st, nullptr,
                                      static_cast<hipEvent_t>(p.ev_agg[1]), dl, p.delta_bias, p.A,
                                      static_cast<const T*>(p.C), z, y, static_cast<const float*>(p.ws_S), sa);
            return hipGetLastError();
        }
    }
    if (p.nchunks > 1) {
        launch_k_agg<T, N, CONV, ZOH, REV>(dim3(gx, p.nchunks - 1, (unsigned)p.batch), st,
                                           static_cast<hipEvent_t>(p.ev_agg[0]), static_cast<hipEvent_t>(p.ev_agg[1]),
                                           x, p.conv_w, p.conv_b, dl, p.delta_bias, p.A, static_cast<const T*>(p.B),
                                           p.ssm_state, p.conv_state, p.ws_S, p.ws_sdt, p.ws_h0, p.ws_c0, sa);
    }
    launch_k_scan<T, N, CONV, GATE, ZOH, false, REV, PART>(
        dim3(gx, p.nchunks, (unsigned)p.batch), st, static_cast<hipEvent_t>(p.ev_main[0]),
        static_cast<hipEvent_t>(p.ev_main[1]), x, p.conv_w, p.conv_b, dl, p.delta_bias, p.A,
        static_cast<const T*>(p.B), static_cast<const T*>(p.C), p.Dskip, z, y, p.ssm_state, p.conv_state, p.ws_S,
        p.ws_sdt, p.ws_h0, p.ws_c0, static_cast<float*>(nullptr), p.ypart, sa);
    return hipGetLastError();
}

template <typename T, int N, bool CONV, bool GATE, bool ZOH>
static hipError_t launch_step_t(const LaunchScan& p) {
    hipStream_t st = static_cast<hipStream_t>(p.stream);
    constexpr int per_block = kStepThreads / 4;   // channels per workgroup (a quad each)
    const unsigned gx = (unsigned)((p.D + per_block - 1) / per_block);
    const unsigned gy = (unsigned)((p.batch + kStepStreams - 1) / kStepStreams);
    hipExtLaunchKernelGGL((k_step<T, N, CONV, GATE, ZOH>), dim3(gx, gy), dim3(kStepThreads), 0, st,
                          static_cast<hipEvent_t>(p.ev_main[0]), static_cast<hipEvent_t>(p.ev_main[1]), 0,
                          static_cast<const T*>(p.x), p.conv_w, p.conv_b, static_cast<const T*>(p.delta),
                          p.delta_bias, p.A, static_cast<const T*>(p.B), static_cast<const T*>(p.C), p.Dskip,
                          static_cast<const T*>(p.z), static_cast<T*>(p.y), p.ssm_state, p.conv_state, (int)p.D,
                          (int)p.batch);
    return hipGetLastError();
}

template <typename T, int N, bool ZOH>
static hipError_t dispatch_flags(const LaunchScan& p, bool step) {
    const bool conv = p.conv_w != nullptr, gate = p.z != nullptr;
    if (step) {
        if (conv && gate) return launch_step_t<T, N, true, true, ZOH>(p);
        if (conv) return launch_step_t<T, N, true, false, ZOH>(p);
        if (gate) return launch_step_t<T, N, false, true, ZOH>(p);
        return launch_step_t<T, N, false, false, ZOH>(p);
    }
    if (p.reverse) {
        if (conv && gate) return launch_scan_t<T, N, true, true, ZOH, true>(p);
        if (conv) return launch_scan_t<T, N, true, false, ZOH, true>(p);
        if (gate) return launch_scan_t<T, N, false, true, ZOH, true>(p);
        return launch_scan_t<T, N, false, false, ZOH, true>(p);
    }
    if (p.ypart) {
        if (conv && gate) return launch_scan_t<T, N, true, true, ZOH, false, true>(p);
        if (conv) return launch_scan_t<T, N, true, false, ZOH, false, true>(p);
        if (gate) return launch_scan_t<T, N, false, true, ZOH, false, true>(p);
        return launch_scan_t<T, N, false, false, ZOH, false, true>(p);
    }
    if (conv && gate) return launch_scan_t<T, N, true, true, ZOH>(p);
    if (conv) return launch_scan_t<T, N, true, false, ZOH>(p);
    if (gate) return launch_scan_t<T, N, false, true, ZOH>(p);
    return launch_scan_t<T, N, false, false, ZOH>(p);
}

template <typename T, bool ZOH>
static hipError_t dispatch_n(const LaunchScan& p, bool step) {
    switch (p.N) {
        case 4: return dispatch_flags<T, 4, ZOH>(p, step);
        case 8: return dispatch_flags<T, 8, ZOH>(p, step);
        case 16: return dispatch_flags<T, 16, ZOH>(p, step);
        case 32: return dispatch_flags<T, 32, ZOH>(p, step);
        case 64: return dispatch_flags<T, 64, ZOH>(p, step);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace selscan
