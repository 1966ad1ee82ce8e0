// Backward kernels of libselscan for gfx950: gradients of every input of the
// forward path (ss_conv_scan_bwd). Included by the instantiation units after
// selscan_device.h.
//
// The gradients are the chain rule through the forward's steps in reverse order.
// The adjoint of the state, g_t = dLoss/dh_t, runs backward in time:
//     g_t = C_t * dyg_t + exp(Delta_{t+1} A) g_{t+1}        (dyg_t = dy_t * SiLU(z_t))
// and every gradient is a product of g_t or dyg_t with forward quantities at the
// same token, h_t and h_{t-1} among them (ozercemkelahmet.com "Mamba", "Step 2":
// the recurrence; "Step 4": states are recomputed rather than stored; gunjandhanuka
// "Mamba", linear-time training). Pipeline, per call:
//   1. k_agg        forward chunk aggregates (as in the forward), when chunked;
//   2. k_scan<CK>   forward recompute writing the state after every 4th token;
//   3. k_bagg       per chunk (after the first): the adjoint arriving at its start
//                   from its own tokens, Q_c = sum_t prod_{k<=t} a_k C_t dyg_t, and its
//                   summed step size, so that chunk c's adjoint carry-in is the fold
//                   gamma_c = Q_{c+1} + exp(A sum Delta_{c+1}) gamma_{c+1}; swept from
//                   the chunk start, dropping state indices whose weight fell below
//                   2^-kAggCutLog2, with an exact fallback when the dropped part may matter;
//   4. k_bwd        per chunk, 4-token segments from the end: recompute the segment
//                   forward from its checkpoint (states kept in registers), then sweep
//                   it backward; channel sums of dB/dC are reduced across the lanes of
//                   a wave and the waves of a workgroup; per-channel parameter sums
//                   and the conv halo of dx at chunk ends go to the workspace;
//   5. k_bwd_sum_*  fixed-order sums of the partials (deterministic results).
#pragma once
#include "selscan_device.h"

namespace selscan {

static_assert(kCkptEvery == 4, "the backward recomputes 4-token segments");

// dW/dA of the zero-order hold near Delta A = 0: Delta^2 (1/2 + x/3 + x^2/8 + x^3/30) with
// x = t ln2 (t = Delta A log2(e), the kernels' exponent)
constexpr float kPsi1 = 0.23104906018664842f;     // ln2 / 3
constexpr float kPsi2 = 0.060056626739775174f;    // ln2^2 / 8
constexpr float kPsi3 = 0.011100821732964315f;    // ln2^3 / 30

struct BwdArgs {
    int64_t L;
    int64_t chunk_len;
    int D;
    int nchunks;
    int64_t nck;          // checkpoint slots per batch row
    int nblk;             // workgroups along d (partials of dB/dC per token)
};

// --------------------------------------------------------------------------
// Sum of V values (V a power of two, >= 4) over the 64 lanes of a wave by
// recursive halving: each level pairs lanes in the two halves of a block and
// keeps half of the values, so no lane adds a value it does not need. Levels:
// lanes 32 apart (permlane32 swap), 16 apart (permlane16 swap), then mirrored
// lanes within 16, 8, 4 and 2 lanes (DPP). On return v[i] (i < R = max(1, V/64))
// on lane l holds the total of value i + (l >> SH) * R, SH = max(0, 6 - log2 V).
template <int V> struct WaveSum {
    static constexpr int LOG = V >= 128 ? 7 : V >= 64 ? 6 : V >= 32 ? 5 : V >= 16 ? 4 : V >= 8 ? 3 : 2;
    static constexpr int R = V >= 64 ? V / 64 : 1;
    static constexpr int SH = LOG >= 6 ? 0 : 6 - LOG;
};

__device__ __forceinline__ unsigned fbits(float v) { return __builtin_bit_cast(unsigned, v); }
__device__ __forceinline__ float bitsf(unsigned v) { return __builtin_bit_cast(float, v); }

// Every control used here permutes lanes within a row of 16 (or a quad), so no source
// lane is out of range, and the sweep runs with all lanes active: bound_ctrl is set
// only because it lets the compiler fold the move into the add that consumes it.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

constexpr int kDppRowMirror = 0x140;       // lane l of a 16-lane row takes lane 15 - l
constexpr int kDppRowHalfMirror = 0x141;   // lane l of an 8-lane half row takes lane 7 - l
constexpr int kDppQuadMirror = 3 | (2 << 2) | (1 << 4) | (0 << 6);
constexpr int kDppQuadSwap = 1 | (0 << 2) | (3 << 4) | (2 << 6);

// one mirrored level: lanes whose bit B is clear keep x, the others keep y; each adds
// its mirror partner's copy of the value it keeps
template <int CTRL, int B>
__device__ __forceinline__ float mirror_level(float x, float y, int lane) {
    const bool lo = (lane & B) == 0;
    const float send = lo ? y : x;
    const float keep = lo ? x : y;
    return keep + dpp_mov<CTRL>(send);
}

template <int C, int CTRL, int B, int V>
__device__ __forceinline__ void mirror_step(float (&v)[V], int lane) {
    if constexpr (C >= 2) {
#pragma unroll
        for (int i = 0; i < C / 2; ++i) v[i] = mirror_level<CTRL, B>(v[i], v[i + C / 2], lane);
    } else {
        v[0] += dpp_mov<CTRL>(v[0]);
    }
}

template <int C> constexpr int halved() { return C >= 2 ? C / 2 : 1; }

template <int V>
__device__ __forceinline__ void wave_sum(float (&v)[V], int lane) {
    static_assert(V >= 4 && (V & (V - 1)) == 0, "power of two");
    // lanes 32 apart: v[i] keeps value i on lanes 0-31 and value i + V/2 on lanes 32-63
#pragma unroll
    for (int i = 0; i < V / 2; ++i) {
        const auto r = __builtin_amdgcn_permlane32_swap(fbits(v[i]), fbits(v[i + V / 2]), false, false);
        v[i] = bitsf(r[0]) + bitsf(r[1]);
    }
    // lanes 16 apart
#pragma unroll
    for (int i = 0; i < V / 4; ++i) {
        const auto r = __builtin_amdgcn_permlane16_swap(fbits(v[i]), fbits(v[i + V / 4]), false, false);
        v[i] = bitsf(r[0]) + bitsf(r[1]);
    }
    constexpr int C0 = V / 4;
    mirror_step<C0, kDppRowMirror, 8>(v, lane);
    constexpr int C1 = halved<C0>();
    mirror_step<C1, kDppRowHalfMirror, 4>(v, lane);
    constexpr int C2 = halved<C1>();
    mirror_step<C2, kDppQuadMirror, 2>(v, lane);
    constexpr int C3 = halved<C2>();
    mirror_step<C3, kDppQuadSwap, 1>(v, lane);
}

// --------------------------------------------------------------------------
// Adjoint chunk aggregates (chunks 1 .. nchunks-1): the adjoint that a chunk's own
// tokens send to the state before it,
//     Q_n = sum_t exp(A_n P_t) C_t[n] dyg_t,   P_t = sum of Delta over the chunk's
//                                               tokens up to and including t,
// and the chunk's summed step size (fp64 running total) for its decay exp(A sum Delta).
// The sweep runs forward from the chunk start, so the weights exp(A_n P_t) only
// shrink (A <= 0): a state index n is dropped (wave-uniformly; in pairs up to d_state
// 32, blocks of d_state/16 above) once exp(A_n P) < 2^-kAggCutLog2 on every
// lane. The dropped part is bounded by
//     |dropped part of Q_n| <= 2^-kAggCutLog2 M + Mh,
//     M  = sum over rows after the first drop, while some index is still active, of
//          max_n |C_t[n]| |dyg_t|,
//     Mh = sum over rows after every index is dropped of exp(A_max P_t) max_n |C_t[n]|
//          |dy_t z_t| (A_max the least negative A, bounding every dropped weight;
//          |SiLU(z)| < |z|), taken per 4-row group at the group's first P.
// Rows after every index is dropped only add their Delta. If that bound exceeds
// 2^-24 max_n |Q_n| (one unit roundoff of the aggregate) on any lane, the wave
// recomputes Q exactly by the backward (Horner) sweep q <- exp(Delta_t A) (q + C_t dyg_t).
// POW (from kPowMinN states): the power fast path, launched twice as the forward
// kernels; each row's weights exp(A_n P) = exp(A_0 P)^(n+1) from one exponential and a
// running power through the active blocks, which under the identity (and the gate on
// A[d, 0]) are always a prefix, as in k_agg.
template <typename T, int N, bool GATE, bool POW = false>
__global__ void __launch_bounds__(kScanThreads)
k_bagg(const T* __restrict__ delta, const float* __restrict__ delta_bias, const float* __restrict__ A,
       const T* __restrict__ Cm, const T* __restrict__ z, const T* __restrict__ dy,
       float* __restrict__ ws_Q, float* __restrict__ ws_qsdt, BwdArgs ba) {
    const int D = ba.D;
    const int d_raw = blockIdx.x * kScanThreads + threadIdx.x;
    const int d = d_raw < D ? d_raw : D - 1;      // clamped lanes repeat the last channel
    if (pow_skip<N, POW>(A + (int64_t)d * N)) return;       // the workgroup runs in the other launch
    const unsigned du = (unsigned)d;
    const int c = blockIdx.y + 1;
    const int b = blockIdx.z;
    const int64_t t0 = (int64_t)c * ba.chunk_len;
    const int64_t t1 = (t0 + ba.chunk_len < ba.L) ? t0 + ba.chunk_len : ba.L;
    const int clen = (int)(t1 - t0);
    float A2[N];
#pragma unroll
    for (int n = 0; n < N; ++n) A2[n] = A[(int64_t)d * N + n] * kLog2e;
    const float dbias = delta_bias ? delta_bias[d] : 0.0f;

    constexpr int R = kScanTile;
    constexpr int U = 4;
    constexpr int NB = N + 1;                     // C values and max_n |C| per row
    static_assert(R % (2 * U) == 0, "a tile holds whole pairs of groups");
    __shared__ float sC[2][R][NB];
    const int tid = threadIdx.x;
    constexpr int TILE_ELEMS = R * N;
    constexpr int PER_THREAD = (TILE_ELEMS + kScanThreads - 1) / kScanThreads;
    static_assert(kScanThreads % N == 0 && 64 % N == 0, "a row's N values sit in consecutive lanes of a wave");
    const int64_t rowbase = (int64_t)b * ba.L + t0;
    const T* Cc = Cm + rowbase * N;
    T tc[PER_THREAD];
    auto tile_fetch = [&](int rlo) {          // rows [rlo, rlo + R) clamped into the chunk
#pragma unroll
        for (int k = 0; k < PER_THREAD; ++k) {
            const int e0 = tid + k * kScanThreads;
            const int e = e0 < TILE_ELEMS ? e0 : TILE_ELEMS - 1;
            int r = rlo + e / N;
            r = r > clen - 1 ? clen - 1 : r;
            tc[k] = Cc[(int64_t)r * N + e % N];
        }
    };
    auto tile_store = [&](int buf) {
#pragma unroll
        for (int k = 0; k < PER_THREAD; ++k) {
            const int e = tid + k * kScanThreads;
            const float v = IO<T>::cvt(tc[k]);
            float m = __builtin_fabsf(v);
#pragma unroll
            for (int o = 1; o < N; o <<= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o, N));
            if (e < TILE_ELEMS) {
                sC[buf][e / N][e % N] = v;
                if (e % N == 0) sC[buf][e / N][N] = m;
            }
        }
    };
    const T* db = delta + rowbase * D;
    const T* zb = GATE ? z + rowbase * D : nullptr;
    const T* yb = dy + rowbase * D;

    // group j holds rows 4j .. 4j+3 (chunk-relative; rows past the chunk end are
    // padding with zero weight), loaded one group ahead into two buffers used
    // alternately; raw I/O bits zero-extended in 32-bit registers
    uint32_t ed[U], ez[U], ey[U], od[U], oz[U], oy[U];
    auto raw = [&](const T* base, int r) -> uint32_t {
        const T v = (base + (int64_t)r * D)[du];
        if constexpr (sizeof(T) == 2) return (uint32_t)v;
        else return __builtin_bit_cast(uint32_t, v);
    };
    auto val = [](uint32_t v) -> float {
        if constexpr (sizeof(T) == 2) return __builtin_bit_cast(float, v << 16);
        else return __builtin_bit_cast(float, v);
    };
    auto load_group = [&](int j, uint32_t* pd, uint32_t* pz, uint32_t* py) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
            int r = U * j + i;
            r = r < clen ? r : clen - 1;
            pd[i] = raw(db, r);
            pz[i] = GATE ? raw(zb, r) : 0u;
            py[i] = raw(yb, r);
        }
    };

    // state indices drop in blocks of BS (pairs up to d_state 32, as in k_agg); a block
    // goes once its least negative exponent A2 * P is below the cut on every lane
    constexpr int BS = N <= 32 ? 2 : N / 16;
    constexpr int NBLK = N / BS;
    static_assert(NBLK <= 32, "one mask bit per block");
    float A2blk[NBLK];
#pragma unroll
    for (int j = 0; j < NBLK; ++j) {
        float m = A2[BS * j];
#pragma unroll
        for (int k = 1; k < BS; ++k) m = __builtin_fmaxf(m, A2[BS * j + k]);
        A2blk[j] = m;
    }
    const uint32_t full = NBLK == 32 ? 0xffffffffu : (1u << NBLK) - 1u;
    uint32_t act = full;
    const float cut = -(float)kAggCutLog2;
    // the least negative exponent: once every index is dropped (all negative then),
    // exp2(A2max * P) bounds each dropped weight at P
    float A2max = A2blk[0];
#pragma unroll
    for (int j = 1; j < NBLK; ++j) A2max = __builtin_fmaxf(A2max, A2blk[j]);

    float q[N];
#pragma unroll
    for (int n = 0; n < N; ++n) q[n] = 0.0f;
    double Psum = 0.0;                            // sum of Delta over the rows swept so far
    float M = 0.0f;                               // rows after the first drop, some index still active
    float Mh = 0.0f;                              // rows after every index is dropped, weighted
    auto group = [&](int j, const uint32_t* cd, const uint32_t* cz, const uint32_t* cy, const float* tile) {
        float dt[U], dyg[U];
        bool valid[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            valid[i] = U * j + i < clen;
            dt[i] = valid[i] ? softplus(val(cd[i]) + dbias) : 0.0f;
        }
        const float pbase = (float)Psum;
        float P[U], part = 0.0f;
#pragma unroll
        for (int i = 0; i < U; ++i) { part += dt[i]; P[i] = pbase + part; }
        Psum += (double)part;
        const float* rowp = tile + (int64_t)(U * j) * NB;    // row 4j of the chunk
        if (act) {
#pragma unroll
            for (int i = 0; i < U; ++i) {
                float g = valid[i] ? val(cy[i]) : 0.0f;
                if (GATE) g *= silu(val(cz[i]));
                dyg[i] = g;
            }
            if (act != full) {
#pragma unroll
                for (int i = 0; i < U; ++i) M = __builtin_fmaf(__builtin_fabsf(dyg[i]), rowp[i * NB + N], M);
            }
            float e0[POW ? U : 1], pw[POW ? U : 1];
            if constexpr (POW) {
#pragma unroll
                for (int i = 0; i < U; ++i) { e0[i] = exp2_fast(A2[0] * P[i]); pw[i] = 1.0f; }
            }
#pragma unroll
            for (int jb = 0; jb < NBLK; ++jb) {
                if ((act >> jb) & 1u) {                  // power path: then so is every block before it
#pragma unroll
                    for (int i = 0; i < U; ++i) {
#pragma unroll
                        for (int k = 0; k < BS; ++k) {
                            const int n = BS * jb + k;
                            float w;
                            if constexpr (POW) {
                                pw[i] *= e0[i];
                                w = pw[i];
                            } else {
                                w = exp2_fast(A2[n] * P[i]);
                            }
                            q[n] = __builtin_fmaf(w, rowp[i * NB + n] * dyg[i], q[n]);
                        }
                    }
                    // weights only shrink further on: drop the block once every lane is below the cut
                    if (!__any(A2blk[jb] * (float)Psum > cut)) act &= ~(1u << jb);
                }
            }
        } else {
            // every row of the group weighs at most exp2(A2max * P) at the group's first
            // P (P only grows): one exponential per group
            const float wt = exp2_fast(A2max * pbase);
            float mg = 0.0f;
#pragma unroll
            for (int i = 0; i < U; ++i) {
                float g = valid[i] ? __builtin_fabsf(val(cy[i])) : 0.0f;
                if (GATE) g *= __builtin_fabsf(val(cz[i]));
                mg = __builtin_fmaf(g, rowp[i * NB + N], mg);
            }
            Mh = __builtin_fmaf(wt, mg, Mh);
        }
    };

    const int ntiles = (clen + R - 1) / R;
    tile_fetch(0);
    tile_store(0);
    load_group(0, ed, ez, ey);
    __syncthreads();
    int buf = 0;
    for (int k = 0; k < ntiles; ++k) {
        if (k + 1 < ntiles) tile_fetch((k + 1) * R);
        const float* tile = &sC[buf][0][0] - (int64_t)(k * R) * NB;   // chunk row r at tile + r * NB
        const int jend = (k + 1) * (R / U);
        for (int j = k * (R / U); j < jend && U * j < clen; j += 2) {
            load_group(j + 1, od, oz, oy);
            group(j, ed, ez, ey, tile);
            load_group(j + 2, ed, ez, ey);
            group(j + 1, od, oz, oy, tile);
        }
        if (k + 1 < ntiles) tile_store(buf ^ 1);
        __syncthreads();
        buf ^= 1;
    }

    float qmax = 0.0f;
#pragma unroll
    for (int n = 0; n < N; ++n) qmax = __builtin_fmaxf(qmax, __builtin_fabsf(q[n]));
    const bool bad = !(__builtin_ldexpf(M, -kAggCutLog2) + Mh <= qmax * 0x1p-24f);
    if (__any(bad)) {
        // exact backward sweep over the chunk (rare: the dropped part was not negligible)
#pragma unroll
        for (int n = 0; n < N; ++n) q[n] = 0.0f;
        double sd = 0.0;
        for (int r = clen - 1; r >= 0; --r) {
            const float dt = softplus(val(raw(db, r)) + dbias);
            float g = val(raw(yb, r));
            if (GATE) g *= silu(val(raw(zb, r)));
            sd += (double)dt;
            const T* crow = Cc + (int64_t)r * N;
#pragma unroll
            for (int n = 0; n < N; ++n) q[n] = exp2_fast(dt * A2[n]) * __builtin_fmaf(IO<T>::cvt(crow[n]), g, q[n]);
        }
        Psum = sd;
    }
    const int64_t ai = ((int64_t)b * (ba.nchunks - 1) + (c - 1)) * D + d;
    ws_qsdt[ai] = (float)Psum;
#pragma unroll
    for (int n = 0; n < N; ++n) ws_Q[ai * N + n] = q[n];
}

// --------------------------------------------------------------------------
// The backward sweep of one chunk (Euler write term). One lane owns one (b, d) as
// in the forward. The chunk is taken in 4-token segments from its end. Within a
// segment the states go in blocks of 4: each block is recomputed forward from the
// checkpoint (the state before the segment), keeping its five states h_{s-1} ..
// h_{s+3} and four decays in registers, then swept backward; the per-token sums over
// states (readout, sum g*B, sum A g a h) collect over the blocks, and the gradients
// that need them follow. Lanes past the last channel repeat it (identical stores)
// and are masked out of the channel sums.
// two waves per SIMD for the Euler form: the long per-token dependency chains
// (recompute, adjoint, lane reductions) need a second wave to overlap; the
// zero-order hold's extra per-state terms (1/A, the coefficient and its A-derivative)
// would spill under that cap, so it runs with the full register file.
//
// ZOH: the zero-order-hold write coefficient W = (exp(Delta A) - 1) / A (Delta where
// A = 0) in place of Delta. Its derivatives: dW/dDelta = exp(Delta A) and
// dW/dA = (Delta exp(Delta A) - W) / A, which cancels for small Delta A and is taken
// there as Delta^2 (1/2 + x/3 + x^2/8 + x^3/30), x = Delta A (the series of
// (x e^x - e^x + 1) / x^2; truncation below 2e-6 for |x| < 0.1).
//
// POW (from kPowMinN states): the power fast path of the forward kernels, taken by the
// workgroups whose channels all have A[d, n] = (n+1) A[d, 0] with A[d, 0] = 0 or
// <= -1/2 (launched twice, each workgroup running in one launch by its vote): the
// recompute's decays are one exponential per token and a multiply chain across the
// state blocks; under the zero-order hold the write coefficients are
// [(a_0 - 1) / A_0] G_n / (n+1) with the geometric sum G_n = 1 + a_0 + ... + a_0^n carried
// beside the chain, kept from the recompute for the sweep.
template <typename T, int N, bool CONV, bool GATE, bool ZOH = false, bool POW = false>
__global__ void __launch_bounds__(kScanThreads) __attribute__((amdgpu_waves_per_eu(N <= 16 && !ZOH ? 2 : 1)))
k_bwd(const T* __restrict__ x, const float* __restrict__ conv_w, const float* __restrict__ conv_b,
      const T* __restrict__ delta, const float* __restrict__ delta_bias, const float* __restrict__ A,
      const T* __restrict__ Bm, const T* __restrict__ Cm, const float* __restrict__ Dskip, const T* __restrict__ z,
      const float* __restrict__ ssm_state0, const float* __restrict__ conv_state0,
      const T* __restrict__ dy, const float* __restrict__ dstate_final, const float* __restrict__ dconv_final,
      T* __restrict__ dx, T* __restrict__ ddelta, T* __restrict__ dz,
      const float* __restrict__ ckpt, const float* __restrict__ ws_Q, const float* __restrict__ ws_qsdt,
      float* __restrict__ ws_dbc,        // [B, L, nblk, 2N] per-workgroup sums of dB, dC
      float* __restrict__ ws_par,        // [B, nchunks, D, N + 8] per-chunk parameter sums
      float* __restrict__ ws_dxh,        // [B, nchunks, D, 3] dx of a chunk's last 3 tokens without the next chunk's share
      float* __restrict__ ws_dc3,        // [B, nchunks, D, 3] conv-input gradient of a chunk's first 3 tokens
      float* __restrict__ dstate_init, float* __restrict__ dconv_init, BwdArgs ba) {
    static_assert(!POW || N >= kPowMinN, "power path only from kPowMinN states");
    constexpr int S = kCkptEvery;
    constexpr int V = 2 * N;                      // per token: dB partials, then dC partials
    constexpr int NBK = N < 4 ? N : 4;            // states recomputed and swept together
    const int D = ba.D;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int d_raw = blockIdx.x * kScanThreads + tid;
    const float livef = d_raw < D ? 1.0f : 0.0f;
    const int d = d_raw < D ? d_raw : D - 1;
    if (pow_skip<N, POW>(A + (int64_t)d * N)) return;       // the workgroup runs in the other launch
    const unsigned du = (unsigned)d;
    const int c = blockIdx.y, b = blockIdx.z;
    const int nC = ba.nchunks;
    const bool last = c == nC - 1;
    const int64_t L = ba.L;
    const int64_t t0 = (int64_t)c * ba.chunk_len;
    const int64_t t1 = (t0 + ba.chunk_len < L) ? t0 + ba.chunk_len : L;
    const int clen = (int)(t1 - t0);
    const int64_t bd = (int64_t)b * D + d;

    float A2[N];
    float iA[ZOH ? N : 1];                        // ZOH: 1/A (0 for the A = 0 states)
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const float av = A[(int64_t)d * N + n];
        const bool zero = ZOH && __builtin_fabsf(av) < kZohZeroA;
        A2[n] = zero ? 0.0f : av * kLog2e;
        if (ZOH) iA[n] = zero ? 0.0f : 1.0f / av;
    }
    const float dbias = delta_bias ? delta_bias[d] : 0.0f;
    const float dsk = Dskip ? Dskip[d] : 0.0f;
    float w0 = 0.f, w1 = 0.f, w2 = 0.f, w3 = 1.f, cb = 0.f;
    if (CONV) {
        w0 = conv_w[d * 4 + 0]; w1 = conv_w[d * 4 + 1]; w2 = conv_w[d * 4 + 2]; w3 = conv_w[d * 4 + 3];
        cb = conv_b ? conv_b[d] : 0.0f;
    }

    // adjoint arriving at the chunk's last state from later tokens (and the final state)
    float gc[N];
#pragma unroll
    for (int n = 0; n < N; ++n) gc[n] = dstate_final ? dstate_final[bd * N + n] : 0.0f;
    for (int cc = nC - 1; cc > c; --cc) {
        const int64_t ai = ((int64_t)b * (nC - 1) + (cc - 1)) * D + d;
        const float sdt = ws_qsdt[ai];
#pragma unroll
        for (int n = 0; n < N; ++n) gc[n] = __builtin_fmaf(exp2_fast(sdt * A2[n]), gc[n], ws_Q[ai * N + n]);
    }

    float dAacc[N];
#pragma unroll
    for (int n = 0; n < N; ++n) dAacc[n] = 0.0f;
    float dDacc = 0.f, dcbacc = 0.f, dbacc = 0.f, dcw0 = 0.f, dcw1 = 0.f, dcw2 = 0.f, dcw3 = 0.f;
    float dc1 = 0.f, dc2 = 0.f, dc3 = 0.f;       // conv-input gradient at t+1, t+2, t+3

    constexpr int R = kScanTile;
    static_assert(R % S == 0, "segments do not cross tiles");
    __shared__ float sbc[2][R][V];
    __shared__ float red[2][S][4][V];
    constexpr int TILE_ELEMS = R * N;
    constexpr int PER_THREAD = (TILE_ELEMS + kScanThreads - 1) / kScanThreads;
    const int64_t rowbase = (int64_t)b * L + t0;
    const T* Bc = Bm + rowbase * N;
    const T* Cc = Cm + rowbase * N;
    T tb[PER_THREAD], tc[PER_THREAD];
    auto tile_fetch = [&](int rlo) {
#pragma unroll
        for (int k = 0; k < PER_THREAD; ++k) {
            const int e0 = tid + k * kScanThreads;
            const int e = e0 < TILE_ELEMS ? e0 : TILE_ELEMS - 1;
            int r = rlo + e / N;
            r = r > clen - 1 ? clen - 1 : r;
            const int64_t off = (int64_t)r * N + e % N;
            tb[k] = Bc[off];
            tc[k] = Cc[off];
        }
    };
    auto tile_store = [&](int buf) {
#pragma unroll
        for (int k = 0; k < PER_THREAD; ++k) {
            const int e = tid + k * kScanThreads;
            if (e < TILE_ELEMS) {
                sbc[buf][e / N][e % N] = IO<T>::cvt(tb[k]);
                sbc[buf][e / N][N + e % N] = IO<T>::cvt(tc[k]);
            }
        }
    };
    const int64_t rowoff = rowbase * D;            // element offset of the chunk's first token
    auto ld = [&](const T* base, int r) -> T { return (base + rowoff + (int64_t)r * D)[du]; };

    const int ntiles = (clen + R - 1) / R;
    tile_fetch((ntiles - 1) * R);
    tile_store(0);
    __syncthreads();
    int buf = 0, rp = 0;
    for (int k = ntiles - 1; k >= 0; --k) {
        if (k > 0) tile_fetch((k - 1) * R);
        const int rlo = k * R;
        const int rhi = (rlo + R < clen) ? rlo + R : clen;
        const float* tile = &sbc[buf][0][0] - (int64_t)rlo * V;
        for (int s = rlo + ((rhi - 1 - rlo) / S) * S; s >= rlo; s -= S) {
            const int ns = (s + S < rhi) ? S : rhi - s;      // tokens in this segment (uniform)
            const int64_t gs = t0 + s;
            // inputs of the segment, every load issued before any is used: xw[j] = x at
            // row s - 3 + j (rows before the sequence start come from the initial
            // history, rows past the segment are not needed), delta, dy, z of its
            // tokens, and the state before it (the checkpoint, or the initial state)
            float xw[S + 3];
            T xraw[S + 3], draw[S], zraw[S], yraw[S];
#pragma unroll
            for (int j = 0; j < S + 3; ++j) {
                int r = s - 3 + j;
                r = r < clen ? r : clen - 1;
                r = t0 + r >= 0 ? r : (int)-t0;
                xraw[j] = ld(x, r);
            }
#pragma unroll
            for (int i = 0; i < S; ++i) {
                const int r = s + (i < ns ? i : ns - 1);
                draw[i] = ld(delta, r);
                yraw[i] = ld(dy, r);
                zraw[i] = GATE ? ld(z, r) : T(0);
            }
            constexpr bool CK_AHEAD = N <= 16;            // all of the state loaded at once
            const vf4* ck = reinterpret_cast<const vf4*>(ckpt) + ((int64_t)b * ba.nck + (gs > 0 ? gs / S - 1 : 0)) * (N / 4) * D + d;
            vf4 ckv[CK_AHEAD ? N / 4 : 1];
            if constexpr (CK_AHEAD) {
                if (gs > 0) {
#pragma unroll
                    for (int q = 0; q < N / 4; ++q) ckv[q] = ck[(int64_t)q * D];
                } else {
#pragma unroll
                    for (int q = 0; q < N / 4; ++q)
                        ckv[q] = ssm_state0 ? vf4{ssm_state0[bd * N + 4 * q], ssm_state0[bd * N + 4 * q + 1],
                                                  ssm_state0[bd * N + 4 * q + 2], ssm_state0[bd * N + 4 * q + 3]}
                                            : vf4{0.0f, 0.0f, 0.0f, 0.0f};
                }
            }
#pragma unroll
            for (int j = 0; j < S + 3; ++j) {
                const int64_t t = t0 + s - 3 + j;
                const bool need = (CONV || j >= 3) && j < ns + 3;
                xw[j] = !need ? 0.0f : t >= 0 ? IO<T>::cvt(xraw[j]) : (conv_state0 ? conv_state0[bd * 3 + (3 + t)] : 0.0f);
            }
            // per-token forward quantities and the gradient of the pre-gate output
            float dtv[S], uv[S], cv[S], vv[S], dyg[S], szv[S];
#pragma unroll
            for (int i = 0; i < S; ++i) {
                if (CONV) {
                    cv[i] = __builtin_fmaf(w3, xw[i + 3], __builtin_fmaf(w2, xw[i + 2], __builtin_fmaf(w1, xw[i + 1], __builtin_fmaf(w0, xw[i], cb))));
                    uv[i] = silu(cv[i]);
                } else {
                    cv[i] = 0.0f;
                    uv[i] = xw[i + 3];
                }
                vv[i] = IO<T>::cvt(draw[i]) + dbias;
                dtv[i] = softplus(vv[i]);
                const float dyv = IO<T>::cvt(yraw[i]);
                if (GATE) {
                    const float zt = IO<T>::cvt(zraw[i]);
                    szv[i] = rcp_fast(1.0f + exp2_fast(-kLog2e * zt));
                    dyg[i] = dyv * zt * szv[i];
                } else {
                    szv[i] = 1.0f;
                    dyg[i] = dyv;
                }
            }
            // per token, summed over the state blocks: readout, sum g*B (ZOH: sum g*W*B),
            // sum A g a h, and for ZOH sum g*a*B
            float yacc[S], sgB[S], sA[S], sgaB[ZOH ? S : 1];
#pragma unroll
            for (int i = 0; i < S; ++i) { yacc[i] = dsk * uv[i]; sgB[i] = 0.0f; sA[i] = 0.0f; }
            // power path: each token's base decay exp(Delta A[d, 0]) and the running power
            // a_0^(j0) carried from one state block to the next
            float pe[POW ? S : 1], pr[POW ? S : 1];
            constexpr int SZ = POW && ZOH ? S : 1;
            float pa[SZ], gsum[SZ], cz[SZ];              // zero-order hold: a_0^n, G_n, (a_0 - 1) / A_0
            if constexpr (POW) {
#pragma unroll
                for (int i = 0; i < S; ++i) {
                    const float t0 = dtv[i] * A2[0];
                    pe[i] = exp2_fast(t0);
                    pr[i] = 1.0f;
                    if constexpr (ZOH) {
                        pa[i] = 1.0f;
                        gsum[i] = 0.0f;
                        cz[i] = zoh_coef(pe[i], t0, dtv[i], iA[0]);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < (ZOH ? S : 1); ++i) sgaB[i] = 0.0f;
            // states in blocks of NBK: recompute the block over the segment from the
            // state before it, then sweep the block backward
#pragma unroll
            for (int j0 = 0; j0 < N; j0 += NBK) {
                float hs[S + 1][NBK];
                if constexpr (CK_AHEAD) {
#pragma unroll
                    for (int q = 0; q < NBK / 4; ++q) {
                        const vf4 v = ckv[j0 / 4 + q];
                        hs[0][4 * q] = v.x; hs[0][4 * q + 1] = v.y; hs[0][4 * q + 2] = v.z; hs[0][4 * q + 3] = v.w;
                    }
                } else if (gs == 0) {
#pragma unroll
                    for (int n = 0; n < NBK; ++n) hs[0][n] = ssm_state0 ? ssm_state0[bd * N + j0 + n] : 0.0f;
                } else {
#pragma unroll
                    for (int q = 0; q < NBK / 4; ++q) {
                        const vf4 v = ck[(int64_t)(j0 / 4 + q) * D];
                        hs[0][4 * q] = v.x; hs[0][4 * q + 1] = v.y; hs[0][4 * q + 2] = v.z; hs[0][4 * q + 3] = v.w;
                    }
                }
                float av[S][NBK];
                float ww[SZ][POW && ZOH ? NBK : 1];         // power path: the coefficients, kept for the sweep
#pragma unroll
                for (int i = 0; i < S; ++i) {
                    const float* brow = tile + (int64_t)(s + i) * V + j0;
                    const float wv = dtv[i] * uv[i];
#pragma unroll
                    for (int n = 0; n < NBK; ++n) {
                        const float tn = dtv[i] * A2[j0 + n];
                        if constexpr (POW) {
                            pr[i] *= pe[i];
                            av[i][n] = pr[i];
                        } else {
                            av[i][n] = exp2_fast(tn);
                        }
                        if constexpr (ZOH) {
                            // general path: the write coefficient is recomputed in the sweep
                            // below rather than kept (registers)
                            float w;
                            if constexpr (POW) {
                                gsum[i] += pa[i];
                                pa[i] *= pe[i];
                                w = (cz[i] * gsum[i]) * (1.0f / (float)(j0 + n + 1));
                                ww[i][n] = w;
                            } else {
                                w = zoh_coef(av[i][n], tn, dtv[i], iA[j0 + n]);
                            }
                            hs[i + 1][n] = __builtin_fmaf(av[i][n], hs[i][n], w * (uv[i] * brow[n]));
                        } else {
                            hs[i + 1][n] = __builtin_fmaf(av[i][n], hs[i][n], wv * brow[n]);
                        }
                    }
                }
#pragma unroll
                for (int i = S - 1; i >= 0; --i) {
                    if (i >= ns) continue;                 // uniform: only the sequence's last segment is short
                    const int r = s + i;
                    const float* brow = tile + (int64_t)r * V + j0;
                    const float* crow = tile + (int64_t)r * V + N + j0;
                    const float dygm = dyg[i] * livef;
                    const float dtum = dtv[i] * uv[i] * livef;
                    const float um = uv[i] * livef;
                    float vals[2 * NBK];
                    float ya = 0.0f, gb = 0.0f, sa = 0.0f, gab = 0.0f;
#pragma unroll
                    for (int n = 0; n < NBK; ++n) {
                        const int m = j0 + n;
                        ya = __builtin_fmaf(crow[n], hs[i + 1][n], ya);
                        const float g = __builtin_fmaf(crow[n], dyg[i], gc[m]);
                        vals[NBK + n] = dygm * hs[i + 1][n];
                        const float gq = g * (av[i][n] * hs[i][n]);
                        sa = __builtin_fmaf(A2[m], gq, sa);
                        if constexpr (ZOH) {
                            const float tn = dtv[i] * A2[m];
                            float w;
                            if constexpr (POW) w = ww[i][n];
                            else w = zoh_coef(av[i][n], tn, dtv[i], iA[m]);
                            const float gB = g * brow[n];
                            vals[n] = g * w * um;
                            gb = __builtin_fmaf(gB, w, gb);
                            gab = __builtin_fmaf(gB, av[i][n], gab);
                            const float dt2 = dtv[i] * dtv[i];
                            const float ser = dt2 * __builtin_fmaf(tn, __builtin_fmaf(tn, __builtin_fmaf(tn, kPsi3, kPsi2), kPsi1), 0.5f);
                            const float dir = __builtin_fmaf(dtv[i], av[i][n], -w) * iA[m];
                            const float dwda = __builtin_fabsf(tn) < kZohSeriesT ? ser : dir;
                            dAacc[m] = __builtin_fmaf(dtv[i], gq, __builtin_fmaf(dwda, gB * uv[i], dAacc[m]));
                        } else {
                            vals[n] = g * dtum;
                            gb = __builtin_fmaf(g, brow[n], gb);
                            dAacc[m] = __builtin_fmaf(dtv[i], gq, dAacc[m]);
                        }
                        gc[m] = av[i][n] * g;
                    }
                    yacc[i] += ya;
                    sgB[i] += gb;
                    sA[i] += sa;
                    if constexpr (ZOH) sgaB[ZOH ? i : 0] += gab;
                    // channel sums of this token's dB/dC partials of the block
                    wave_sum<2 * NBK>(vals, lane);
                    using WB = WaveSum<2 * NBK>;
                    if ((lane & ((1 << WB::SH) - 1)) == 0) {
#pragma unroll
                        for (int q = 0; q < WB::R; ++q) {
                            const int jv = q + (lane >> WB::SH) * WB::R;      // 0 .. 2*NBK-1
                            const int col = jv < NBK ? j0 + jv : N + j0 + (jv - NBK);
                            red[rp][i][wave][col] = vals[q];
                        }
                    }
                }
            }
            // per-token gradients that need every state
#pragma unroll
            for (int i = S - 1; i >= 0; --i) {
                if (i >= ns) continue;
                const int r = s + i;
                const int64_t row = (int64_t)r * D;
                if (GATE) {
                    const float zt = IO<T>::cvt(zraw[i]);
                    const float dzv = IO<T>::cvt(yraw[i]) * yacc[i] * szv[i] * __builtin_fmaf(zt, 1.0f - szv[i], 1.0f);
                    Buf<T>(dz + rowoff + row).st(IO<T>::bits(dzv), du * (unsigned)sizeof(T), 0u);
                }
                dDacc = __builtin_fmaf(dyg[i], uv[i], dDacc);
                // Euler: dW/dDelta = 1 and du gets Delta sum g B; ZOH: dW/dDelta = a and
                // du gets sum g W B directly
                const float dDelta = __builtin_fmaf(sA[i], kLn2, uv[i] * (ZOH ? sgaB[ZOH ? i : 0] : sgB[i]));
                const float dU = __builtin_fmaf(dsk, dyg[i], ZOH ? sgB[i] : dtv[i] * sgB[i]);
                const float ddel = dDelta * rcp_fast(1.0f + exp2_fast(-kLog2e * vv[i]));   // softplus' = sigmoid
                Buf<T>(ddelta + rowoff + row).st(IO<T>::bits(ddel), du * (unsigned)sizeof(T), 0u);
                dbacc += ddel;
                float dxv;
                if (CONV) {
                    const float sc = rcp_fast(1.0f + exp2_fast(-kLog2e * cv[i]));
                    const float dc = dU * sc * __builtin_fmaf(cv[i], 1.0f - sc, 1.0f);    // SiLU'
                    dcbacc += dc;
                    dcw0 = __builtin_fmaf(dc, xw[i], dcw0);
                    dcw1 = __builtin_fmaf(dc, xw[i + 1], dcw1);
                    dcw2 = __builtin_fmaf(dc, xw[i + 2], dcw2);
                    dcw3 = __builtin_fmaf(dc, xw[i + 3], dcw3);
                    dxv = __builtin_fmaf(w3, dc, __builtin_fmaf(w2, dc1, __builtin_fmaf(w1, dc2, w0 * dc3)));
                    dc3 = dc2; dc2 = dc1; dc1 = dc;
                    const int64_t t = t0 + r;
                    if (last && dconv_final && t >= L - 3) dxv += dconv_final[bd * 3 + (t - (L - 3))];
                } else {
                    dxv = dU;
                }
                if (CONV && !last && r >= clen - 3)
                    ws_dxh[(((int64_t)b * nC + c) * D + d) * 3 + (r - (clen - 3))] = dxv;
                else
                    Buf<T>(dx + rowoff + row).st(IO<T>::bits(dxv), du * (unsigned)sizeof(T), 0u);
            }
            __syncthreads();
            for (int e = tid; e < ns * V; e += kScanThreads) {
                const int i = e / V, j = e % V;
                const float sum = (red[rp][i][0][j] + red[rp][i][1][j]) + (red[rp][i][2][j] + red[rp][i][3][j]);
                ws_dbc[((rowbase + s + i) * ba.nblk + blockIdx.x) * V + j] = sum;
            }
            rp ^= 1;
        }
        if (k > 0) tile_store(buf ^ 1);
        __syncthreads();
        buf ^= 1;
    }

    float* pp = ws_par + (((int64_t)b * nC + c) * D + d) * (N + 8);
#pragma unroll
    for (int n = 0; n < N; ++n) pp[n] = dAacc[n];
    pp[N] = dDacc;
    pp[N + 1] = dcw0; pp[N + 2] = dcw1; pp[N + 3] = dcw2; pp[N + 4] = dcw3;
    pp[N + 5] = dcbacc;
    pp[N + 6] = dbacc;
    if (CONV && c > 0) {
        float* e3 = ws_dc3 + (((int64_t)b * nC + c) * D + d) * 3;
        e3[0] = dc1; e3[1] = dc2; e3[2] = dc3;
    }
    if (c == 0) {
        if (dstate_init) {
#pragma unroll
            for (int n = 0; n < N; ++n) dstate_init[bd * N + n] = gc[n];
        }
        if (CONV && dconv_init) {
            // history positions -3, -2, -1: x_{-3+k'} feeds tokens 0..2 through tap k
            float p[3] = {w0 * dc1, __builtin_fmaf(w1, dc1, w0 * dc2),
                          __builtin_fmaf(w2, dc1, __builtin_fmaf(w1, dc2, w0 * dc3))};
            if (last && dconv_final && L < 3) {
#pragma unroll
                for (int k2 = 0; k2 < 3; ++k2)
                    if (L + k2 < 3) p[L + k2] += dconv_final[bd * 3 + k2];
            }
            dconv_init[bd * 3 + 0] = p[0]; dconv_init[bd * 3 + 1] = p[1]; dconv_init[bd * 3 + 2] = p[2];
        }
    }
}

// --------------------------------------------------------------------------
// Fixed-order sums of the partials.

// dB, dC [B, L, N]: sum over the workgroups along d
template <int N>
__global__ void __launch_bounds__(256)
k_bwd_sum_dbc(const float* __restrict__ ws_dbc, float* __restrict__ dB, float* __restrict__ dC, int64_t rows, int nblk) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;    // over rows * 2N
    if (i >= rows * 2 * N) return;
    const int64_t row = i / (2 * N);
    const int j = (int)(i % (2 * N));
    float s = 0.0f;
    for (int k = 0; k < nblk; ++k) s += ws_dbc[(row * nblk + k) * 2 * N + j];
    if (j < N) dB[row * N + j] = s;
    else dC[row * N + (j - N)] = s;
}

// parameter gradients: sum over (batch row, chunk)
template <int N>
__global__ void __launch_bounds__(256)
k_bwd_sum_par(const float* __restrict__ ws_par, int parts, int D, float* __restrict__ dA, float* __restrict__ dD,
              float* __restrict__ dconv_w, float* __restrict__ dconv_b, float* __restrict__ ddelta_bias) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;    // over D * (N + 7)
    if (i >= (int64_t)D * (N + 7)) return;
    const int d = (int)(i / (N + 7));
    const int k = (int)(i % (N + 7));
    float s = 0.0f;
    for (int p = 0; p < parts; ++p) s += ws_par[((int64_t)p * D + d) * (N + 8) + k];
    if (k < N) dA[(int64_t)d * N + k] = s;
    else if (k == N) { if (dD) dD[d] = s; }
    else if (k <= N + 4) { if (dconv_w) dconv_w[d * 4 + (k - N - 1)] = s; }
    else if (k == N + 5) { if (dconv_b) dconv_b[d] = s; }
    else { if (ddelta_bias) ddelta_bias[d] = s; }
}

// dx of each chunk's last 3 tokens: the chunk's own share plus the next chunk's
template <typename T>
__global__ void __launch_bounds__(256)
k_bwd_dx_halo(const float* __restrict__ ws_dxh, const float* __restrict__ ws_dc3, const float* __restrict__ conv_w,
              T* __restrict__ dx, int64_t L, int64_t chunk_len, int nC, int D, int Bsz) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;    // over B * (nC - 1) * D
    if (i >= (int64_t)Bsz * (nC - 1) * D) return;
    const int d = (int)(i % D);
    const int c = (int)((i / D) % (nC - 1));
    const int b = (int)(i / ((int64_t)D * (nC - 1)));
    const float w0 = conv_w[d * 4 + 0], w1 = conv_w[d * 4 + 1], w2 = conv_w[d * 4 + 2];
    const float* p = ws_dxh + (((int64_t)b * nC + c) * D + d) * 3;
    const float* e = ws_dc3 + (((int64_t)b * nC + c + 1) * D + d) * 3;
    const int64_t t1 = (int64_t)(c + 1) * chunk_len;
    const float v0 = __builtin_fmaf(w0, e[0], p[0]);
    const float v1 = __builtin_fmaf(w1, e[0], __builtin_fmaf(w0, e[1], p[1]));
    const float v2 = __builtin_fmaf(w2, e[0], __builtin_fmaf(w1, e[1], __builtin_fmaf(w0, e[2], p[2])));
    IO<T>::st(dx + ((int64_t)b * L + t1 - 3) * D + d, v0);
    IO<T>::st(dx + ((int64_t)b * L + t1 - 2) * D + d, v1);
    IO<T>::st(dx + ((int64_t)b * L + t1 - 1) * D + d, v2);
}

// --------------------------------------------------------------------------
// launcher

template <typename T, int N, bool CONV, bool GATE, bool ZOH>
static hipError_t launch_bwd_t(const LaunchBwd& q) {
    const LaunchScan& p = q.f;
    hipStream_t st = static_cast<hipStream_t>(p.stream);
    const T* x = static_cast<const T*>(p.x);
    const T* dl = static_cast<const T*>(p.delta);
    const T* z = static_cast<const T*>(p.z);
    const T* Bm = static_cast<const T*>(p.B);
    const T* Cm = static_cast<const T*>(p.C);
    const unsigned gx = (unsigned)((p.D + kScanThreads - 1) / kScanThreads);
    const int nC = p.nchunks;
    ScanArgs sa{p.L, p.chunk_len, (int)p.D, nC, q.nck};
    BwdArgs ba{p.L, p.chunk_len, (int)p.D, nC, q.nck, (int)gx};
    if (nC > 1 && (p.chunk_len % kScanTile != 0 || p.chunk_len < kScanTile)) return hipErrorInvalidValue;
    if (nC > 1) {
        launch_k_agg<T, N, CONV, ZOH, false>(dim3(gx, nC - 1, (unsigned)p.batch), st, nullptr, nullptr, x, p.conv_w,
                                             p.conv_b, dl, p.delta_bias, p.A, Bm, p.ssm_state, p.conv_state, p.ws_S,
                                             p.ws_sdt, p.ws_h0, p.ws_c0, sa);
    }
    launch_k_scan<T, N, CONV, false, ZOH, true, false, false>(
        dim3(gx, nC, (unsigned)p.batch), st, nullptr, nullptr, x, p.conv_w, p.conv_b, dl, p.delta_bias, p.A, Bm, Cm,
        p.Dskip, static_cast<const T*>(nullptr), static_cast<T*>(nullptr), p.ssm_state, p.conv_state, p.ws_S,
        p.ws_sdt, p.ws_h0, p.ws_c0, q.ws_ckpt, static_cast<float*>(nullptr), sa);
    const T* dy = static_cast<const T*>(q.dy);
    if (nC > 1) {
        hipLaunchKernelGGL((k_bagg<T, N, GATE, false>), dim3(gx, nC - 1, (unsigned)p.batch), dim3(kScanThreads), 0,
                           st, dl, p.delta_bias, p.A, Cm, z, dy, q.ws_Q, q.ws_qsdt, ba);
        if constexpr (N >= kPowMinN)
            hipLaunchKernelGGL((k_bagg<T, N, GATE, true>), dim3(gx, nC - 1, (unsigned)p.batch), dim3(kScanThreads),
                               0, st, dl, p.delta_bias, p.A, Cm, z, dy, q.ws_Q, q.ws_qsdt, ba);
    }
    // the sweep (general and, from kPowMinN states, power launches; the events bracket both)
    auto sweep = [&](auto pow_tag, hipEvent_t e0, hipEvent_t e1) {
        constexpr bool P = decltype(pow_tag)::value;
        hipExtLaunchKernelGGL((k_bwd<T, N, CONV, GATE, ZOH, P>), dim3(gx, nC, (unsigned)p.batch), dim3(kScanThreads),
                              0, st, e0, e1, 0, x, p.conv_w, p.conv_b, dl, p.delta_bias, p.A, Bm, Cm, p.Dskip, z,
                              p.ssm_state, p.conv_state, dy, q.dstate_final, q.dconv_final, static_cast<T*>(q.dx),
                              static_cast<T*>(q.ddelta), static_cast<T*>(q.dz), q.ws_ckpt, q.ws_Q, q.ws_qsdt,
                              q.ws_dbc, q.ws_par, q.ws_dxh, q.ws_dc3, q.dstate_init, q.dconv_init, ba);
    };
    const hipEvent_t ev0 = static_cast<hipEvent_t>(p.ev_main[0]), ev1 = static_cast<hipEvent_t>(p.ev_main[1]);
    if constexpr (N >= kPowMinN) {
        sweep(Tag<false>{}, ev0, nullptr);
        sweep(Tag<true>{}, nullptr, ev1);
    } else {
        sweep(Tag<false>{}, ev0, ev1);
    }
    const int64_t rows = p.batch * p.L;
    hipLaunchKernelGGL((k_bwd_sum_dbc<N>), dim3((unsigned)((rows * 2 * N + 255) / 256)), dim3(256), 0, st,
                       q.ws_dbc, q.dB, q.dC, rows, (int)gx);
    hipLaunchKernelGGL((k_bwd_sum_par<N>), dim3((unsigned)((p.D * (N + 7) + 255) / 256)), dim3(256), 0, st,
                       q.ws_par, (int)(p.batch * nC), (int)p.D, q.dA, q.dD, q.dconv_w, q.dconv_b, q.ddelta_bias);
    if (CONV && nC > 1) {
        const int64_t n = p.batch * (nC - 1) * p.D;
        hipLaunchKernelGGL((k_bwd_dx_halo<T>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                           q.ws_dxh, q.ws_dc3, p.conv_w, static_cast<T*>(q.dx), p.L, p.chunk_len, nC, (int)p.D,
                           (int)p.batch);
    }
    return hipGetLastError();
}

template <typename T, int N, bool ZOH>
static hipError_t dispatch_bwd_flags(const LaunchBwd& q) {
    const bool conv = q.f.conv_w != nullptr, gate = q.f.z != nullptr;
    if (conv && gate) return launch_bwd_t<T, N, true, true, ZOH>(q);
    if (conv) return launch_bwd_t<T, N, true, false, ZOH>(q);
    if (gate) return launch_bwd_t<T, N, false, true, ZOH>(q);
    return launch_bwd_t<T, N, false, false, ZOH>(q);
}

template <typename T, bool ZOH>
static hipError_t dispatch_bwd(const LaunchBwd& q) {
    switch (q.f.N) {
        case 4: return dispatch_bwd_flags<T, 4, ZOH>(q);
        case 8: return dispatch_bwd_flags<T, 8, ZOH>(q);
        case 16: return dispatch_bwd_flags<T, 16, ZOH>(q);
        case 32: return dispatch_bwd_flags<T, 32, ZOH>(q);
        case 64: return dispatch_bwd_flags<T, 64, ZOH>(q);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace selscan
