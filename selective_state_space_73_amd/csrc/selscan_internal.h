// Internal interface between the C-ABI layer and the HIP kernels of libselscan.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "selscan.h"

namespace selscan {

constexpr int kScanThreads = 256;   // channels per workgroup of the scan kernels (4 waves)
constexpr int kStepThreads = 256;   // lanes per workgroup of the decode-step kernel (4 per channel)
constexpr int kStepStreams = 4;     // streams each lane quad of the decode-step kernel handles
constexpr int kScanTile = 64;       // tokens of B/C staged in LDS at a time
// The plain forward over several chunks adds each chunk's carry afterwards (k_fold,
// k_corr) when chunks hold at least kCorrMinChunk tokens: its cost follows the tokens
// over which the carry has not yet decayed (about 800 with steps of 0.02 on average),
// so shorter chunks take the aggregate pass (k_agg) before the main pass instead.
constexpr int64_t kCorrMinChunk = 1024;
// Lane-quad forward path (k_agg_q / k_scan_q), for d_state <= 16: taken when one lane
// per channel, even with 64-token chunks, gives fewer than kQuadMaxTileWaves waves that
// hold a channel (two per SIMD) and the quad layout at least doubles that count (its
// lanes repeat the per-token work, about 1.6 times the instructions per row). It chunks
// for about kQuadTargetLanes lanes (four waves per SIMD), with chunks of at least
// kQuadMinChunk tokens and at most kQuadMaxChunks chunks (a chunk folds the aggregates
// of every earlier one).
constexpr int64_t kQuadMaxTileWaves = 2048;
constexpr int64_t kQuadTargetLanes = 4 * 1024 * 64;
constexpr int64_t kQuadMinChunk = 16;
constexpr int64_t kQuadMaxChunks = 128;

// Everything a launch needs, already validated by the C-ABI layer.
struct LaunchScan {
    int64_t batch, L, D;
    int N;
    bool bf16;
    bool zoh;       // zero-order-hold write term instead of Euler
    bool reverse;   // the reversed pass of a bidirectional scan: reads ypart, adds its output, writes y
    bool quad;      // forward only: the lane-quad kernels (chunking of the quad rule)
    float* ypart;   // [B, L, D] fp32 forward output of a bidirectional scan (written by the
                    // forward pass when reverse is false, read by the reversed pass)
    const void* x; const float* conv_w; const float* conv_b; const void* delta; const float* delta_bias;
    const float* A; const void* B; const void* C; const float* Dskip; const void* z; void* y;
    float* ssm_state; float* conv_state;
    // chunking and workspace (scan only)
    int nchunks; int64_t chunk_len;
    float* ws_S;    // [B, nchunks, D, N] chunk end states (the aggregate pass: slots of all but the last)
    float* ws_sdt;  // [B, nchunks, D] summed step sizes (likewise)
    float* ws_h0;   // [B, D, N]
    float* ws_c0;   // [B, D, K-1]
    void* stream;
    void* ev_agg[2];   // optional hipEvent_t pair recorded around the aggregate kernel (the plain
                       // forward over several chunks: around the carry-correction kernel)
    void* ev_main[2];  // optional hipEvent_t pair recorded around the main kernel
};

// The backward: the forward's launch description (its ssm_state / conv_state are
// the initial states, read only) plus the gradients and the backward workspace.
struct LaunchBwd {
    LaunchScan f;
    const void* dy; const float* dstate_final; const float* dconv_final;
    void* dx; void* ddelta; void* dz;
    float* dB; float* dC; float* dA; float* dD; float* dconv_w; float* dconv_b; float* ddelta_bias;
    float* dstate_init; float* dconv_init;
    float* ws_ckpt;   // [B, nck, N/4, D, 4] state after every 4th token
    float* ws_Q;      // [B, nchunks-1, D, N] adjoint aggregates of chunks 1..nchunks-1
    float* ws_qsdt;   // [B, nchunks-1, D] their summed step sizes
    float* ws_dbc;    // [B, L, nblk, 2N] per-workgroup sums of dB, dC
    float* ws_par;    // [B, nchunks, D, N + 8] per-chunk parameter sums
    float* ws_dxh;    // [B, nchunks, D, 3] partial dx of each chunk's last 3 tokens
    float* ws_dc3;    // [B, nchunks, D, 3] conv-input gradient of each chunk's first 3 tokens
    int64_t nck;      // checkpoint slots per batch row
};

// Elementwise kernels of the block (selscan_block.h): one launch description for all.
// The norm reads the block input in the I/O dtype (bf16 or not); everything else is fp32.
struct LaunchBlockOps {
    enum Op { kRmsNorm, kConvSilu, kConvHistory, kConvStep } op;
    bool bf16;
    const void* in; void* out;
    const float* w; float eps;                 // RMSNorm scale and epsilon
    const float* conv_w; const float* conv_b; float* hist;
    int64_t rows; int cols;                    // rows of the norm; channels (d_model or d_inner)
    int64_t L; int64_t batch;                  // sequence length and batch (streams for the step)
    void* stream;
};
hipError_t launch_block_op(const LaunchBlockOps& p);

// Y[M, N] = X[M, K] W[N, K]^T (+ R[M, N]), row-major, fp32 accumulation (selscan_gemm.h).
// X is fp32; W is bf16 (bf16 = true: X enters the matrix cores as two bf16 terms) or fp32;
// Y and R are bf16 (y_bf16, only with bf16 weights) or fp32. The N output columns may go
// to up to three separate row-major matrices: columns [0, cols[0]) to Y[0], the next
// cols[1] to Y[1], the rest to Y[2] (cols[1] = cols[2] = 0 for a single output). R (one
// output only) may equal Y[0].
struct LaunchGemm {
    bool bf16;
    bool y_bf16;
    const void* X; const void* W; const void* R;
    void* Y[3]; int64_t cols[3];
    int64_t M, N, K;
    float* part;          // fp32 workspace of gemm_plan(...).part_bytes for split-K launches
    void* stream;
};
hipError_t launch_gemm(const LaunchGemm& p);

// Tile width, K depth per split and split count of a GEMM launch. Launches that would
// give the GPU few workgroups split K over up to kGemmMaxSplits workgroups per output
// tile; each writes an fp32 partial and a second kernel sums them in split order.
constexpr int kGemmTargetGroups = 1024;
constexpr int kGemmMaxSplits = 16;
struct GemmPlan {
    int tile;             // 64 or 128
    int bk;               // K depth of one LDS stage
    int splits;           // >= 1
    int64_t kper;         // K range of one split (a multiple of bk)
    size_t part_bytes;    // fp32 partials [splits, M, N] (0 when splits == 1)
};
inline GemmPlan gemm_plan(int64_t M, int64_t N, int64_t K, bool bf16) {
    GemmPlan g{};
    const int64_t t128 = ((N + 127) / 128) * ((M + 127) / 128);
    g.tile = t128 < 512 ? 64 : 128;
    g.bk = g.tile == 64 ? (bf16 ? 64 : 32) : (bf16 ? 32 : 16);
    const int64_t tiles = ((N + g.tile - 1) / g.tile) * ((M + g.tile - 1) / g.tile);
    const int64_t steps = (K + g.bk - 1) / g.bk;
    int64_t s = 1;
    // split while the grid is short of workgroups and every split keeps >= 2 stages
    // (a single row of output tiles, as in decode, keeps one launch: there the split's
    // second kernel would cost more than it saves)
    while (M > g.tile && s < kGemmMaxSplits && tiles * s * 2 <= kGemmTargetGroups && steps >= 4 * s) s *= 2;
    g.kper = ((steps + s - 1) / s) * g.bk;
    g.splits = (int)((K + g.kper - 1) / g.kper);
    if (g.splits < 1) g.splits = 1;
    g.part_bytes = g.splits > 1 ? (size_t)g.splits * (size_t)M * (size_t)N * sizeof(float) : 0;
    return g;
}

// Records the calling thread's error detail (ss_last_error) and returns s.
ss_status set_error(ss_status s, const char* msg);
// The scan's own dims check (ss_conv_scan_fwd / ss_step), for callers that validate first.
ss_status validate_dims(const ss_dims* d, bool step);

// One entry per instantiation unit (I/O dtype x write rule); step selects the
// decode-step kernel instead of the full-sequence scan.
hipError_t launch_f32_euler(const LaunchScan& p, bool step);
hipError_t launch_f32_zoh(const LaunchScan& p, bool step);
hipError_t launch_bf16_euler(const LaunchScan& p, bool step);
hipError_t launch_bf16_zoh(const LaunchScan& p, bool step);
hipError_t launch_bwd_f32_euler(const LaunchBwd& p);
hipError_t launch_bwd_bf16_euler(const LaunchBwd& p);
hipError_t launch_bwd_f32_zoh(const LaunchBwd& p);
hipError_t launch_bwd_bf16_zoh(const LaunchBwd& p);

}  // namespace selscan
