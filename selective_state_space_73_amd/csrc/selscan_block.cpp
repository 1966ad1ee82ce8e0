// Host pipeline of the Mamba block around the scan (ss_block_fwd / ss_block_step).
//
// The block (bembew.net "Overview of Mamba (SSM) Model", "How the Mamba Block Works";
// ozercemkelahmet.com "Mamba", "The block"; inferensys.com "Mamba", block list):
// RMSNorm, a widening projection into the main branch and the gate, causal conv +
// SiLU on the main branch, step size / B / C as small projections of that branch
// (ai360xpert.com "Mamba", "The selection mechanism"), the selective scan with its
// D skip and SiLU gate, the projection back to the model width and the residual.
// Every step runs in this library's kernels: the projections are its MFMA GEMM
// (row-major activations times transposed row-major weights, fp32 accumulation), with
// the residual fused into the output projection's epilogue. The activations between the
// steps are fp32 whatever the I/O dtype, and the scan runs on its fp32 kernels: only the
// block's input, its output and the GEMM weights have the I/O dtype. With bf16 weights
// the GEMM feeds each fp32 activation to the matrix cores as two bf16 terms (hi + lo), so
// no step rounds an activation to bf16.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "selscan.h"
#include "selscan_internal.h"

namespace {

ss_status failf(ss_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    return selscan::set_error(s, buf);
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Y[M, Nout] (+)= X[M, K] * W[Nout, K]^T, all row-major; X fp32, W bf16 (bf16) or fp32,
// Y and Cres bf16 (y_bf16) or fp32. Cres (if not null) is added and may equal Y0. The Nout
// columns go to Y0 (c0 of them), Y1 (c1) and Y2 (the rest); part is the fp32 split-K
// workspace (selscan::gemm_plan).
ss_status gemm(bool bf16, bool y_bf16, int64_t M, int64_t Nout, int64_t K, const void* W, const void* X,
               const void* Cres, void* Y0, int64_t c0, void* Y1, int64_t c1, void* Y2, float* part, hipStream_t st) {
    selscan::LaunchGemm g{};
    g.bf16 = bf16;
    g.y_bf16 = y_bf16;
    g.X = X; g.W = W; g.R = Cres;
    g.Y[0] = Y0; g.Y[1] = Y1; g.Y[2] = Y2;
    g.cols[0] = c0; g.cols[1] = c1; g.cols[2] = Nout - c0 - c1;
    g.M = M; g.N = Nout; g.K = K;
    g.part = part;
    g.stream = st;
    const hipError_t e = selscan::launch_gemm(g);
    if (e != hipSuccess)
        return failf(SS_ERR_HIP, "GEMM %lld x %lld x %lld launch failed: %s", (long long)M, (long long)Nout,
                     (long long)K, hipGetErrorString(e));
    return SS_OK;
}

struct BlockLayout {
    size_t xn, xi, z, u, dr, bm, cm, delta, y, scan, part, total;
};

// the scan inside the block: fp32 activations whatever the block's I/O dtype
ss_dims scan_dims(const ss_block_dims& d, bool step) {
    ss_dims s{};
    s.batch = d.batch;
    s.seqlen = step ? 1 : d.seqlen;
    s.d_inner = d.d_inner;
    s.d_state = d.d_state;
    s.d_conv = d.d_conv;
    s.io_dtype = SS_F32;
    s.discretization = d.discretization;
    return s;
}

BlockLayout block_layout(const ss_block_dims& d, bool step) {
    BlockLayout l{};
    const size_t es = 4;                                 // every activation is fp32
    const size_t M = (size_t)d.batch * (size_t)(step ? 1 : d.seqlen);
    const size_t dm = (size_t)d.d_model, di = (size_t)d.d_inner, N = (size_t)d.d_state, R = (size_t)d.dt_rank;
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off = align256(off + bytes); return o; };
    l.xn = take(M * dm * es);
    l.xi = take(M * di * es);
    l.z = take(M * di * es);
    l.u = take(M * di * es);
    l.dr = take(M * R * es);
    l.bm = take(M * N * es);
    l.cm = take(M * N * es);
    l.delta = take(M * di * es);
    l.y = take(M * di * es);
    const ss_dims sd = scan_dims(d, step);
    l.scan = take(step ? 0 : ss_workspace_bytes(&sd));
    // fp32 partials of the projections that split K (the largest of them; one at a time)
    const bool bf16 = d.io_dtype == SS_BF16;
    const int64_t Mi = (int64_t)M;
    size_t part = 0;
    const size_t cand[] = {selscan::gemm_plan(Mi, 2 * (int64_t)di, (int64_t)dm, bf16).part_bytes,
                           selscan::gemm_plan(Mi, (int64_t)(R + 2 * N), (int64_t)di, bf16).part_bytes,
                           selscan::gemm_plan(Mi, (int64_t)di, (int64_t)R, bf16).part_bytes,
                           selscan::gemm_plan(Mi, (int64_t)dm, (int64_t)di, bf16).part_bytes};
    for (size_t c : cand) part = c > part ? c : part;
    l.part = take(part);
    l.total = off;
    return l;
}

ss_status check_block(const ss_block_dims* d, const ss_block_weights* w, const void* x, const void* out,
                      const float* ssm_state, const float* conv_state, bool step) {
    if (!d || !w) return failf(SS_ERR_INVALID_ARG, "dims or weights is NULL");
    if (d->batch < 1 || (!step && d->seqlen < 1) || d->d_model < 1 || d->d_inner < 1 || d->dt_rank < 1)
        return failf(SS_ERR_INVALID_ARG, "block sizes must be positive");
    if (d->d_model > (int64_t(1) << 20) || d->dt_rank > 4096)
        return failf(SS_ERR_INVALID_ARG, "d_model or dt_rank out of range");
    if (!(d->norm_eps > 0.0f)) return failf(SS_ERR_INVALID_ARG, "norm_eps must be positive");
    if (!x || !out) return failf(SS_ERR_INVALID_ARG, "x or out is NULL");
    const void* req[] = {w->norm_w, w->W_in, w->conv_w, w->W_x, w->W_dt, w->A, w->W_out};
    const char* names[] = {"norm_w", "W_in", "conv_w", "W_x", "W_dt", "A", "W_out"};
    for (int i = 0; i < 7; ++i)
        if (!req[i]) return failf(SS_ERR_INVALID_ARG, "weights.%s is NULL", names[i]);
    if (step && (!ssm_state || !conv_state)) return failf(SS_ERR_INVALID_ARG, "ss_block_step needs both states");
    const size_t es = d->io_dtype == SS_BF16 ? 2 : 4;
    const size_t xbytes = (size_t)d->batch * (size_t)(step ? 1 : d->seqlen) * (size_t)d->d_model * es;
    const uintptr_t x0 = (uintptr_t)x, o0 = (uintptr_t)out;
    if (x0 != o0 && x0 < o0 + xbytes && o0 < x0 + xbytes)
        return failf(SS_ERR_INVALID_ARG, "out overlaps x (only out == x is allowed)");
    const void* aligned[] = {x, out, w->W_in, w->W_x, w->W_dt, w->W_out};
    for (const void* p : aligned)
        if ((uintptr_t)p & 15u) return failf(SS_ERR_INVALID_ARG, "activations and GEMM weights must be 16-byte aligned");
    const void* f4[] = {w->norm_w, w->conv_w, w->conv_b, w->dt_bias, w->A, w->Dskip, ssm_state, conv_state};
    for (const void* p : f4)
        if ((uintptr_t)p & 3u) return failf(SS_ERR_INVALID_ARG, "parameters and states must be 4-byte aligned");
    if (ssm_state && ((uintptr_t)ssm_state & 15u)) return failf(SS_ERR_INVALID_ARG, "ssm_state not 16-byte aligned");
    if (d->d_conv != 4) return failf(SS_ERR_UNSUPPORTED, "d_conv %d: only 4 is built", d->d_conv);
    if (d->io_dtype != SS_F32 && d->io_dtype != SS_BF16)
        return failf(SS_ERR_UNSUPPORTED, "io_dtype %d unknown", d->io_dtype);
    // the scan's own checks (sizes, d_state, dtype, discretization) before anything is enqueued
    const ss_dims sd = scan_dims(*d, step);
    return selscan::validate_dims(&sd, step);
}

ss_status run_block(const ss_block_dims* d, const ss_block_weights* w, const void* x, void* out, float* ssm_state,
                    float* conv_state, void* workspace, size_t workspace_bytes, void* stream, bool step) {
    ss_status s = check_block(d, w, x, out, ssm_state, conv_state, step);
    if (s != SS_OK) return s;
    const ss_dims sd = scan_dims(*d, step);
    const BlockLayout l = block_layout(*d, step);
    if (!workspace || workspace_bytes < l.total)
        return failf(SS_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, l.total);
    if ((uintptr_t)workspace & 255u) return failf(SS_ERR_INVALID_ARG, "workspace not 256-byte aligned");
    const bool bf16 = d->io_dtype == SS_BF16;
    char* ws = static_cast<char*>(workspace);
    void* xn = ws + l.xn; void* xi = ws + l.xi; void* z = ws + l.z; void* u = ws + l.u; void* dr = ws + l.dr;
    void* bm = ws + l.bm; void* cm = ws + l.cm; void* delta = ws + l.delta; void* y = ws + l.y;
    float* part = reinterpret_cast<float*>(ws + l.part);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t L = step ? 1 : d->seqlen;
    const int64_t M = d->batch * L;
    const int64_t dm = d->d_model, di = d->d_inner, N = d->d_state, R = d->dt_rank;

    selscan::LaunchBlockOps op{};
    op.bf16 = bf16;
    op.stream = stream;
    op.op = selscan::LaunchBlockOps::kRmsNorm;
    op.in = x; op.out = xn; op.w = w->norm_w; op.eps = d->norm_eps; op.rows = M; op.cols = (int)dm;
    if (selscan::launch_block_op(op) != hipSuccess) return failf(SS_ERR_HIP, "RMSNorm launch failed");

    // in_proj: the first d_inner rows of W_in give the main branch, the next the gate
    if ((s = gemm(bf16, false, M, 2 * di, dm, w->W_in, xn, nullptr, xi, di, z, di, nullptr, part, st)) != SS_OK)
        return s;

    op = selscan::LaunchBlockOps{};
    op.bf16 = bf16;
    op.stream = stream;
    op.in = xi; op.out = u; op.conv_w = w->conv_w; op.conv_b = w->conv_b; op.hist = conv_state;
    op.cols = (int)di; op.L = L; op.batch = d->batch;
    if (step) {
        op.op = selscan::LaunchBlockOps::kConvStep;
        if (selscan::launch_block_op(op) != hipSuccess) return failf(SS_ERR_HIP, "conv step launch failed");
    } else {
        op.op = selscan::LaunchBlockOps::kConvSilu;
        if (selscan::launch_block_op(op) != hipSuccess) return failf(SS_ERR_HIP, "conv launch failed");
        if (conv_state) {
            op.op = selscan::LaunchBlockOps::kConvHistory;
            if (selscan::launch_block_op(op) != hipSuccess) return failf(SS_ERR_HIP, "conv history launch failed");
        }
    }

    // x_proj: rows [0, R) of W_x give the step-size rank, then N rows for B and N for C
    if ((s = gemm(bf16, false, M, R + 2 * N, di, w->W_x, u, nullptr, dr, R, bm, N, cm, part, st)) != SS_OK)
        return s;
    if ((s = gemm(bf16, false, M, di, R, w->W_dt, dr, nullptr, delta, di, nullptr, 0, nullptr, part, st)) != SS_OK)
        return s;

    ss_args a{};
    a.x = u; a.delta = delta; a.delta_bias = w->dt_bias; a.A = w->A; a.B = bm; a.C = cm; a.Dskip = w->Dskip;
    a.z = z; a.y = y; a.ssm_state = ssm_state;
    s = step ? ss_step(&sd, &a, stream) : ss_conv_scan_fwd(&sd, &a, ws + l.scan, ss_workspace_bytes(&sd), stream);
    if (s != SS_OK) return s;

    return gemm(bf16, bf16, M, dm, di, w->W_out, y, x, out, dm, nullptr, 0, nullptr, part, st);
}

}  // namespace

extern "C" {

size_t ss_block_workspace_bytes(const ss_block_dims* dims, int step) {
    if (!dims || dims->batch < 1 || dims->d_model < 1 || dims->d_inner < 1 || dims->dt_rank < 1 ||
        (!step && dims->seqlen < 1))
        return 0;
    return block_layout(*dims, step != 0).total;
}

ss_status ss_block_fwd(const ss_block_dims* dims, const ss_block_weights* weights, const void* x, void* out,
                       float* ssm_state, float* conv_state, void* workspace, size_t workspace_bytes, void* stream) {
    return run_block(dims, weights, x, out, ssm_state, conv_state, workspace, workspace_bytes, stream, false);
}

ss_status ss_block_step(const ss_block_dims* dims, const ss_block_weights* weights, const void* x, void* out,
                        float* ssm_state, float* conv_state, void* workspace, size_t workspace_bytes, void* stream) {
    return run_block(dims, weights, x, out, ssm_state, conv_state, workspace, workspace_bytes, stream, true);
}

}  // extern "C"
