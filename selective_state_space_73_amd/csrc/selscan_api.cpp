// C ABI of libselscan: argument validation, workspace layout, launch dispatch.
// Declared in include/selscan.h. Nothing here touches the device before all
// arguments have been validated, so a rejected call enqueues nothing.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <climits>
#include <string>

#include "selscan.h"
#include "selscan_internal.h"

namespace {

thread_local std::string g_last_error;
thread_local void* g_events[4] = {nullptr, nullptr, nullptr, nullptr};   // see ss_time_next_call

void take_events(selscan::LaunchScan& p) {
    p.ev_agg[0] = g_events[0]; p.ev_agg[1] = g_events[1];
    p.ev_main[0] = g_events[2]; p.ev_main[1] = g_events[3];
    for (void*& e : g_events) e = nullptr;
}

void drop_events() {
    for (void*& e : g_events) e = nullptr;
}

ss_status fail(ss_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

constexpr int64_t kMaxGridYZ = 65535;
constexpr int64_t kMinChunk = 64;         // shortest chunk: one B/C tile
constexpr int64_t kTargetGroups = 512;    // workgroups (of 4 waves) the scan aims to launch

bool supported_n(int n) { return n == 4 || n == 8 || n == 16 || n == 32 || n == 64; }

size_t io_size(int dt) { return dt == SS_BF16 ? 2 : 4; }

int64_t chunk_len_for(int64_t L, int64_t nc) {
    const int64_t len = (L + nc - 1) / nc;
    return nc > 1 ? (len + selscan::kScanTile - 1) / selscan::kScanTile * selscan::kScanTile : len;
}

// Chunk count for the full-sequence scan. One chunk when batch x channel
// workgroups already fill the GPU; otherwise enough chunks (each at least
// kMinChunk tokens) to reach about kTargetGroups workgroups.
int choose_chunks(const ss_dims& d) {
    const int64_t col_groups = (d.d_inner + selscan::kScanThreads - 1) / selscan::kScanThreads;
    const int64_t base = d.batch * col_groups;
    int64_t nc = 1;
    if (base < 256) nc = (kTargetGroups + base - 1) / base;
    const int64_t max_by_len = d.seqlen / kMinChunk > 0 ? d.seqlen / kMinChunk : 1;
    if (nc > max_by_len) nc = max_by_len;
    if (nc > d.seqlen) nc = d.seqlen;
    if (nc > kMaxGridYZ) nc = kMaxGridYZ;
    if (nc < 1) nc = 1;
    // equalise: every chunk has ceil(L / nc) tokens, rounded up to whole B/C tiles,
    // except the last (chunk starts are multiples of the tile, hence of the
    // backward's checkpoint spacing)
    const int64_t len = chunk_len_for(d.seqlen, nc);
    return (int)((d.seqlen + len - 1) / len);
}

// The lane-quad chunk count: about kQuadTargetLanes lanes (4 per channel), chunks of
// at least kQuadMinChunk tokens, at most kQuadMaxChunks; every chunk but the last is full.
int quad_chunks(const ss_dims& d) {
    const int64_t lanes = 4 * d.batch * d.d_inner;
    int64_t nc = (selscan::kQuadTargetLanes + lanes - 1) / lanes;
    if (nc > selscan::kQuadMaxChunks) nc = selscan::kQuadMaxChunks;
    if (nc > d.seqlen / selscan::kQuadMinChunk) nc = d.seqlen / selscan::kQuadMinChunk;
    if (nc < 1) nc = 1;
    const int64_t len = (d.seqlen + nc - 1) / nc;
    return (int)((d.seqlen + len - 1) / len);
}

// The forward's lane-quad path (k_agg_q / k_scan_q): d_state <= 16, fewer than
// kQuadMaxTileWaves channel-holding waves on the one-lane kernels with the chunks
// above, and at least twice as many on the quad kernels.
bool quad_path(const ss_dims& d) {
    if (d.d_state > 16) return false;
    const int64_t tile_waves = d.batch * ((d.d_inner + 63) / 64) * choose_chunks(d);
    if (tile_waves >= selscan::kQuadMaxTileWaves) return false;
    const int64_t quad_waves = d.batch * ((4 * d.d_inner + 63) / 64) * quad_chunks(d);
    return quad_waves >= 2 * tile_waves;
}

struct Layout {
    int nchunks = 1;
    int64_t chunk_len = 0;
    bool quad = false;
    size_t off_S = 0, off_sdt = 0, off_h0 = 0, off_c0 = 0, total = 0;
};

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// fwd: the plain forward (ss_conv_scan_fwd), which may take the lane-quad path; the
// bidirectional and backward passes keep whole-tile chunks.
Layout layout(const ss_dims& d, bool fwd = false) {
    Layout l;
    l.quad = fwd && quad_path(d);
    l.nchunks = l.quad ? quad_chunks(d) : choose_chunks(d);
    l.chunk_len = l.quad ? (d.seqlen + l.nchunks - 1) / l.nchunks : chunk_len_for(d.seqlen, l.nchunks);
    const size_t B = (size_t)d.batch, D = (size_t)d.d_inner, N = (size_t)d.d_state;
    size_t off = 0;
    if (l.nchunks > 1) {
        // a slot per chunk: the plain forward writes every chunk's end state and step sum,
        // the aggregate pass (bidirectional and backward) those of all but the last
        const size_t na = (size_t)l.nchunks;
        l.off_S = off;   off = align256(off + B * na * D * N * sizeof(float));
        l.off_sdt = off; off = align256(off + B * na * D * sizeof(float));
        l.off_h0 = off;  off = align256(off + B * D * N * sizeof(float));
        l.off_c0 = off;  off = align256(off + B * D * (size_t)(d.d_conv - 1) * sizeof(float));
    }
    l.total = off;
    return l;
}

// Backward workspace: the forward's (chunk aggregates) followed by the checkpoints,
// the adjoint aggregates and the partial sums.
struct BwdLayout {
    Layout f;
    int64_t nck = 0;
    int nblk = 0;
    size_t off_ckpt = 0, off_Q = 0, off_qsdt = 0, off_dbc = 0, off_par = 0, off_dxh = 0, off_dc3 = 0, total = 0;
};

BwdLayout bwd_layout(const ss_dims& d) {
    BwdLayout l;
    l.f = layout(d);
    const size_t B = (size_t)d.batch, L = (size_t)d.seqlen, D = (size_t)d.d_inner, N = (size_t)d.d_state;
    const size_t nC = (size_t)l.f.nchunks;
    l.nck = d.seqlen / 4;
    l.nblk = (int)((d.d_inner + selscan::kScanThreads - 1) / selscan::kScanThreads);
    size_t off = l.f.total;
    l.off_ckpt = off; off = align256(off + B * (size_t)l.nck * D * N * sizeof(float));
    l.off_Q = off;    off = align256(off + B * (nC - 1) * D * N * sizeof(float));
    l.off_qsdt = off; off = align256(off + B * (nC - 1) * D * sizeof(float));
    l.off_dbc = off;  off = align256(off + B * L * (size_t)l.nblk * 2 * N * sizeof(float));
    l.off_par = off;  off = align256(off + B * nC * D * (N + 8) * sizeof(float));
    l.off_dxh = off;  off = align256(off + B * nC * D * 3 * sizeof(float));
    l.off_dc3 = off;  off = align256(off + B * nC * D * 3 * sizeof(float));
    l.total = off;
    return l;
}

ss_status check_dims(const ss_dims* d, bool step) {
    if (!d) return fail(SS_ERR_INVALID_ARG, "dims is NULL");
    if (d->discretization != SS_EULER && d->discretization != SS_ZOH)
        return fail(SS_ERR_INVALID_ARG, "dims.discretization %d unknown", d->discretization);
    if (d->batch < 1 || d->batch > kMaxGridYZ)
        return fail(SS_ERR_INVALID_ARG, "batch %lld outside [1, %lld]", (long long)d->batch, (long long)kMaxGridYZ);
    if (!step && d->seqlen < 1) return fail(SS_ERR_INVALID_ARG, "seqlen %lld < 1", (long long)d->seqlen);
    if (d->d_inner < 1 || d->d_inner > (int64_t(1) << 26))
        return fail(SS_ERR_INVALID_ARG, "d_inner %lld outside [1, 2^26]", (long long)d->d_inner);
    if (!step && d->seqlen > INT32_MAX)
        return fail(SS_ERR_INVALID_ARG, "seqlen %lld above 2^31-1", (long long)d->seqlen);
    if (!supported_n(d->d_state)) return fail(SS_ERR_UNSUPPORTED, "d_state %d not in {4,8,16,32,64}", d->d_state);
    if (d->d_conv != 4) return fail(SS_ERR_UNSUPPORTED, "d_conv %d: only 4 is built", d->d_conv);
    if (d->io_dtype != SS_F32 && d->io_dtype != SS_BF16)
        return fail(SS_ERR_UNSUPPORTED, "io_dtype %d unknown", d->io_dtype);
    if (!step) {
        const double elems = (double)d->batch * (double)d->seqlen * (double)d->d_inner;
        if (elems > 9.0e18 / 64) return fail(SS_ERR_INVALID_ARG, "tensor too large");
    }
    return SS_OK;
}

struct Range { const void* p; size_t bytes; const char* name; };

bool overlap(const Range& a, const Range& b) {
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + a.bytes, b0 = (uintptr_t)b.p, b1 = b0 + b.bytes;
    return a0 < b1 && b0 < a1;
}

// bwd: the arguments of the backward (the forward's inputs; y is not used there, the
// outputs are checked by check_grads)
ss_status check_args(const ss_dims& d, const ss_args* a, bool step, bool bwd = false) {
    if (!a) return fail(SS_ERR_INVALID_ARG, "args is NULL");
    const int64_t L = step ? 1 : d.seqlen;
    const size_t es = io_size(d.io_dtype);
    const size_t BLD = (size_t)d.batch * (size_t)L * (size_t)d.d_inner;
    const size_t BLN = (size_t)d.batch * (size_t)L * (size_t)d.d_state;
    const size_t D = (size_t)d.d_inner, N = (size_t)d.d_state, K = (size_t)d.d_conv;
    const size_t BD = (size_t)d.batch * D;
    struct Req { const void* p; const char* name; };
    const Req req[] = {{a->x, "x"}, {a->delta, "delta"}, {a->A, "A"}, {a->B, "B"}, {a->C, "C"}, {a->y, "y"}};
    const int nreq = bwd ? 5 : 6;                  // the backward does not use y (the last entry)
    for (int i = 0; i < nreq; ++i)
        if (!req[i].p) return fail(SS_ERR_INVALID_ARG, "%s is NULL", req[i].name);
    if (step && !a->ssm_state) return fail(SS_ERR_INVALID_ARG, "ss_step needs ssm_state");
    if (step && a->conv_w && !a->conv_state) return fail(SS_ERR_INVALID_ARG, "ss_step with conv_w needs conv_state");
    if (!a->conv_w && a->conv_state) return fail(SS_ERR_INVALID_ARG, "conv_state given without conv_w");

    const Range in[] = {
        {a->x, BLD * es, "x"}, {a->delta, BLD * es, "delta"}, {a->z, BLD * es, "z"},
        {a->B, BLN * es, "B"}, {a->C, BLN * es, "C"}, {a->A, D * N * 4, "A"},
        {a->conv_w, D * K * 4, "conv_w"}, {a->conv_b, D * 4, "conv_b"},
        {a->delta_bias, D * 4, "delta_bias"}, {a->Dskip, D * 4, "Dskip"},
        {a->ssm_state, BD * N * 4, "ssm_state"}, {a->conv_state, BD * (K - 1) * 4, "conv_state"},
    };
    for (const Range& r : in)
        if (r.p && ((uintptr_t)r.p & 3u)) return fail(SS_ERR_INVALID_ARG, "%s not 4-byte aligned", r.name);
    if (!bwd && ((uintptr_t)a->y & 3u)) return fail(SS_ERR_INVALID_ARG, "y not 4-byte aligned");
    if (a->ssm_state && ((uintptr_t)a->ssm_state & 15u))
        return fail(SS_ERR_INVALID_ARG, "ssm_state not 16-byte aligned");
    const Range yr{bwd ? nullptr : a->y, BLD * es, "y"};
    for (const Range& r : in)
        if (overlap(yr, r)) return fail(SS_ERR_INVALID_ARG, "y overlaps %s", r.name);
    if (overlap(Range{a->ssm_state, BD * N * 4, "ssm_state"}, Range{a->conv_state, BD * (K - 1) * 4, "conv_state"}))
        return fail(SS_ERR_INVALID_ARG, "ssm_state overlaps conv_state");
    for (int i = 0; i < 10; ++i) {
        if (overlap(Range{a->ssm_state, BD * N * 4, "ssm_state"}, in[i]))
            return fail(SS_ERR_INVALID_ARG, "ssm_state overlaps %s", in[i].name);
        if (overlap(Range{a->conv_state, BD * (K - 1) * 4, "conv_state"}, in[i]))
            return fail(SS_ERR_INVALID_ARG, "conv_state overlaps %s", in[i].name);
    }
    return SS_OK;
}

selscan::LaunchScan make_launch(const ss_dims& d, const ss_args& a, void* stream) {
    selscan::LaunchScan p{};
    p.batch = d.batch; p.L = d.seqlen; p.D = d.d_inner; p.N = d.d_state; p.bf16 = d.io_dtype == SS_BF16;
    p.zoh = d.discretization == SS_ZOH;
    p.x = a.x; p.conv_w = a.conv_w; p.conv_b = a.conv_b; p.delta = a.delta; p.delta_bias = a.delta_bias;
    p.A = a.A; p.B = a.B; p.C = a.C; p.Dskip = a.Dskip; p.z = a.z; p.y = a.y;
    p.ssm_state = a.ssm_state; p.conv_state = a.conv_state;
    p.stream = stream;
    return p;
}

ss_status check_grads(const ss_dims& d, const ss_args* a, const ss_grads* g) {
    if (!g) return fail(SS_ERR_INVALID_ARG, "grads is NULL");
    const size_t es = io_size(d.io_dtype);
    const size_t B = (size_t)d.batch, L = (size_t)d.seqlen, D = (size_t)d.d_inner, N = (size_t)d.d_state;
    const size_t K = (size_t)d.d_conv;
    const size_t BLD = B * L * D, BLN = B * L * N;
    struct Req { const void* p; const char* name; };
    const Req req[] = {{g->dy, "dy"}, {g->dx, "dx"}, {g->ddelta, "ddelta"}, {g->dB, "dB"}, {g->dC, "dC"}, {g->dA, "dA"}};
    for (const Req& r : req)
        if (!r.p) return fail(SS_ERR_INVALID_ARG, "grads.%s is NULL", r.name);
    if (a->z && !g->dz) return fail(SS_ERR_INVALID_ARG, "grads.dz is required when z is given");
    if (!a->z && g->dz) return fail(SS_ERR_INVALID_ARG, "grads.dz given without z");
    if (!a->conv_w && (g->dconv_final || g->dconv_w || g->dconv_b || g->dconv_init))
        return fail(SS_ERR_INVALID_ARG, "conv gradients given without conv_w");
    const Range outs[] = {
        {g->dx, BLD * es, "dx"}, {g->ddelta, BLD * es, "ddelta"}, {g->dz, BLD * es, "dz"},
        {g->dB, BLN * 4, "dB"}, {g->dC, BLN * 4, "dC"}, {g->dA, D * N * 4, "dA"}, {g->dDskip, D * 4, "dDskip"},
        {g->dconv_w, D * K * 4, "dconv_w"}, {g->dconv_b, D * 4, "dconv_b"}, {g->ddelta_bias, D * 4, "ddelta_bias"},
        {g->dstate_init, B * D * N * 4, "dstate_init"}, {g->dconv_init, B * D * (K - 1) * 4, "dconv_init"},
    };
    const Range ins[] = {
        {a->x, BLD * es, "x"}, {a->delta, BLD * es, "delta"}, {a->z, BLD * es, "z"}, {a->B, BLN * es, "B"},
        {a->C, BLN * es, "C"}, {a->A, D * N * 4, "A"}, {a->conv_w, D * K * 4, "conv_w"}, {a->conv_b, D * 4, "conv_b"},
        {a->delta_bias, D * 4, "delta_bias"}, {a->Dskip, D * 4, "Dskip"},
        {a->ssm_state, B * D * N * 4, "ssm_state"}, {a->conv_state, B * D * (K - 1) * 4, "conv_state"},
        {g->dy, BLD * es, "dy"}, {g->dstate_final, B * D * N * 4, "dstate_final"},
        {g->dconv_final, B * D * (K - 1) * 4, "dconv_final"},
    };
    for (const Range& r : outs)
        if (r.p && ((uintptr_t)r.p & 3u)) return fail(SS_ERR_INVALID_ARG, "%s not 4-byte aligned", r.name);
    for (const Range& r : ins)
        if (r.p && ((uintptr_t)r.p & 3u)) return fail(SS_ERR_INVALID_ARG, "%s not 4-byte aligned", r.name);
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
        for (const Range& r : ins)
            if (overlap(outs[i], r)) return fail(SS_ERR_INVALID_ARG, "%s overlaps %s", outs[i].name, r.name);
        for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
            if (overlap(outs[i], outs[j])) return fail(SS_ERR_INVALID_ARG, "%s overlaps %s", outs[i].name, outs[j].name);
    }
    return SS_OK;
}

hipError_t launch(const selscan::LaunchScan& p, bool step) {
    if (p.bf16) return p.zoh ? selscan::launch_bf16_zoh(p, step) : selscan::launch_bf16_euler(p, step);
    return p.zoh ? selscan::launch_f32_zoh(p, step) : selscan::launch_f32_euler(p, step);
}

// Bidirectional workspace: the scan's (used by each pass in turn), then the forward
// pass's fp32 output [B, L, D].
Layout bidir_layout(const ss_dims& d, size_t* off_part = nullptr) {
    Layout l = layout(d);
    const size_t off = align256(l.total);
    if (off_part) *off_part = off;
    l.total = off + (size_t)d.batch * (size_t)d.seqlen * (size_t)d.d_inner * sizeof(float);
    return l;
}

// The workspace of a full-sequence call: size, alignment, no overlap with the arguments.
ss_status check_workspace(const Layout& l, const ss_args& a, const void* workspace, size_t workspace_bytes) {
    if (l.total > 0 && (!workspace || workspace_bytes < l.total))
        return fail(SS_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, l.total);
    if (workspace && ((uintptr_t)workspace & 255u)) return fail(SS_ERR_INVALID_ARG, "workspace not 256-byte aligned");
    const Range wr{workspace, l.total, "workspace"};
    const Range others[] = {{a.x, 1, "x"}, {a.y, 1, "y"}, {a.B, 1, "B"}, {a.C, 1, "C"},
                            {a.delta, 1, "delta"}, {a.ssm_state, 1, "ssm_state"}};
    for (const Range& r : others)
        if (overlap(wr, r)) return fail(SS_ERR_INVALID_ARG, "workspace overlaps %s", r.name);
    return SS_OK;
}

void attach_workspace(selscan::LaunchScan& p, const Layout& l, void* workspace) {
    char* ws = static_cast<char*>(workspace);
    p.nchunks = l.nchunks;
    p.chunk_len = l.chunk_len;
    p.quad = l.quad;
    if (l.nchunks > 1) {
        p.ws_S = reinterpret_cast<float*>(ws + l.off_S);
        p.ws_sdt = reinterpret_cast<float*>(ws + l.off_sdt);
        p.ws_h0 = reinterpret_cast<float*>(ws + l.off_h0);
        p.ws_c0 = reinterpret_cast<float*>(ws + l.off_c0);
    }
}

}  // namespace

namespace selscan {
ss_status set_error(ss_status s, const char* msg) {
    g_last_error = msg;
    return s;
}
ss_status validate_dims(const ss_dims* d, bool step) { return check_dims(d, step); }
}  // namespace selscan

extern "C" {

size_t ss_workspace_bytes(const ss_dims* dims) {
    if (check_dims(dims, false) != SS_OK) return 0;
    return layout(*dims, true).total;
}

ss_status ss_scan_plan(const ss_dims* dims, int32_t pass, ss_plan* plan) {
    if (!plan) return fail(SS_ERR_INVALID_ARG, "plan is NULL");
    if (pass != SS_PASS_FWD && pass != SS_PASS_BIDIR && pass != SS_PASS_BWD)
        return fail(SS_ERR_INVALID_ARG, "pass %d unknown", pass);
    const ss_status s = check_dims(dims, false);
    if (s != SS_OK) return s;
    const Layout l = layout(*dims, pass == SS_PASS_FWD);
    plan->nchunks = l.nchunks;
    plan->chunk_len = l.chunk_len;
    plan->lane_quad = l.quad ? 1 : 0;
    plan->carry_correction =
        (pass == SS_PASS_FWD && l.nchunks > 1 && !l.quad && l.chunk_len >= selscan::kCorrMinChunk) ? 1 : 0;
    return SS_OK;
}

size_t ss_bidir_workspace_bytes(const ss_dims* dims) {
    if (check_dims(dims, false) != SS_OK) return 0;
    return bidir_layout(*dims).total;
}

ss_status ss_conv_scan_fwd(const ss_dims* dims, const ss_args* args, void* workspace,
                           size_t workspace_bytes, void* stream) {
    ss_status s = check_dims(dims, false);
    if (s == SS_OK) s = check_args(*dims, args, false);
    const Layout l = s == SS_OK ? layout(*dims, true) : Layout{};
    if (s == SS_OK) s = check_workspace(l, *args, workspace, workspace_bytes);
    if (s != SS_OK) { drop_events(); return s; }

    selscan::LaunchScan p = make_launch(*dims, *args, stream);
    take_events(p);
    attach_workspace(p, l, workspace);
    const hipError_t e = launch(p, false);
    if (e != hipSuccess) return fail(SS_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return SS_OK;
}

ss_status ss_conv_scan_bidir_fwd(const ss_dims* dims, const ss_args* args, const ss_dir_args* rev,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    ss_status s = check_dims(dims, false);
    if (s == SS_OK) s = check_args(*dims, args, false);
    if (s == SS_OK && (args->ssm_state || args->conv_state))
        s = fail(SS_ERR_INVALID_ARG, "a bidirectional scan takes no states (ssm_state and conv_state must be NULL)");
    // the backward direction: the forward's arguments with its own parameters
    ss_args ra{};
    if (s == SS_OK) {
        ra = *args;
        if (rev) {
            ra.conv_w = rev->conv_w; ra.conv_b = rev->conv_b; ra.delta = rev->delta; ra.delta_bias = rev->delta_bias;
            ra.A = rev->A; ra.B = rev->B; ra.C = rev->C; ra.Dskip = rev->Dskip;
        }
        s = check_args(*dims, &ra, false);
        if (s != SS_OK) s = fail(s, "backward direction: %s", std::string(g_last_error).c_str());
    }
    size_t off_part = 0;
    const Layout l = s == SS_OK ? bidir_layout(*dims, &off_part) : Layout{};
    if (s == SS_OK) s = check_workspace(l, *args, workspace, workspace_bytes);
    if (s == SS_OK) s = check_workspace(l, ra, workspace, workspace_bytes);
    if (s != SS_OK) { drop_events(); return s; }

    // forward pass (its gated output to the fp32 buffer), then the reversed pass (adds
    // its own and writes y); the scan's part of the workspace is reused in stream order
    float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + off_part);
    selscan::LaunchScan pf = make_launch(*dims, *args, stream);
    attach_workspace(pf, l, workspace);
    pf.ypart = part;
    selscan::LaunchScan pr = make_launch(*dims, ra, stream);
    pr.reverse = true;
    pr.ypart = part;
    take_events(pr);
    attach_workspace(pr, l, workspace);
    hipError_t e = launch(pf, false);
    if (e == hipSuccess) e = launch(pr, false);
    if (e != hipSuccess) return fail(SS_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return SS_OK;
}

ss_status ss_step(const ss_dims* dims, const ss_args* args, void* stream) {
    ss_status s = check_dims(dims, true);
    if (s == SS_OK) s = check_args(*dims, args, true);
    if (s != SS_OK) { drop_events(); return s; }
    ss_dims one = *dims;
    one.seqlen = 1;
    selscan::LaunchScan p = make_launch(one, *args, stream);
    take_events(p);
    const hipError_t e = launch(p, true);
    if (e != hipSuccess) return fail(SS_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return SS_OK;
}

size_t ss_bwd_workspace_bytes(const ss_dims* dims) {
    if (check_dims(dims, false) != SS_OK) return 0;
    return bwd_layout(*dims).total;
}

ss_status ss_conv_scan_bwd(const ss_dims* dims, const ss_args* args, const ss_grads* grads, void* workspace,
                           size_t workspace_bytes, void* stream) {
    ss_status s = check_dims(dims, false);
    if (s == SS_OK) s = check_args(*dims, args, false, true);
    if (s == SS_OK) s = check_grads(*dims, args, grads);
    if (s != SS_OK) { drop_events(); return s; }
    const BwdLayout l = bwd_layout(*dims);
    if (!workspace || workspace_bytes < l.total) {
        drop_events();
        return fail(SS_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, l.total);
    }
    if ((uintptr_t)workspace & 255u) { drop_events(); return fail(SS_ERR_INVALID_ARG, "workspace not 256-byte aligned"); }
    const Range wr{workspace, l.total, "workspace"};
    const Range others[] = {{args->x, 1, "x"}, {args->B, 1, "B"}, {args->C, 1, "C"}, {args->delta, 1, "delta"},
                            {args->ssm_state, 1, "ssm_state"}, {grads->dy, 1, "dy"}, {grads->dx, 1, "dx"},
                            {grads->ddelta, 1, "ddelta"}, {grads->dB, 1, "dB"}, {grads->dC, 1, "dC"},
                            {grads->dA, 1, "dA"}};
    for (const Range& r : others)
        if (overlap(wr, r)) { drop_events(); return fail(SS_ERR_INVALID_ARG, "workspace overlaps %s", r.name); }

    selscan::LaunchBwd q{};
    q.f = make_launch(*dims, *args, stream);
    q.f.y = nullptr;
    take_events(q.f);
    char* ws = static_cast<char*>(workspace);
    q.f.nchunks = l.f.nchunks;
    q.f.chunk_len = l.f.chunk_len;
    if (l.f.nchunks > 1) {
        q.f.ws_S = reinterpret_cast<float*>(ws + l.f.off_S);
        q.f.ws_sdt = reinterpret_cast<float*>(ws + l.f.off_sdt);
        q.f.ws_h0 = reinterpret_cast<float*>(ws + l.f.off_h0);
        q.f.ws_c0 = reinterpret_cast<float*>(ws + l.f.off_c0);
    }
    q.dy = grads->dy; q.dstate_final = grads->dstate_final; q.dconv_final = grads->dconv_final;
    q.dx = grads->dx; q.ddelta = grads->ddelta; q.dz = grads->dz;
    q.dB = grads->dB; q.dC = grads->dC; q.dA = grads->dA; q.dD = grads->dDskip;
    q.dconv_w = grads->dconv_w; q.dconv_b = grads->dconv_b; q.ddelta_bias = grads->ddelta_bias;
    q.dstate_init = grads->dstate_init; q.dconv_init = grads->dconv_init;
    q.ws_ckpt = reinterpret_cast<float*>(ws + l.off_ckpt);
    q.ws_Q = reinterpret_cast<float*>(ws + l.off_Q);
    q.ws_qsdt = reinterpret_cast<float*>(ws + l.off_qsdt);
    q.ws_dbc = reinterpret_cast<float*>(ws + l.off_dbc);
    q.ws_par = reinterpret_cast<float*>(ws + l.off_par);
    q.ws_dxh = reinterpret_cast<float*>(ws + l.off_dxh);
    q.ws_dc3 = reinterpret_cast<float*>(ws + l.off_dc3);
    q.nck = l.nck;
    const hipError_t e = q.f.bf16 ? (q.f.zoh ? selscan::launch_bwd_bf16_zoh(q) : selscan::launch_bwd_bf16_euler(q))
                                  : (q.f.zoh ? selscan::launch_bwd_f32_zoh(q) : selscan::launch_bwd_f32_euler(q));
    if (e != hipSuccess) return fail(SS_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return SS_OK;
}

ss_status ss_time_next_call(void* agg_start, void* agg_stop, void* main_start, void* main_stop) {
    g_events[0] = agg_start; g_events[1] = agg_stop; g_events[2] = main_start; g_events[3] = main_stop;
    return SS_OK;
}

const char* ss_status_str(ss_status s) {
    switch (s) {
        case SS_OK: return "ok";
        case SS_ERR_INVALID_ARG: return "invalid argument";
        case SS_ERR_UNSUPPORTED: return "unsupported configuration";
        case SS_ERR_WORKSPACE: return "workspace missing or too small";
        case SS_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* ss_last_error(void) { return g_last_error.c_str(); }

int ss_version(void) { return SS_VERSION; }

}  // extern "C"
