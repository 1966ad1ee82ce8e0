// Host-side launch walk (CPU test infrastructure; no GPU code).
//
// Part 1, the block pipeline: ss_block_fwd / ss_block_step run on the host against
// fake, non-overlapping device address ranges, with the kernel launchers replaced by
// recorders (mock_launch.cpp). Every recorded launch is then checked: each pointer it
// reads or writes, over the extent the kernel covers (GEMM operands, outputs, residual
// and split-K partials from the library's own gemm_plan; the norm and conv rows; the
// scan's inputs, states and chunk workspace), must lie inside one registered buffer, and
// ranges of different workspace slices must not overlap. GEMM K splits must all be
// non-empty and every grid extent within the launch limits.
//
// Part 2, the aggregate pass's index arithmetic: a host transcription of the row,
// tile and LDS-row indices one lane of k_agg visits (tile fetch rows, delta and x rows
// of each prefetched group, the staged-row reads of each group, the conv window's rows
// before the chunk) for every chunk of a sequence, checked against [0, L) and the tile.
//
// Prints one line per case and "FAIL ..." lines for violations; exits 1 on any.
#include <cinttypes>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "selscan.h"
#include "selscan_internal.h"
#include "walk.h"

namespace {

struct Buf { std::string name; uintptr_t base; size_t size; bool ws; };
std::vector<Buf> bufs;
uintptr_t next_addr = uintptr_t(1) << 40;
int failures = 0;
bool plant = false;

void fail(const std::string& what) {
    std::printf("FAIL %s\n", what.c_str());
    ++failures;
}

uintptr_t alloc(const std::string& name, size_t size, bool ws = false) {
    const uintptr_t a = next_addr;
    bufs.push_back({name, a, size, ws});
    next_addr += ((size + 4095) / 4096) * 4096 + (1 << 20);
    return a;
}

struct Use { std::string role; uintptr_t a, b; };
std::vector<Use> ws_uses;     // ranges used inside the workspace, for the overlap check

void check(const char* role, const void* p, size_t bytes) {
    if (!p || bytes == 0) return;
    const uintptr_t a = (uintptr_t)p;
    for (const Buf& b : bufs) {
        if (a >= b.base && a < b.base + b.size) {
            if (a + bytes > b.base + b.size)
                fail(std::string(role) + ": " + std::to_string(bytes) + " bytes at offset " +
                     std::to_string(a - b.base) + " run past " + b.name + " (" + std::to_string(b.size) + " bytes)");
            if (b.ws) ws_uses.push_back({role, a, a + bytes});
            return;
        }
    }
    fail(std::string(role) + ": pointer outside every buffer");
}

void check_gemm(const selscan::LaunchGemm& g) {
    const size_t ew = g.bf16 ? 2 : 4, ey = g.y_bf16 ? 2 : 4;
    const int64_t M = g.M, N = g.N, K = g.K;
    check("gemm X", g.X, (size_t)M * K * 4);
    check("gemm W", g.W, (size_t)N * K * ew);
    const int64_t c2 = N - g.cols[0] - g.cols[1];
    const int64_t cols[3] = {g.cols[0], g.cols[1], c2};
    for (int i = 0; i < 3; ++i)
        if (cols[i] > 0) check("gemm Y", g.Y[i], (size_t)M * cols[i] * ey);
    if (c2 < 0) fail("gemm: output columns exceed N");
    if (g.R) check("gemm residual", g.R, (size_t)M * N * ey);
    const selscan::GemmPlan p = selscan::gemm_plan(M, N, K, g.bf16);
    if (p.splits > 1) {
        if (!g.part) fail("gemm: split K without a partial buffer");
        check("gemm partials", g.part, (size_t)p.splits * M * N * 4);
        if (p.part_bytes != (size_t)p.splits * M * N * 4) fail("gemm: part_bytes disagrees with the splits");
    }
    const int64_t kall = (K + p.bk - 1) / p.bk;
    for (int z = 0; z < p.splits; ++z)
        if ((int64_t)z * (p.kper / p.bk) >= kall) fail("gemm: empty K split");
    const int64_t gx = (N + p.tile - 1) / p.tile, gy = (M + p.tile - 1) / p.tile;
    if (gx > INT32_MAX || gy > 65535 || p.splits > 65535) fail("gemm: grid extent");
}

void check_op(const selscan::LaunchBlockOps& o) {
    const size_t eio = o.bf16 ? 2 : 4;
    switch (o.op) {
        case selscan::LaunchBlockOps::kRmsNorm:
            check("norm in", o.in, (size_t)o.rows * o.cols * eio);
            check("norm out", o.out, (size_t)o.rows * o.cols * 4);
            check("norm w", o.w, (size_t)o.cols * 4);
            break;
        case selscan::LaunchBlockOps::kConvSilu:
            check("conv in", o.in, (size_t)o.batch * o.L * o.cols * 4);
            check("conv out", o.out, (size_t)o.batch * o.L * o.cols * 4);
            check("conv hist", o.hist, (size_t)o.batch * o.cols * 3 * 4);
            check("conv w", o.conv_w, (size_t)o.cols * 16);
            if (o.batch > 65535) fail("conv: grid z extent");
            break;
        case selscan::LaunchBlockOps::kConvHistory:
            check("conv-history in", o.in, (size_t)o.batch * o.L * o.cols * 4);
            check("conv-history hist", o.hist, (size_t)o.batch * o.cols * 3 * 4);
            break;
        case selscan::LaunchBlockOps::kConvStep:
            check("conv-step in", o.in, (size_t)o.batch * o.cols * 4);
            check("conv-step out", o.out, (size_t)o.batch * o.cols * 4);
            check("conv-step hist", o.hist, (size_t)o.batch * o.cols * 3 * 4);
            break;
    }
}

void check_scan(const selscan::LaunchScan& p, bool step, bool bf16) {
    const size_t es = bf16 ? 2 : 4;
    const int64_t L = step ? 1 : p.L;
    const size_t BLD = (size_t)p.batch * L * p.D, BLN = (size_t)p.batch * L * p.N;
    check("scan x", p.x, BLD * es);
    check("scan delta", p.delta, BLD * es);
    check("scan z", p.z, BLD * es);
    check("scan y", p.y, BLD * es);
    check("scan B", p.B, BLN * es);
    check("scan C", p.C, BLN * es);
    check("scan A", p.A, (size_t)p.D * p.N * 4);
    check("scan delta_bias", p.delta_bias, (size_t)p.D * 4);
    check("scan Dskip", p.Dskip, (size_t)p.D * 4);
    check("scan ssm_state", p.ssm_state, (size_t)p.batch * p.D * p.N * 4);
    check("scan conv_state", p.conv_state, (size_t)p.batch * p.D * 3 * 4);
    if (!step && p.nchunks > 1) {
        // the plain forward's main pass writes a slot per chunk (k_corr reads them back)
        const size_t na = (size_t)p.nchunks;
        check("scan ws_S", p.ws_S, (size_t)p.batch * na * p.D * p.N * 4);
        check("scan ws_sdt", p.ws_sdt, (size_t)p.batch * na * p.D * 4);
        check("scan ws_h0", p.ws_h0, (size_t)p.batch * p.D * p.N * 4);
        check("scan ws_c0", p.ws_c0, (size_t)p.batch * p.D * 3 * 4);
        if ((int64_t)(p.nchunks - 1) * p.chunk_len >= p.L) fail("scan: last chunk empty");
        // k_corr reads the last three rows of x for the final conv history
        if (!p.quad && p.L < 3) fail("scan: sequence shorter than the conv history");
        if (!p.quad && (p.chunk_len % selscan::kScanTile != 0)) fail("scan: chunk not whole tiles");
        if ((int64_t)p.nchunks * p.chunk_len < p.L) fail("scan: chunks do not cover L");
    }
    if (p.batch > 65535 || p.nchunks > 65535) fail("scan: grid extent");
}

void check_ws_overlap() {
    for (size_t i = 0; i < ws_uses.size(); ++i)
        for (size_t j = i + 1; j < ws_uses.size(); ++j) {
            const Use& u = ws_uses[i];
            const Use& v = ws_uses[j];
            if (u.a == v.a) continue;                   // the same slice in two roles
            if (u.a < v.b && v.a < u.b) fail("workspace slices overlap: " + u.role + " and " + v.role);
        }
}

struct BlockCase { const char* name; int64_t B, L, dm, di; int N, R; int io; bool step; bool states; };

void run_block(const BlockCase& c) {
    bufs.clear();
    ws_uses.clear();
    walk::records.clear();
    const size_t eio = c.io == SS_BF16 ? 2 : 4;
    ss_block_dims d{};
    d.batch = c.B; d.seqlen = c.L; d.d_model = c.dm; d.d_inner = c.di; d.d_state = c.N; d.d_conv = 4;
    d.dt_rank = c.R; d.io_dtype = c.io; d.discretization = SS_EULER; d.norm_eps = 1e-5f;
    const int64_t M = c.B * (c.step ? 1 : c.L);
    ss_block_weights w{};
    w.norm_w = (const float*)alloc("norm_w", c.dm * 4);
    w.W_in = (const void*)alloc("W_in", 2 * c.di * c.dm * eio);
    w.conv_w = (const float*)alloc("conv_w", c.di * 16);
    w.conv_b = (const float*)alloc("conv_b", c.di * 4);
    w.W_x = (const void*)alloc("W_x", (c.R + 2 * c.N) * c.di * eio);
    w.W_dt = (const void*)alloc("W_dt", c.di * c.R * eio);
    w.dt_bias = (const float*)alloc("dt_bias", c.di * 4);
    w.A = (const float*)alloc("A", c.di * c.N * 4);
    w.Dskip = (const float*)alloc("Dskip", c.di * 4);
    w.W_out = (const void*)alloc("W_out", c.dm * c.di * eio);
    void* x = (void*)alloc("x", M * c.dm * eio);
    void* out = (void*)alloc("out", M * c.dm * eio);
    float* hs = c.states ? (float*)alloc("ssm_state", c.B * c.di * c.N * 4) : nullptr;
    float* cs = c.states ? (float*)alloc("conv_state", c.B * c.di * 3 * 4) : nullptr;
    const size_t wsb = ss_block_workspace_bytes(&d, c.step ? 1 : 0);
    // planted mistake (self-test of this checker): the registered workspace is 4 KiB
    // shorter than the size the library asked for and is told it has
    void* ws = (void*)alloc("workspace", plant ? wsb - 4096 : wsb, true);
    const ss_status s = c.step ? ss_block_step(&d, &w, x, out, hs, cs, ws, wsb, nullptr)
                               : ss_block_fwd(&d, &w, x, out, hs, cs, ws, wsb, nullptr);
    if (s != SS_OK) fail(std::string(c.name) + ": call rejected: " + ss_last_error());
    int ng = 0, no = 0, ns = 0;
    for (const walk::Rec& r : walk::records) {
        if (r.kind == walk::kGemm) { check_gemm(r.gemm); ++ng; }
        else if (r.kind == walk::kBlockOp) { check_op(r.op); ++no; }
        else if (r.kind == walk::kScan || r.kind == walk::kStep) { check_scan(r.scan, r.kind == walk::kStep, r.bf16); ++ns; }
    }
    check_ws_overlap();
    std::printf("block %-28s M %8" PRId64 " workspace %12zu bytes: %d GEMM, %d elementwise, %d scan launches\n", c.name, M,
                wsb, ng, no, ns);
}

// ---------------------------------------------------------------------------
// Part 2: index arithmetic of one k_agg lane (see selscan_device.h, k_agg).

constexpr int kTile = selscan::kScanTile;    // R in the kernel

void agg_case(int64_t L, int64_t chunk_len, int nchunks, int N, int U, bool rev) {
    const int R = kTile;
    const int NB = N + 1;
    int bad = 0;
    auto inL = [&](int64_t v, const char* what) {
        if (v < 0 || v >= L) {
            if (bad++ < 5) std::printf("FAIL agg L=%" PRId64 " cl=%" PRId64 " N=%d U=%d rev=%d: %s token %" PRId64 "\n",
                                       L, chunk_len, N, U, (int)rev, what, v);
        }
    };
    for (int c = 0; c + 1 < nchunks; ++c) {
        const int64_t t0 = (int64_t)c * chunk_len;
        const int clen = (int)chunk_len;                       // every chunk but the last is full
        if (clen % R != 0) { std::printf("FAIL agg: chunk length not whole tiles\n"); ++bad; }
        const bool first = t0 == 0;
        if (!first && t0 < 3 + U) { std::printf("FAIL agg: a later chunk starts before row 3 + U\n"); ++bad; }
        const int xlo = first ? 0 : -(3 + U);
        // tile_fetch(rlo): element e of the tile -> chunk-relative row rlo + e / N (rlo >= 0)
        const int ntiles = clen / R;
        for (int k = 0; k < ntiles; ++k) {
            const int rlo = clen - (k + 1) * R;
            if (rlo < 0) { if (bad++ < 5) std::printf("FAIL agg: tile starts at row %d\n", rlo); }
            const int tile_elems = R * N;
            for (int e = 0; e < tile_elems; ++e) inL(t0 + rlo + e / N, "B tile row");
        }
        // load_rows(top, lo): rows max(top - i, lo), i < U, at byte offsets from the group's
        // lowest-address row (non-negative, and below 2^32 for any d_inner up to 2^26)
        auto load_rows = [&](int top, int lo, const char* what) {
            const int hi = top > lo ? top : lo;
            const int bot = top - (U - 1) > lo ? top - (U - 1) : lo;
            for (int i = 0; i < U; ++i) {
                const int r = top - i > lo ? top - i : lo;
                const int64_t rel = rev ? hi - r : r - bot;
                if (rel < 0 || rel >= U) { if (bad++ < 5) std::printf("FAIL agg: %s offset %" PRId64 " rows\n", what, rel); }
                inL(t0 + r, what);
            }
        };
        auto load_group = [&](int gr) {
            load_rows(gr - 1, 0, "delta row");
            load_rows(gr - 4, xlo, "x row");
        };
        auto group = [&](int gr, int rhi, bool edge) {
            for (int i = 0; i < U; ++i) {
                // staged row of the B value (and max |B|) of row gr-1-i, relative to the tile
                const int row = (gr - 1 - i) - (rhi - R);
                if (row < 0 || row >= R) {
                    if (bad++ < 5) std::printf("FAIL agg: LDS row %d outside the tile\n", row);
                }
                const int idx_last = row * NB + N;              // max |B| entry, the row's last
                if (idx_last >= R * NB) { if (bad++ < 5) std::printf("FAIL agg: LDS index %d\n", idx_last); }
                const int r = gr - 1 - i;
                // x_{r-3}: from the initial history exactly where it precedes the sequence
                // (the kernel's rule: chunk 0's last group, and with 2-row groups the one before)
                const bool from_hist = first && ((gr == U && U - 4 - i < 0) || (U < 3 && gr == 2 * U && 2 * U - 4 - i < 0));
                const bool needs_hist = t0 + r - 3 < 0;
                if (from_hist != needs_hist) {
                    if (bad++ < 5) std::printf("FAIL agg: x_{r-3} source wrong at token %" PRId64 "\n", t0 + r);
                }
                if (edge && gr != U) { if (bad++ < 5) std::printf("FAIL agg: edge group at row %d\n", gr); }
                if (edge && U < 8) { if (bad++ < 5) std::printf("FAIL agg: separate edge group with %d-row groups\n", U); }
            }
        };
        // the conv window before the sweep: rows clen-1, clen-2, clen-3
        for (int j = 1; j <= 3; ++j) inL(t0 + clen - j, "window row");
        load_group(clen);
        for (int k = 0; k < ntiles; ++k) {
            const int rhi = clen - k * R;
            const bool edge = first && k + 1 == ntiles;
            for (int gr = rhi; gr > rhi - R; gr -= 2 * U) {
                load_group(gr - U);
                group(gr, rhi, false);
                load_group(gr - 2 * U);
                group(gr - U, rhi, U == 8 && edge && gr - U == U);   // the separate copy: 8-row groups
            }
        }
    }
    if (bad) failures += bad;
    std::printf("agg L=%-7" PRId64 " chunk %-6" PRId64 " chunks %-4d N=%-2d U=%d %s: %s\n", L, chunk_len, nchunks, N, U,
                rev ? "reversed" : "forward ", bad ? "out of bounds" : "in bounds");
}

}  // namespace

int main(int argc, char** argv) {
    plant = argc > 1 && std::strcmp(argv[1], "--plant") == 0;
    const BlockCase cases[] = {
        {"block_train B8 L2048 d2560", 8, 2048, 2560, 5120, 16, 160, SS_BF16, false, true},
        {"block_train no states", 8, 2048, 2560, 5120, 16, 160, SS_BF16, false, false},
        {"block_bf16 B2 L1024 d512", 2, 1024, 512, 1024, 16, 32, SS_BF16, false, true},
        {"block_f32 B2 L1024 d512", 2, 1024, 512, 1024, 16, 32, SS_F32, false, true},
        {"decode S64 d512 bf16", 64, 1, 512, 1024, 16, 32, SS_BF16, true, true},
        {"decode S64 d512 f32", 64, 1, 512, 1024, 16, 32, SS_F32, true, true},
        {"decode S64 d2560 bf16", 64, 1, 2560, 5120, 16, 160, SS_BF16, true, true},
        {"decode S8 d512 bf16", 8, 1, 512, 1024, 16, 32, SS_BF16, true, true},
        {"ragged B3 L67 d48", 3, 67, 48, 96, 8, 3, SS_BF16, false, true},
        {"split-K B1 L200 d1001", 1, 200, 1001, 2002, 16, 63, SS_BF16, false, true},
        {"long B1 L8192 d64", 1, 8192, 64, 128, 16, 4, SS_F32, false, true},
        {"wide B3 L1500 d512", 3, 1500, 512, 1024, 16, 32, SS_BF16, false, true},
        {"L8192 B2 d512", 2, 8192, 512, 1024, 16, 32, SS_BF16, false, true},
        {"d_state 64 B2 L300 d256", 2, 300, 256, 512, 64, 16, SS_BF16, false, true},
    };
    for (const BlockCase& c : cases) run_block(c);
    // aggregate pass: the chunkings the library picks for the benchmark shapes and the tests,
    // plus d_state 64 with 8-row groups (the configuration that once faulted)
    struct A { int64_t L, cl; int nc; };
    const A ag[] = {{131072, 2048, 64}, {65536, 1024, 64}, {65536, 512, 128}, {16384, 128, 128}, {16384, 256, 64},
                    {2048, 512, 4}, {3001, 64, 47}, {200, 64, 4}, {192, 64, 3}};
    for (const A& a : ag)
        for (int N : {4, 8, 16, 32, 64})
            for (int U : {2, 4, 8})
                for (bool rev : {false, true}) agg_case(a.L, a.cl, a.nc, N, U, rev);
    std::printf("%s: %d violation(s)\n", failures ? "FAILED" : "ok", failures);
    return failures ? 1 : 0;
}
