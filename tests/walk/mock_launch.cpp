// Host-only stand-ins for the library's kernel launchers: every launch description the
// C-ABI layer and the block pipeline hand to the kernels is recorded instead of run, so
// a CPU test can check each one's address ranges against the buffers they must stay in.
// Test infrastructure; no GPU code.
#include <vector>

#include "selscan_internal.h"
#include "walk.h"

namespace walk {
std::vector<Rec> records;
}

namespace selscan {

static hipError_t rec_scan(const LaunchScan& p, bool step, bool bf16, bool zoh) {
    walk::Rec r{};
    r.kind = step ? walk::kStep : walk::kScan;
    r.scan = p;
    r.bf16 = bf16;
    r.zoh = zoh;
    walk::records.push_back(r);
    return hipSuccess;
}
hipError_t launch_f32_euler(const LaunchScan& p, bool step) { return rec_scan(p, step, false, false); }
hipError_t launch_f32_zoh(const LaunchScan& p, bool step) { return rec_scan(p, step, false, true); }
hipError_t launch_bf16_euler(const LaunchScan& p, bool step) { return rec_scan(p, step, true, false); }
hipError_t launch_bf16_zoh(const LaunchScan& p, bool step) { return rec_scan(p, step, true, true); }

static hipError_t rec_bwd(const LaunchBwd& p) {
    walk::Rec r{};
    r.kind = walk::kBwd;
    r.bwd = p;
    walk::records.push_back(r);
    return hipSuccess;
}
hipError_t launch_bwd_f32_euler(const LaunchBwd& p) { return rec_bwd(p); }
hipError_t launch_bwd_bf16_euler(const LaunchBwd& p) { return rec_bwd(p); }
hipError_t launch_bwd_f32_zoh(const LaunchBwd& p) { return rec_bwd(p); }
hipError_t launch_bwd_bf16_zoh(const LaunchBwd& p) { return rec_bwd(p); }

hipError_t launch_block_op(const LaunchBlockOps& p) {
    walk::Rec r{};
    r.kind = walk::kBlockOp;
    r.op = p;
    walk::records.push_back(r);
    return hipSuccess;
}

hipError_t launch_gemm(const LaunchGemm& p) {
    walk::Rec r{};
    r.kind = walk::kGemm;
    r.gemm = p;
    walk::records.push_back(r);
    return hipSuccess;
}

}  // namespace selscan
