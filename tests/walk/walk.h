// Launch records of the host-side launch walk (mock_launch.cpp, block_walk.cpp).
#pragma once
#include <vector>

#include "selscan_internal.h"

namespace walk {
enum Kind { kScan, kStep, kBwd, kBlockOp, kGemm };
struct Rec {
    Kind kind;
    bool bf16, zoh;
    selscan::LaunchScan scan;
    selscan::LaunchBwd bwd;
    selscan::LaunchBlockOps op;
    selscan::LaunchGemm gemm;
};
extern std::vector<Rec> records;
}  // namespace walk
