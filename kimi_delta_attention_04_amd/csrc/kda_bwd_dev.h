// Definitions the backward's kernels share (kda_bwd.hip, kda_bwd_scan.hip).
#pragma once

#include "kda_device.h"

namespace kda {

// Record of the backward's states scan (kda_bwd_scan.hip fscan_kernel), per
// (chunk slot, head), written by the prep kernel: Kt and Wm = P^T Kb Gam in
// bf16, in the Kt and W^T operand layouts of RecLayout<128>, and the chunk
// decay (fp32).
struct StatesRec {
    static constexpr int KTH = 0;
    static constexpr int WTH = 4096;
    static constexpr int GAM = 8192;
    static constexpr int BYTES = 9216;        // 9 one-kilobyte units
};

}  // namespace kda
