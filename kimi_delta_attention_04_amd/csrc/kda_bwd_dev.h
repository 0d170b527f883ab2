// Definitions the backward's kernels share (kda_bwd.hip, kda_bwd_scan.hip).
#pragma once

#include "kda_device.h"

namespace kda {

// Record of the backward's states scan (kda_bwd_scan.hip fscan_kernel), per
// (chunk slot, head) at head dimension KD, written by the prep kernel: Kt and
// Wm = P^T Kb Gam in bf16, in the Kt and W^T operand layouts of
// RecLayout<KD>, and the chunk decay (fp32).  The decay region is 128
// channels long at every KD (the scan's decay loads cover 128 channels; past
// KD they read zeros that no state row uses).  9 KB at KD = 128, 5 KB at 64.
template <int KD>
struct StatesRecT {
    static_assert(KD == 64 || KD == 128, "backward head dimensions");
    static constexpr int KTH = 0;
    static constexpr int WTH = 32 * KD;
    static constexpr int GAM = 64 * KD;
    static constexpr int BYTES = (64 * KD + 4 * 128 + 1023) / 1024 * 1024;
};

}  // namespace kda
