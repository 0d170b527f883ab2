// Definitions the backward's kernels share (kda_bwd.hip, kda_bwd_scan.hip).
#pragma once

#include "kda_device.h"

namespace kda {

// Record of the backward's states scan (kda_bwd_scan.hip fscan_kernel), per
// (chunk slot, head) at head dimension KD, written by the prep kernel: Kt and
// Wm = P^T Kb Gam in bf16, in the Kt and W^T operand layouts of
// RecLayout<KD>, and the chunk decay (fp32).  The decay region holds
// max(KD, 128) channels (the scans' decay loads cover 128 channels at a
// time; past KD they read zeros that no state row uses).  5 KB at KD = 64,
// 9 KB at 128, 17 KB at 256.
template <int KD>
struct StatesRecT {
    static_assert(KD == 64 || KD == 128 || KD == 256, "backward head dimensions");
    static constexpr int GAMC = KD > 128 ? KD : 128;   // channels of the decay region
    static constexpr int KTH = 0;
    static constexpr int WTH = 32 * KD;
    static constexpr int GAM = 64 * KD;
    static constexpr int BYTES = (64 * KD + 4 * GAMC + 1023) / 1024 * 1024;
};

// Floats per (chunk slot, head) of the backward's dt_bias partial sums.
template <int KD>
constexpr int bwd_pd_stride() { return KD > 128 ? KD : 128; }

}  // namespace kda
