// MFMA kernel instances: the grouped forward of the MoE grouped GEMM (X rows
// grouped by expert, one [K,N] weight per group), bf16 out, with the fused
// per-token slot epilogue.
#include "mfma_launch.h"

namespace detgemm {

hipError_t launch_moe_grouped(int cfg, const MfmaParams &p, const GroupTable &g, int64_t tiles,
                              hipStream_t st) {
    switch (cfg) {
    case 5:
        return launch_wide_grouped<4, 2, 2, 4, 2, 1, 4, 1, 2>(p, g, tiles, st);
    case 7:
        return launch_wide_grouped<4, 2, 2, 4, 2, 3, 2, 1, 2>(p, g, tiles, st);
    case 8:
        return launch_wide_grouped<4, 2, 2, 4, 3, 1, 4, 1, 2>(p, g, tiles, st);
    case 9:
        return launch_wide_grouped<4, 2, 2, 4, 3, 3, 2, 1, 2>(p, g, tiles, st);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace detgemm
