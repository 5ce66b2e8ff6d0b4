// MFMA kernel instances: both operands K-major (fwd_rhs_transposed, da).
#include "mfma_launch.h"

namespace detgemm {

hipError_t launch_kk_bf16(int cfg, const TreeSel &t, const MfmaParams &p, int64_t tiles, hipStream_t st) {
    return launch_layout<true, true, OUT_BF16>(cfg, t, p, tiles, st);
}

}  // namespace detgemm
