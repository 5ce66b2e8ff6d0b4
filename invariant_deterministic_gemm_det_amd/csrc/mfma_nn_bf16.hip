// MFMA kernel instances: both operands MN-major (db).
#include "mfma_launch.h"

namespace detgemm {

hipError_t launch_nn_bf16(int cfg, const TreeSel &t, const MfmaParams &p, int64_t tiles, hipStream_t st) {
    return launch_layout<false, false, OUT_BF16>(cfg, t, p, tiles, st);
}

}  // namespace detgemm
