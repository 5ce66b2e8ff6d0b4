// MFMA kernel instances: both operands MN-major, transposed store (db_transposed).
#include "mfma_launch.h"

namespace detgemm {

hipError_t launch_nn_bf16t(int cfg, const TreeSel &t, const MfmaParams &p, int64_t tiles, hipStream_t st) {
    return launch_layout<false, false, OUT_BF16_T>(cfg, t, p, tiles, st);
}

}  // namespace detgemm
