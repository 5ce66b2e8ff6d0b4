// MFMA kernel instances: leaf inspection of the forward layout.
#include "mfma_launch.h"

namespace detgemm {

hipError_t launch_leaves(int cfg, const TreeSel &t, const MfmaParams &p, int64_t tiles, hipStream_t st) {
    return launch_layout<true, false, OUT_LEAVES>(cfg, t, p, tiles, st);
}

}  // namespace detgemm
