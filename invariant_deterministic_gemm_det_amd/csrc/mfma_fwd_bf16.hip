// MFMA kernel instances: forward, B given as [K,N].
#include "mfma_launch.h"

namespace detgemm {

hipError_t launch_fwd_bf16(int cfg, const TreeSel &t, const MfmaParams &p, int64_t tiles, hipStream_t st) {
    return launch_layout<true, false, OUT_BF16>(cfg, t, p, tiles, st);
}

}  // namespace detgemm
