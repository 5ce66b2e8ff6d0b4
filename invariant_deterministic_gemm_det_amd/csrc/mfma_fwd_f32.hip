// MFMA kernel instances: forward with fp32 output.
#include "mfma_launch.h"

namespace detgemm {

hipError_t launch_fwd_f32(int cfg, const TreeSel &t, const MfmaParams &p, int64_t tiles, hipStream_t st) {
    return launch_layout<true, false, OUT_F32>(cfg, t, p, tiles, st);
}

}  // namespace detgemm
