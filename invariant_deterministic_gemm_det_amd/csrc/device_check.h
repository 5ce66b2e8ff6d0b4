// Shared by the library's translation units: DET_GEMM_OK when the current
// device is a gfx950, else DET_GEMM_EHIP (checked once per device).
#pragma once

namespace detgemm {
int check_device();
}  // namespace detgemm
