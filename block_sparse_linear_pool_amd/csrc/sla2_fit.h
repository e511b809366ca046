// Launcher of the stage-1 alpha fit (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>

namespace sla2 {

// alpha[h][i] = clip(<O_full - O_l, O_s - O_l> / |O_s - O_l|^2, 0, 1) over the 128 rows x d of
// query block i and all B batches (1 where the branches agree); [B, H, N, d] fp32 inputs.
hipError_t launch_fit_alpha(int B, int H, int N, const float* O_full, const float* O_s,
                            const float* O_l, float* alpha, hipStream_t s);

}  // namespace sla2
