// Launcher of the cross-head transform + per-token INT4 kernel (cross_head.hip).
#pragma once

#include "common.h"

namespace quarot {

// Cross-head transform (H_{n_h} (x) I_128, normalised) + per-token INT4 of
// rows of n_heads * 128 fp16 values; n_heads a power of two <= 64.
// Arguments already validated.
int launch_cross_head_quant(const __half* z, int64_t rows, int n_heads, int64_t ld_z,
                            float clip_ratio, uint8_t* q_out, int64_t ld_q, __half* scale_out,
                            float* z_rot, hipStream_t stream);

}  // namespace quarot
