// Host entry of path 5 (ce_wave.h), compiled in its own translation unit.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "ce_rowops.h"

namespace ce_wave {

// Bytes of a row per lane that the path-5 kernel takes for rows of C
// elements of es bytes loaded in vb-byte vectors (16, 32, 64, 128 or 256),
// or 0 when it has no configuration for them (rows above 16 KB, 4-byte
// vectors above 8 KB, vectors narrower than 4 bytes).
int lane_bytes(int64_t C, int es, int vb);

// Launches the path-5 kernel: dtype a CE_* value, op a ce::RowOp, grad
// whether the per-element output is written (kOpCE: gradient, kOpSoftmax:
// the softmax).  The caller has checked the arguments and that
// lane_bytes(C, es, vb) is not 0.  Returns CE_OK, CE_ERR_PATH or
// CE_ERR_LAUNCH.
int launch(int dtype, int op, bool grad, int vb, const void* logits, const int32_t* targets,
           int64_t B, int C, const ce::RowArgs& rs, void* out, float* rows_out, hipStream_t st);

// Bytes of a row per lane of the path-5 softmax backward (16 to 128: rows of
// up to 8 KB), or 0 when it has no configuration for the rows.
int bwd_lane_bytes(int64_t C, int es, int vb);

// Launches the path-5 softmax backward (y, dy, dx contiguous [B, C], at the
// same address modulo 16); the caller has checked the arguments and that
// bwd_lane_bytes(C, es, vb) is not 0.  Returns CE_OK, CE_ERR_PATH or
// CE_ERR_LAUNCH.
int launch_bwd(int dtype, int vb, const void* y, const void* dy, int64_t B, int C, void* dx,
               hipStream_t st);

}  // namespace ce_wave
