// Logit gradient of the fused projection from stored logits (host <-> device
// interface of fused_grad_kernel.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lce {

// For token rows whose fp32 logits z [rows, ld] and log-sum-exp lse [rows] are
// stored, write the bf16 logit gradient dz [rows, ld]:
//     dz_ij = g_i (e^(z_ij - lse_i) - [j == t_i]),
// g_i = grad[0] / grad_tokens (grad_mean) or grad[i]; NaN rows for targets
// outside [0, vocab).  Columns in [vocab, ld) get values for whatever the
// padding holds and are never meaningful.  ld is a multiple of 4; rows * ld
// fits the buffers; ld * 4 < 2^31.
struct FusedGradRowsArgs {
  const float* z;
  const float* lse;
  const int64_t* target;
  const float* grad;
  int grad_mean;
  int64_t grad_tokens;
  int64_t rows;
  int64_t vocab;
  int64_t ld;
  uint16_t* dz;
};
hipError_t launch_fused_grad_rows(const FusedGradRowsArgs& a, hipStream_t stream);

// out [cols, rows] = transpose of in [rows, cols], 16-bit elements, both
// row-major and contiguous.
hipError_t launch_transpose_u16(const uint16_t* in, int64_t rows, int64_t cols, uint16_t* out,
                                hipStream_t stream);

}  // namespace lce
