// Logit gradient of the fused projection + cross-entropy from stored logits,
// for gfx950.  The pages give only the forward; this is its derivative:
//
//     dz_ij = g_i (e^(z_ij - lse_i) - [j == t_i])
//
// with the fp32 logits z and log-sum-exp lse written by the fused kernel's
// store mode.  One workgroup per token row streams the row in 16-byte chunks
// (four logits) and writes four bf16 gradients (8 bytes, round to nearest
// even) per chunk; the row is read and written once, so the kernel is bound
// by HBM bandwidth (6 bytes per logit).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fused_grad.h"
#include "lce_internal.h"
#include "lce_device.h"
#include "mfma_common.h"

namespace lce {

namespace {
constexpr int kGThreads = 256;
constexpr int kGU = 4;  // chunks per thread in flight
}  // namespace

__global__ __launch_bounds__(kGThreads) void fused_grad_rows_kernel(
    const float* __restrict__ z, const float* __restrict__ lse, const int64_t* __restrict__ target,
    const float* __restrict__ grad, int grad_mean, int64_t grad_tokens, int64_t vocab, int64_t ld,
    uint16_t* __restrict__ dz) {
  const int64_t row = blockIdx.x;
  const int64_t t = target[row];
  const bool valid = t >= 0 && t < vocab;
  float g = grad_mean ? grad[0] / (float)grad_tokens : grad[row];
  if (!valid) g = __builtin_nanf("");
  const float L = lse[row] * kLog2e;
  const int tc = valid ? (int)(t >> 2) : -1;  // chunk holding the target
  const int te = (int)(t & 3);
  const uint32_t nch = (uint32_t)(ld / 4);
  const __amdgpu_buffer_rsrc_t src = make_rsrc(z + row * ld, nch * 16u);
  const __amdgpu_buffer_rsrc_t dst = make_rsrc(dz + row * ld, nch * 8u);
  for (uint32_t c0 = threadIdx.x; c0 < nch; c0 += kGThreads * kGU) {
    f32x4 v[kGU];
#pragma unroll
    for (int u = 0; u < kGU; ++u)  // chunks past the row read 0 and are not stored
      v[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           src, (c0 + u * kGThreads) * 16u, 0, 2 /* nt */));
#pragma unroll
    for (int u = 0; u < kGU; ++u) {
      const uint32_t c = c0 + u * kGThreads;
      float d[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        d[e] = g * exp2_fast(__builtin_fmaf(v[u][e], kLog2e, -L));
        if ((int)c == tc && e == te) d[e] -= g;
      }
      const u32x2 packed = {
          __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{d[0], d[1]}), bf16x2)),
          __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{d[2], d[3]}), bf16x2))};
      __builtin_amdgcn_raw_buffer_store_b64(packed, dst, c * 8u, 0, 0);
    }
  }
}

// Transpose of a [rows, cols] matrix of 16-bit elements through 64 x 64 LDS
// tiles (the +1 column of padding keeps the transposed reads off one bank).
// Reads and writes are coalesced along the tile's rows.
__global__ __launch_bounds__(256) void transpose_u16_kernel(const uint16_t* __restrict__ in,
                                                            int64_t rows, int64_t cols,
                                                            uint16_t* __restrict__ out) {
  __shared__ uint16_t tile[64][65];
  const int64_t col_tiles = (cols + 63) / 64;  // one-dimensional grid: row tile x col tile
  const int64_t r0 = (int64_t)blockIdx.x / col_tiles * 64, c0 = (int64_t)blockIdx.x % col_tiles * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 64 x 4 threads
#pragma unroll
  for (int i = 0; i < 64; i += 4) {
    const int64_t r = r0 + ty + i, c = c0 + tx;
    if (r < rows && c < cols) tile[ty + i][tx] = in[r * cols + c];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 64; i += 4) {
    const int64_t c = c0 + ty + i, r = r0 + tx;  // output row c, column r
    if (c < cols && r < rows) out[c * rows + r] = tile[tx][ty + i];
  }
}

hipError_t launch_transpose_u16(const uint16_t* in, int64_t rows, int64_t cols, uint16_t* out,
                                hipStream_t stream) {
  const int64_t blocks = ((cols + 63) / 64) * ((rows + 63) / 64);
  if (!grid_fits(blocks, 256)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(transpose_u16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, in, rows,
                     cols, out);
  return hipGetLastError();
}

hipError_t launch_fused_grad_rows(const FusedGradRowsArgs& a, hipStream_t stream) {
  if (!grid_fits(a.rows, kGThreads)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(fused_grad_rows_kernel, dim3((unsigned)a.rows), dim3(kGThreads), 0, stream,
                     a.z, a.lse, a.target, a.grad, a.grad_mean, a.grad_tokens, a.vocab, a.ld,
                     (uint16_t*)a.dz);
  return hipGetLastError();
}

}  // namespace lce
