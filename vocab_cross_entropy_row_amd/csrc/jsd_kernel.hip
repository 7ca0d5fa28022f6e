// Fused projection + generalized Jensen-Shannon divergence for gfx950.
//
// KernelIndex "Fused linear + JSD" (description and Semantics block): student
// and teacher activations (tokens x hidden) projected through their own
// vocab x hidden heads, then a generalized JSD between the two distributions,
// averaged over tokens ("batchmean"), with the logits never stored.  The page
// names the divergence without printing it; with P = softmax(student logits),
// Q = softmax(teacher logits) and M = beta P + (1 - beta) Q, per token
//
//     JSD = beta KL(P || M) + (1 - beta) KL(Q || M),  KL(A || B) = sum_j A_j ln(A_j / B_j).
//
// Each term needs both distributions normalised, so the work is two passes:
//   1. the log-sum-exp of each head's logits per token: the cross-entropy
//      kernel in its log-sum-exp mode, once per head;
//   2. either the stored path, where pass 1 also wrote both heads' fp32
//      logits and jsd_stored_rows_kernel (here) streams them once, or the
//      recompute path, the fused kernel's JSD mode (fused_kernel.hip), which
//      multiplies both heads again tile by tile; then per element
//      beta P (lp - ln M) + (1 - beta) Q (lq - ln M)  with lp = z_s - lse_s,
//      lq = z_t - lse_t, summed per token over the vocab (jsd_term).  Every
//      such term is >= 0 (log-sum inequality), so the sum does not cancel;
//      the term is evaluated relative to max(lp, lq), so that a probability
//      below the fp32 range gives 0 and never 0 * infinity.
// This file holds the stored path's row kernel and the merge of the
// recompute path's per-segment sums.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lce_device.h"
#include "lce_internal.h"
#include "mfma_common.h"

namespace lce {

// Divergence of token rows whose logits are stored: zs and zt are [rows, z_ld]
// fp32 (the first vocab columns of each row are the logits), lse_s / lse_t the
// rows' log-sum-exp.  One workgroup per row streams both rows with 16-byte
// buffer loads (kJRU chunks of each per lane in flight) and writes the row's
// sum to dst[row].  Summation order is fixed: per lane in chunk order, then
// the wave and workgroup reductions.
namespace {
constexpr int kJRThreads = 256;
constexpr int kJRU = 4;
constexpr int kJRPolicy = 2;  // nontemporal: each stored logit is read once
}  // namespace

__global__ __launch_bounds__(kJRThreads) void jsd_stored_rows_kernel(
    const float* __restrict__ zs, const float* __restrict__ zt, int64_t z_ld, int64_t vocab,
    const float* __restrict__ lse_s, const float* __restrict__ lse_t, float beta,
    float* __restrict__ dst) {
  const int64_t row = blockIdx.x;
  const float As = lse_s[row];
  const float At = lse_t[row];
  const uint32_t bytes = (uint32_t)vocab * 4u;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(zs + row * z_ld, bytes);
  const __amdgpu_buffer_rsrc_t rt = make_rsrc(zt + row * z_ld, bytes);
  const int nch = (int)((vocab + 3) / 4);
  float acc = 0.0f;
  for (int c0 = threadIdx.x; c0 < nch; c0 += kJRThreads * kJRU) {
    f32x4 a[kJRU], b[kJRU];
#pragma unroll
    for (int u = 0; u < kJRU; ++u) {
      const uint32_t off = (uint32_t)(c0 + u * kJRThreads) * 16u;  // past the row: reads 0
      a[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kJRPolicy));
      b[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rt, off, 0, kJRPolicy));
    }
#pragma unroll
    for (int u = 0; u < kJRU; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t j = (int64_t)(c0 + u * kJRThreads) * 4 + e;
        const float t = jsd_term(a[u][e] - As, b[u][e] - At, beta);
        acc += j < vocab ? t : 0.0f;
      }
  }
  acc = wave_sum(acc);
  __shared__ float red[kJRThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float tot = red[0];
#pragma unroll
    for (int q = 1; q < kJRThreads / 64; ++q) tot += red[q];
    dst[row] = tot;
  }
}

// One thread per token: the segments' sums in segment order, then the
// per-token divergence or the deterministic batch mean.
__global__ __launch_bounds__(kRowThreads) void fused_jsd_merge_kernel(
    int64_t tokens, int segments, const float* __restrict__ part, float* __restrict__ out,
    uint64_t* __restrict__ slots, unsigned* __restrict__ epoch, int reduce_mean) {
  const unsigned mean_tag = mean_begin(epoch, reduce_mean);
  const int64_t row = (int64_t)blockIdx.x * kRowThreads + threadIdx.x;
  float v = 0.0f;
  if (row < tokens) {
    for (int s = 0; s < segments; ++s) v += part[(int64_t)s * tokens + row];
    if (!reduce_mean) out[row] = v;
  }
  if (reduce_mean) {
    __shared__ float red[kRowThreads];
    red[threadIdx.x] = v;
    __syncthreads();
#pragma unroll
    for (int w = kRowThreads / 2; w > 0; w >>= 1) {
      if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
      __syncthreads();
    }
    finish_mean(red[0], slots, epoch, mean_tag, out, tokens);
  }
}

hipError_t launch_jsd(const JsdArgs& a, hipStream_t stream) {
  if (!grid_fits((a.tokens + kRowThreads - 1) / kRowThreads, kRowThreads))
    return hipErrorInvalidConfiguration;
  hipError_t e = launch_fused_jsd_partial(a, stream);
  if (e != hipSuccess) return e;
  const int64_t blocks = (a.tokens + kRowThreads - 1) / kRowThreads;
  hipLaunchKernelGGL(fused_jsd_merge_kernel, dim3((unsigned)blocks), dim3(kRowThreads), 0, stream,
                     a.tokens, a.segments, (const float*)a.partials, a.out, a.mean_slots, a.epoch,
                     a.reduce_mean);
  return hipGetLastError();
}

hipError_t launch_jsd_rows(const JsdRowsArgs& a, hipStream_t stream) {
  if (!grid_fits(a.rows, kJRThreads)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(jsd_stored_rows_kernel, dim3((unsigned)a.rows), dim3(kJRThreads), 0, stream,
                     a.zs, a.zt, a.z_ld, a.vocab, a.lse_s, a.lse_t, a.beta, a.dst);
  return hipGetLastError();
}

hipError_t launch_jsd_mean(int64_t tokens, const float* per_token, float* out, uint64_t* slots,
                           unsigned* epoch, hipStream_t stream) {
  const int64_t blocks = (tokens + kRowThreads - 1) / kRowThreads;
  if (!grid_fits(blocks, kRowThreads)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(fused_jsd_merge_kernel, dim3((unsigned)blocks), dim3(kRowThreads), 0, stream,
                     tokens, 1, per_token, out, slots, epoch, 1);
  return hipGetLastError();
}

}  // namespace lce
