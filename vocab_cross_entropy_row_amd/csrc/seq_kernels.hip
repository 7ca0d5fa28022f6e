// Per-sequence sums of target log-probabilities (the building block of the
// "Fused linear + CPO loss" page's preference loss, whose formula the page does
// not give): out[b] = -sum_s loss[b * seq + s], one wave per sequence, lanes
// summing strided tokens in a fixed order and then the wave reduction.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lce_device.h"
#include "lce_internal.h"

namespace lce {

__global__ __launch_bounds__(kRowThreads) void seq_logprob_sum_kernel(const float* __restrict__ loss,
                                                                      int64_t batch, int64_t seq,
                                                                      float* __restrict__ out) {
  constexpr int kWaves = kRowThreads / 64;
  const int lane = threadIdx.x & 63;
  const int64_t b = (int64_t)blockIdx.x * kWaves + wave_uniform(threadIdx.x >> 6);
  if (b >= batch) return;
  const float* l = loss + b * seq;
  float acc = 0.0f;
  for (int64_t s = lane; s < seq; s += 64) acc += l[s];
  const float total = wave_sum(acc);
  if (lane == 0) out[b] = -total;
}

hipError_t launch_seq_logprob_sums(const float* loss, int64_t batch, int64_t seq, float* out,
                                   hipStream_t st) {
  constexpr int kWaves = kRowThreads / 64;
  const int64_t blocks = (batch + kWaves - 1) / kWaves;
  if (!grid_fits(blocks, kRowThreads)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(seq_logprob_sum_kernel, dim3((unsigned)blocks), dim3(kRowThreads), 0, st, loss,
                     batch, seq, out);
  return hipGetLastError();
}

}  // namespace lce
