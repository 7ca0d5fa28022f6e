// Measurement probes for bench.py (not part of liblce).
//
// stream_read_kernel reads a device buffer once with 16-byte nontemporal buffer
// loads, the loads the row kernels stream logits with, and does nothing else
// with the data but fold it into one register per lane: what a plain read of a
// workload's bytes costs, for comparison with the kernel that reads them (not
// a peak: the long-row kernels read faster than it does).
//
// valu_rate_kernel times the vector arithmetic of the row fold: 8 independent
// chains per lane of v_exp_f32, of v_fma_f32, or of the whole bf16 fold step
// (decode one half of a 32-bit word, FMA, exponential, add), in a grid that
// fills every wave slot.
//
// Build (done by __graft_entry__.build()):
//   hipcc -O3 --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops
//         -shared -fPIC bench_probe.hip -o bench_probe.so
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kU = 8;           // 16-byte chunks per lane in flight
constexpr int kMaxBlocks = 2048;  // 8 resident 256-thread workgroups on each of 256 CUs

// Loads at or past `bytes` read no memory and return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// The buffer is cut into tiles of kThreads * kU chunks (32 KiB); workgroup b reads tiles
// b, b + gridDim.x, ..., and in a tile lane l reads chunks l, l + kThreads, ..., so one wave
// instruction reads 1 KiB of consecutive memory and a workgroup's loads in flight cover one
// contiguous tile (the row kernels likewise read each 8 KiB row contiguously).  bytes <= 2^31
// (host check), so byte offsets, below bytes + 32 KiB, fit 32 bits.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const void* src, uint32_t bytes,
                                                               uint32_t* sink) {
  const __amdgpu_buffer_rsrc_t rs = rsrc(src, bytes);
  const uint32_t chunks = bytes / 16u;
  constexpr uint32_t kTile = kThreads * kU;
  uint32_t acc = 0;
  for (uint32_t t = blockIdx.x; t * kTile < chunks; t += gridDim.x) {
    const uint32_t c0 = t * kTile + threadIdx.x;
    u32x4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u)  // chunks past the end read zero
      v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rs, (c0 + (uint32_t)u * kThreads) * 16u, 0, 2 /* nt */));
#pragma unroll
    for (int u = 0; u < kU; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;  // keeps the loads live; a store almost never happens
}

// MODE 0: a = 2^a; 1: a = a * 0.999 + 1e-7; 2: a += 2^(z * log2(e) - 3) with z the high or
// low bf16 half of a word that changes every step.  Each thread writes one value, so no
// chain is dead code.
template <int MODE>
__global__ __launch_bounds__(kThreads) void valu_rate_kernel(float* out, int iters, float seed) {
  float a[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = seed * (float)(threadIdx.x + j) * 1e-6f;
  uint32_t r = __float_as_uint(seed) ^ threadIdx.x;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (MODE == 0) {
        a[j] = __builtin_amdgcn_exp2f(a[j]);
      } else if constexpr (MODE == 1) {
        a[j] = __builtin_fmaf(a[j], 0.999f, 1e-7f);
      } else {
        const uint32_t w = r + (uint32_t)j * 0x9e3779b9u;
        const float z = (j & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
        a[j] += __builtin_amdgcn_exp2f(__builtin_fmaf(z, 1.442695f, -3.0f));
      }
    }
    r += 0x7f4a7c15u;
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += a[j];
  out[blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

// Enqueue one valu_rate_kernel<mode> launch of `blocks` workgroups of 256 threads, each
// thread taking `iters` steps of its 8 chains; `out` holds blocks * 256 floats.  Returns a
// hipError_t value: hipErrorInvalidValue for mode outside 0..2, blocks outside 1..65535 or
// iters outside 1..2^20.
extern "C" __attribute__((visibility("default"))) int bench_valu_rate(int mode, float* out,
                                                                       int blocks, int iters,
                                                                       hipStream_t stream) {
  if (!out || mode < 0 || mode > 2 || blocks < 1 || blocks > 65535 || iters < 1 ||
      iters > (1 << 20))
    return (int)hipErrorInvalidValue;
  if (mode == 0)
    hipLaunchKernelGGL(valu_rate_kernel<0>, dim3(blocks), dim3(kThreads), 0, stream, out, iters, 0.5f);
  else if (mode == 1)
    hipLaunchKernelGGL(valu_rate_kernel<1>, dim3(blocks), dim3(kThreads), 0, stream, out, iters, 0.5f);
  else
    hipLaunchKernelGGL(valu_rate_kernel<2>, dim3(blocks), dim3(kThreads), 0, stream, out, iters, 0.5f);
  return (int)hipGetLastError();
}

// Enqueue one read of `bytes` bytes at `src` (16-byte aligned, bytes a multiple of 16 and
// at most 2^31) on `stream`.  `sink` is a 4-byte device buffer the kernel may write.
// Returns a hipError_t value: hipErrorInvalidValue for arguments out of that range.
extern "C" __attribute__((visibility("default"))) int bench_stream_read(const void* src,
                                                                         uint64_t bytes,
                                                                         uint32_t* sink,
                                                                         hipStream_t stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || bytes > (uint64_t(1) << 31) ||
      (uintptr_t)src % 16 != 0)
    return (int)hipErrorInvalidValue;
  const uint64_t per_block = (uint64_t)kThreads * kU * 16;
  uint64_t blocks = (bytes + per_block - 1) / per_block;
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, src,
                     (uint32_t)bytes, sink);
  return (int)hipGetLastError();
}
