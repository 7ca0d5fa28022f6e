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
// mfma_lds_kernel is the fused projection kernel's inner loop with nothing else: per wave
// and k-step, 8 v_mfma_f32_32x32x16_bf16 on a 128 x 64 tile whose 6 fragments (1 KiB each)
// come from LDS one k-step ahead, a workgroup barrier every 4 k-steps, and 8 direct-to-LDS
// 1 KiB buffer loads per wave every 4 k-steps (from a 1 MiB buffer that stays in L2), in
// 8-wave workgroups, one per CU.  Variants add these parts one at a time, so the cycles each
// costs the matrix cores can be read off (s_memtime cycles per wave).
//
// lds_read_kernel measures LDS read throughput alone: W waves per workgroup, one workgroup
// per CU, each wave reading 1 KiB blocks with ds_read_b128, 8 per step, folded with xor.
//
// Build (done by __graft_entry__.build()):
//   hipcc -O3 --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops
//         -shared -fPIC bench_probe.hip -o bench_probe.so
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kSkWaves = 8;
constexpr int kSkThreads = 64 * kSkWaves;
constexpr int kSkLdsBytes = 96 * 1024;   // one workgroup per CU (64 KiB used)
constexpr int kSkBlocks = 256;
constexpr uint32_t kSkSrcBytes = 1u << 20;

// VARIANT 0: MFMAs only (fragments fixed in registers); 1: fragment reads only; 2: MFMAs and
// fragment reads; 3: as 2 plus a barrier every 4 k-steps; 4: as 3 plus the DMAs.  Fragment
// reads cover LDS bytes [0, 32 KiB) (32 blocks of 1 KiB, one per wave instruction), DMAs
// write [32 KiB, 64 KiB).  iters is a positive multiple of 4 (host check).
template <int VARIANT>
__global__ __launch_bounds__(kSkThreads) void mfma_lds_kernel(int iters, unsigned long long* cycles,
                                                               float* sink, const uint32_t* src) {
  extern __shared__ u32x4 lds[];
  for (int i = threadIdx.x; i < 4096; i += kSkThreads)
    lds[i] = (u32x4){0x3f803f80u ^ (uint32_t)(i * 0x00010001u & 0x007f007fu), 0xbf003e80u,
                     0x3e803f00u ^ (uint32_t)i, 0x3f80bf80u};
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f32x16 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = (f32x16)(0.0f);
  uint32_t x = 0;
  bf16x8 a[2][4], b[2][2];
  auto rd = [&](int it, int k) -> u32x4 { return lds[((it * 6 + k + wave * 13) & 31) * 64 + lane]; };
  auto frags = [&](int it, int p) {
#pragma unroll
    for (int k = 0; k < 4; ++k) a[p][k] = __builtin_bit_cast(bf16x8, rd(it, k));
#pragma unroll
    for (int k = 0; k < 2; ++k) b[p][k] = __builtin_bit_cast(bf16x8, rd(it, 4 + k));
  };
  const __amdgpu_buffer_rsrc_t rs = rsrc(src, kSkSrcBytes);
  auto dma = [&](int it, int i) {  // 1 KiB: source offset < 1 MiB, LDS [32 KiB, 64 KiB)
    const uint32_t vo = (uint32_t)(((it * 8 + i + wave * 5) & 1023) * 1024 + lane * 16);
    uint32_t* dst = reinterpret_cast<uint32_t*>(lds) + (32 * 1024 + ((wave + kSkWaves * i) & 31) * 1024) / 4;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)dst, 16, vo, 0, 0, 0);
  };
  auto step = [&](int it, auto pc) {
    constexpr int p = decltype(pc)::value;
    if constexpr (VARIANT == 1) {
#pragma unroll
      for (int k = 0; k < 6; ++k) {
        const u32x4 v = rd(it, k);
        x += (v.x ^ v.y) + (v.z ^ v.w);
      }
    } else {
      if constexpr (VARIANT >= 2) frags(it + 1, p ^ 1);
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int aa = 0; aa < 4; ++aa)
          acc[bb * 4 + aa] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[p][aa], b[p][bb], acc[bb * 4 + aa], 0, 0, 0);
    }
  };
  frags(0, 0);
  if (VARIANT == 0) frags(1, 1);
  __syncthreads();
  const unsigned long long t0 = clock64();
  for (int it = 0; it < iters; it += 4) {
    if constexpr (VARIANT == 4)
      for (int i = 0; i < 4; ++i) dma(it, i);
    step(it, std::integral_constant<int, 0>{});
    step(it + 1, std::integral_constant<int, 1>{});
    step(it + 2, std::integral_constant<int, 0>{});
    if constexpr (VARIANT == 4) __builtin_amdgcn_s_waitcnt((0xF << 8) | (0x7 << 4) | 4);  // vmcnt(4)
    if constexpr (VARIANT >= 3) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      __asm__ volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");
    }
    step(it + 3, std::integral_constant<int, 1>{});
    if constexpr (VARIANT == 4)
      for (int i = 4; i < 8; ++i) dma(it, i);
  }
  __builtin_amdgcn_s_waitcnt(0);
  const unsigned long long t1 = clock64();
  float sum = (float)x;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) sum += acc[k][e];
  sink[blockIdx.x * kSkThreads + threadIdx.x] = sum;
  if (lane == 0) cycles[blockIdx.x * kSkWaves + wave] = t1 - t0;
}

// W waves; reads cover LDS bytes [0, 64 KiB) (64 blocks of 1 KiB), 96 KiB requested so that
// one workgroup runs per CU.
template <int W>
__global__ __launch_bounds__(64 * W) void lds_read_kernel(int iters, unsigned long long* cycles,
                                                          uint32_t* sink) {
  extern __shared__ u32x4 lds[];
  for (int i = threadIdx.x; i < 4096; i += 64 * W) lds[i] = (u32x4){(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  u32x4 x = (u32x4){0u, 0u, 0u, 0u};
  const unsigned long long t0 = clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) x ^= lds[((it * 8 + k + wave * 5) & 63) * 64 + lane];
  }
  const unsigned long long t1 = clock64();
  sink[blockIdx.x * 64 * W + threadIdx.x] = x.x ^ x.y ^ x.z ^ x.w;
  if (lane == 0) cycles[blockIdx.x * W + wave] = t1 - t0;
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

// Enqueue one mfma_lds_kernel<variant> launch: 256 workgroups of 8 waves, `iters` k-steps
// per wave.  `cycles` holds 2048 uint64 (each wave's loop cycles), `sink` 256 * 512 floats,
// `src` 1 MiB of device memory (the DMA source; 16-byte aligned).  Returns a hipError_t
// value: hipErrorInvalidValue for variant outside 0..4, iters outside 4..2^20 or not a
// multiple of 4, or a null pointer.
extern "C" __attribute__((visibility("default"))) int bench_mfma_lds(int variant, unsigned long long* cycles,
                                                                      float* sink, const void* src,
                                                                      int iters, hipStream_t stream) {
  if (!cycles || !sink || !src || (uintptr_t)src % 16 != 0 || variant < 0 || variant > 4 ||
      iters < 4 || iters > (1 << 20) || iters % 4 != 0)
    return (int)hipErrorInvalidValue;
  const uint32_t* s = static_cast<const uint32_t*>(src);
  hipError_t e = hipSuccess;
#define SK_LAUNCH(V)                                                                              \
  e = hipFuncSetAttribute((const void*)mfma_lds_kernel<V>, hipFuncAttributeMaxDynamicSharedMemorySize, \
                          kSkLdsBytes);                                                           \
  if (e != hipSuccess) return (int)e;                                                             \
  hipLaunchKernelGGL(mfma_lds_kernel<V>, dim3(kSkBlocks), dim3(kSkThreads), kSkLdsBytes, stream,  \
                     iters, cycles, sink, s);
  switch (variant) {
    case 0: SK_LAUNCH(0) break;
    case 1: SK_LAUNCH(1) break;
    case 2: SK_LAUNCH(2) break;
    case 3: SK_LAUNCH(3) break;
    default: SK_LAUNCH(4) break;
  }
#undef SK_LAUNCH
  return (int)hipGetLastError();
}

// Enqueue one lds_read_kernel<waves> launch (waves 4, 8 or 16): 256 workgroups, `iters`
// steps of 8 reads per wave.  `cycles` holds 256 * waves uint64, `sink` 256 * 64 * waves
// uint32.  Returns a hipError_t value: hipErrorInvalidValue for other wave counts, iters
// outside 1..2^20 or a null pointer.
extern "C" __attribute__((visibility("default"))) int bench_lds_read(int waves, unsigned long long* cycles,
                                                                      uint32_t* sink, int iters,
                                                                      hipStream_t stream) {
  if (!cycles || !sink || iters < 1 || iters > (1 << 20) || (waves != 4 && waves != 8 && waves != 16))
    return (int)hipErrorInvalidValue;
  hipError_t e = hipSuccess;
#define LR_LAUNCH(W)                                                                                \
  e = hipFuncSetAttribute((const void*)lds_read_kernel<W>, hipFuncAttributeMaxDynamicSharedMemorySize, \
                          kSkLdsBytes);                                                             \
  if (e != hipSuccess) return (int)e;                                                               \
  hipLaunchKernelGGL(lds_read_kernel<W>, dim3(kSkBlocks), dim3(64 * W), kSkLdsBytes, stream, iters,   \
                     cycles, sink);
  if (waves == 4) {
    LR_LAUNCH(4)
  } else if (waves == 8) {
    LR_LAUNCH(8)
  } else {
    LR_LAUNCH(16)
  }
#undef LR_LAUNCH
  return (int)hipGetLastError();
}
