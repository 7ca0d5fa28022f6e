// Building blocks shared by the MFMA kernels (fused projection + cross-entropy,
// fused projection + JSD): fragment types, the LDS row swizzle, the LDS-only
// workgroup barrier and explicit vmcnt waits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lce {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Physical 16-byte chunk of logical chunk `c` in LDS row `r` (rows of 128 B):
// a ds_read_b128 of 8 or 16 consecutive rows at one logical chunk touches
// every bank once.  The map is its own inverse.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r & 7) ^ ((r >> 3) & 1)); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Workgroup barrier ordering LDS accesses only.  __syncthreads() also orders
// global memory, which makes the compiler drain every outstanding load
// (vmcnt(0)) at the barrier, including the slab DMAs meant to stay in flight
// across it; their completion is waited for explicitly (wait_vmcnt).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are done
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// s_waitcnt vmcnt(N) with the other counters left free (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | (0xF << 8) | (0x7 << 4) | (N & 0xF));
}

}  // namespace lce
