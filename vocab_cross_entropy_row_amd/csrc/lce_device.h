// Device helpers shared by liblce's kernels (gfx950, wave64).
//
// Log-sum-exp state.  A row's softmax normaliser is kept as (m, s): m is the
// largest logit seen and s = sum_j 2^(z_j * L - M) with L = log2(e) rounded
// to fp32 and M = fp32(m * L).  Each exponent z * L - M is formed by one FMA,
// so it is rounded once, after the cancellation; the rounding of M itself is
// undone at the end with its exact residual fma(m, L, -M):
//     ln sum_j e^(z_j) - z_t  =  (m - z_t) + ln2 * (log2(s) - fma(m, L, -M)).
// The target logit is subtracted from m before the small term is added, so
// only that small term carries fp32 rounding, even when every logit is large
// (rows shifted by 2^15 keep full accuracy).
//
// Two states merge by rescaling both to the larger max; because each state is
// scaled to its own M, a factor of exactly 1 is used when the maxima agree
// (this also covers empty states with m = -inf).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lce {

constexpr float kLog2e = 1.44269504088896340736f;  // log2(e)
constexpr float kLn2 = 0.69314718055994530942f;    // ln(2)
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// bf16 -> fp32 is exact: the bf16 pattern is the upper half of the fp32 pattern.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

struct Lse {
  float m;  // running max (kNegInf when empty)
  float s;  // sum of 2^(z*L - fp32(m*L))
};

__device__ __forceinline__ Lse lse_empty() { return {kNegInf, 0.0f}; }

// Factor that rescales a state with max `m_old` to the max `m_new` (>= m_old):
// 2^(fp32(m_old*L) - fp32(m_new*L)).  Both products must be the rounded values
// the sums were built against, so contraction into an FMA is switched off (a
// fused form would drop the rounding of m_old*L, up to half an ulp of |m|*L).
// For nearby maxima the difference of the two products is exact.
__device__ __forceinline__ float lse_rescale(float m_old, float m_new) {
#pragma clang fp contract(off)
  return (m_old == m_new) ? 1.0f : exp2_fast(m_old * kLog2e - m_new * kLog2e);
}

__device__ __forceinline__ Lse lse_merge(Lse a, Lse b) {
  const float m = fmaxf(a.m, b.m);
  return {m, a.s * lse_rescale(a.m, m) + b.s * lse_rescale(b.m, m)};
}

// ln(sum_j e^z_j) - z of a non-empty state.  (m - z) is formed first: both are
// logits of the same row, so the difference is exact or nearly so even when
// the logits are large, and only the small term ln(s) carries rounding.
__device__ __forceinline__ float lse_minus(Lse st, float z) {
  const float M = st.m * kLog2e;
  const float resid = __builtin_fmaf(st.m, kLog2e, -M);
  return (st.m - z) + kLn2 * (log2_fast(st.s) - resid);
}

// ------------------------------------------------------------ wave64 cross-lane
// Butterfly over all 64 lanes: quad swaps (DPP quad_perm), half-row and row
// mirrors (DPP), then the 16- and 32-lane swaps of gfx950 (v_permlane16_swap,
// v_permlane32_swap).  Every lane ends with the same value, and the order of
// operations is fixed, so the result is bitwise reproducible.

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <typename Op>
__device__ __forceinline__ float wave_allreduce(float v, Op op) {
  v = op(v, dpp_f<kDppQuadXor1>(v));
  v = op(v, dpp_f<kDppQuadXor2>(v));
  v = op(v, dpp_f<kDppRowHalfMirror>(v));
  v = op(v, dpp_f<kDppRowMirror>(v));
  {
    auto p = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
    v = op(__int_as_float(p[0]), __int_as_float(p[1]));
  }
  {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
    v = op(__int_as_float(p[0]), __int_as_float(p[1]));
  }
  return v;
}

struct MaxOp {
  __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct AddOp {
  __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};

__device__ __forceinline__ float wave_max(float v) { return wave_allreduce(v, MaxOp{}); }
__device__ __forceinline__ float wave_sum(float v) { return wave_allreduce(v, AddOp{}); }

// Combine the 64 lanes' states: global max first, then each lane rescales its
// own sum to it, then one sum reduction.  All lanes return the row state.
__device__ __forceinline__ Lse wave_lse(Lse st) {
  const float m = wave_max(st.m);
  const float s = wave_sum(st.s * lse_rescale(st.m, m));
  return {m, s};
}

// Swap partner across the two 32-lane halves (lane l <-> lane l ^ 32).
__device__ __forceinline__ float half_swap(float v) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  // p[0] holds the low half in both halves, p[1] the high half in both halves.
  return (__lane_id() < 32) ? __int_as_float(p[1]) : __int_as_float(p[0]);
}

__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// ------------------------------------------------------------ deterministic mean
// Every workgroup leaves one fp32 partial; the workgroup that finishes last
// adds all partials in a fixed order and writes the mean.  No float atomics
// are used, so the result is bitwise reproducible.
//
// Finding the last workgroup: a two-level integer ticket.  Workgroup b counts
// itself in group counter b % G (G <= 64 counters, each on its own 256-byte
// line so they do not serialise on one address); the workgroup that completes
// a group counts the group in the top counter; the one that completes the top
// counter is last.  Each completing workgroup resets the counter it completed,
// so all counters are zero again when the kernel ends.
//
// Visibility across the XCDs (each has its own L2): the partials are written
// and read only with agent-scope atomic stores and loads, which are coherent
// at agent scope by themselves, and each writer waits for its store to
// complete (s_waitcnt) before it touches a counter.  A release/acquire fence
// pair would instead write back (and invalidate) a whole L2 per workgroup.
//
// Only wave 0 takes part: the other waves of the workgroup retire at once, so
// the hand-off's memory round trips do not hold their slots.
constexpr int kTicketGroups = 64;
constexpr int kTicketStride = 64;  // unsigned ints (256 bytes) between counters

// `block_sum` must be valid in thread 0; every thread of the workgroup calls
// this after its last barrier.  Threads of waves other than 0 return at once.
__device__ __forceinline__ void finish_mean(float block_sum, float* partials, unsigned* ticket,
                                            float* out, int64_t tokens) {
  if (threadIdx.x >= 64) return;
  const unsigned lane = threadIdx.x;
  const unsigned nblocks = gridDim.x * gridDim.y;
  const unsigned bid = blockIdx.y * gridDim.x + blockIdx.x;
  const unsigned G = nblocks < (unsigned)kTicketGroups ? nblocks : (unsigned)kTicketGroups;
  const unsigned g = bid % G;
  const unsigned group_size = nblocks / G + (g < nblocks % G ? 1u : 0u);
  unsigned* group_ctr = ticket + g * kTicketStride;
  unsigned* top_ctr = ticket + kTicketGroups * kTicketStride;
  int last = 0;
  if (lane == 0) {
    __hip_atomic_store(&partials[bid], block_sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);  // the partial store has completed
    if (__hip_atomic_fetch_add(group_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
        group_size - 1) {
      __hip_atomic_store(group_ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);
      last = __hip_atomic_fetch_add(top_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == G - 1;
    }
  }
  if (!wave_uniform(last)) return;
  float acc = 0.0f;
  for (unsigned i = lane; i < nblocks; i += 64)
    acc += __hip_atomic_load(&partials[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const float total = wave_sum(acc);
  if (lane == 0) {
    out[0] = total / (float)tokens;
    __hip_atomic_store(top_ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace lce
