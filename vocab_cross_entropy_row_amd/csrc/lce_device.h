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

// The same butterfly over groups of N consecutive lanes (N = 8, 16 or 32: its
// first 3, 4 or 5 steps); every lane ends with its group's value.
template <int N, typename Op>
__device__ __forceinline__ float group_allreduce(float v, Op op) {
  static_assert(N == 8 || N == 16 || N == 32, "group of 8, 16 or 32 lanes");
  v = op(v, dpp_f<kDppQuadXor1>(v));
  v = op(v, dpp_f<kDppQuadXor2>(v));
  v = op(v, dpp_f<kDppRowHalfMirror>(v));
  if constexpr (N >= 16) v = op(v, dpp_f<kDppRowMirror>(v));
  if constexpr (N >= 32) {
    auto p = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
    v = op(__int_as_float(p[0]), __int_as_float(p[1]));
  }
  return v;
}

// Combine the 64 lanes' states: global max first, then each lane rescales its
// own sum to it, then one sum reduction.  All lanes return the row state.
__device__ __forceinline__ Lse wave_lse(Lse st) {
  const float m = wave_max(st.m);
  const float s = wave_sum(st.s * lse_rescale(st.m, m));
  return {m, s};
}

// The same over groups of N consecutive lanes (one row per group).
template <int N>
__device__ __forceinline__ Lse group_lse(Lse st) {
  const float m = group_allreduce<N>(st.m, MaxOp{});
  const float s = group_allreduce<N>(st.s * lse_rescale(st.m, m), AddOp{});
  return {m, s};
}

// Swap partner across the two 32-lane halves (lane l <-> lane l ^ 32).
__device__ __forceinline__ float half_swap(float v) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  // p[0] holds the low half in both halves, p[1] the high half in both halves.
  return (__lane_id() < 32) ? __int_as_float(p[1]) : __int_as_float(p[0]);
}

__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Buffer resource over `bytes` bytes at `base` (raw, unswizzled): a load whose
// VGPR offset plus immediate offset is at or past `bytes` reads no memory and
// returns zero.  gfx9 word 3: 32-bit data format, no swizzle.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// ------------------------------------------------------------ deterministic mean
// Every workgroup contributes one fp32 partial; one workgroup adds all
// partials in a fixed order and writes the mean.  No float atomics are used,
// so the result is bitwise reproducible.
//
// The finisher is the workgroup with the highest index.  Workgroups are
// dispatched in index order, so when the finisher starts every other
// workgroup has started and none waits on anything: the finisher's wait for
// the partials always ends.  Every other workgroup writes its partial as one
// 64-bit agent-scope atomic store of (tag, value) and retires at once,
// without any returning atomic.  The tag is the launch's epoch + 1: each
// workgroup reads the epoch word when it starts (mean_begin, so the load's
// latency hides under its rows) and the finisher advances it for the next
// launch on this buffer.  The finisher polls each slot until it carries this
// launch's tag, so data and flag arrive together; slots left by earlier
// launches carry older tags (a new buffer is zeroed, and tags start at 1).
// After the last row the chain is the last partial's store and one read of
// it.  Agent-scope atomics are coherent across the XCDs (each has its own L2)
// without writing back or invalidating an L2.  The finisher's polling is
// bounded (kPollBudget re-reads per lane, a short sleep between them): a
// launch that runs out of it writes NaN instead of hanging.
//
// In the other workgroups only thread 0 stores; the finisher's waves all read.
constexpr int kEpochWord = 0;                  // the mean state's header: the epoch word
constexpr unsigned kPollBudget = 1u << 24;     // safety net: never reached by a correct launch

__device__ __forceinline__ uint64_t mean_slot(unsigned tag, float v) {
  return ((uint64_t)tag << 32) | __float_as_uint(v);
}

// The launch's tag (epoch + 1), read by thread 0 of a workgroup when it
// starts; 0 (unused) without a mean or in the only workgroup.  Pass the result
// to finish_mean.
__device__ __forceinline__ unsigned mean_begin(const unsigned* epoch, int reduce_mean) {
  unsigned tag = 0;
  if (reduce_mean && threadIdx.x == 0 && gridDim.x * gridDim.y > 1)
    tag = __hip_atomic_load(epoch + kEpochWord, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  return tag;
}

// `block_sum` and `tag` (from mean_begin) must be valid in thread 0; every
// thread of the workgroup calls this after its last barrier.  `slots` holds
// one 64-bit slot per workgroup.  In the finisher every wave reads a share of
// the slots (slot i goes to wave (i / 64) mod W and lane i mod 64), each lane
// adding its share in fp64 in slot order; the waves' sums are then added in
// wave order.
__device__ __forceinline__ void finish_mean(float block_sum, uint64_t* slots, unsigned* epoch,
                                            unsigned tag, float* out, int64_t tokens) {
  const unsigned nblocks = gridDim.x * gridDim.y;
  if (nblocks == 1) {  // the only workgroup: no hand-off (same result as the general path)
    if (threadIdx.x == 0) out[0] = block_sum / (float)tokens;
    return;
  }
  const unsigned bid = blockIdx.y * gridDim.x + blockIdx.x;
  if (bid != nblocks - 1) {
    if (threadIdx.x == 0)
      __hip_atomic_store(&slots[bid], mean_slot(tag, block_sum), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  constexpr int kMaxWaves = 16;
  __shared__ unsigned fin_tag;
  __shared__ float fin_own, fin_sum[kMaxWaves];
  __shared__ int fin_bad[kMaxWaves];
  const unsigned lane = threadIdx.x & 63u;
  const unsigned wave = threadIdx.x >> 6;
  const unsigned W = (blockDim.x + 63u) >> 6;  // at most kMaxWaves
  if (threadIdx.x == 0) {
    fin_tag = tag;
    fin_own = block_sum;
  }
  __syncthreads();
  tag = fin_tag;
  const float own = fin_own;
  constexpr int kInFlight = 8;  // slot loads per lane in flight
  const unsigned stride = 64u * W;
  // Each lane adds its share (nblocks / (64 W) partials, up to hundreds of
  // thousands for the largest grids) in fp64, so the sum's rounding does not
  // grow with the number of workgroups.
  double acc = 0.0;
  bool ok = true;
  unsigned budget = kPollBudget;
  for (unsigned base = lane + 64u * wave; base < nblocks; base += stride * kInFlight) {
    uint64_t v[kInFlight];
#pragma unroll
    for (int j = 0; j < kInFlight; ++j) {
      const unsigned i = base + stride * j;
      v[j] = (i < nblocks && i != bid)
                 ? __hip_atomic_load(&slots[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                 : mean_slot(tag, own);
    }
#pragma unroll
    for (int j = 0; j < kInFlight; ++j) {
      const unsigned i = base + stride * j;
      if (i >= nblocks) break;
      while ((unsigned)(v[j] >> 32) != tag && budget > 0) {
        --budget;
        __builtin_amdgcn_s_sleep(2);
        v[j] = __hip_atomic_load(&slots[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      ok = ok && (unsigned)(v[j] >> 32) == tag;
      acc += (double)__uint_as_float((unsigned)v[j]);
    }
  }
  const float wsum = wave_sum((float)acc);
  const bool wave_ok = __builtin_amdgcn_ballot_w64(!ok) == 0;
  if (lane == 0) {
    fin_sum[wave] = wsum;
    fin_bad[wave] = wave_ok ? 0 : 1;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float total = 0.0f;
    bool all_ok = true;
    for (unsigned w = 0; w < W; ++w) {
      total += fin_sum[w];
      all_ok = all_ok && fin_bad[w] == 0;
    }
    out[0] = all_ok ? total / (float)tokens : __builtin_nanf("");
    __hip_atomic_store(epoch + kEpochWord, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ------------------------------------------------------------ generalized JSD
// One vocab entry's divergence term  beta P (ln P - ln M) + (1 - beta) Q (ln Q - ln M)
// from lp = ln P and lq = ln Q.  Relative to mx = max(lp, lq): ln M = mx + ln S
// with S = beta e^u + (1 - beta) e^w >= min(beta, 1 - beta), u = lp - mx and
// w = lq - mx (one of them 0), so no underflowing P, Q or M reaches the
// logarithm, and a term below the fp32 range is 0.
__device__ __forceinline__ float jsd_term(float lp, float lq, float beta) {
  const float mx = __builtin_fmaxf(lp, lq);
  const float u = lp - mx, w = lq - mx;
  const float e = exp2_fast((u + w) * kLog2e);  // e^(-|lp - lq|)
  const float eu = lp >= lq ? 1.0f : e;
  const float ew = lp >= lq ? e : 1.0f;
  const float ls = kLn2 * log2_fast(beta * eu + (1.0f - beta) * ew);
  return exp2_fast(mx * kLog2e) * (beta * eu * (u - ls) + (1.0f - beta) * ew * (w - ls));
}

}  // namespace lce
