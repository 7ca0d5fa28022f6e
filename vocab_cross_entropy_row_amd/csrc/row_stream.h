// Device-side building blocks shared by the row kernels (forward, shard
// statistics, gradient): 16-byte chunk types, the split of a row into an
// aligned body and scalar edges, the batch folds of the running
// (max, sum-exp) state, and the streaming loops over a row's aligned body.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lce_device.h"
#include "lce_internal.h"

namespace lce {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Vec;
template <>
struct Vec<float> {
  static constexpr int kElems = 4;
  typedef f32x4 raw;
  __device__ __forceinline__ static raw neg_inf() { return (raw)(kNegInf); }
  __device__ __forceinline__ static float get(const raw& r, int e) { return r[e]; }
  __device__ __forceinline__ static float get_again(const raw& r, int e) { return r[e]; }
  __device__ __forceinline__ static float scalar(const float* p) { return *p; }
};
template <>
struct Vec<uint16_t> {  // bf16 bit patterns, two per 32-bit word
  static constexpr int kElems = 8;
  typedef u32x4 raw;
  __device__ __forceinline__ static raw neg_inf() { return (raw)(0xff80ff80u); }  // bf16 -inf pairs
  __device__ __forceinline__ static float get(const raw& r, int e) {
    return (e & 1) ? bf16_hi(r[e >> 1]) : bf16_lo(r[e >> 1]);
  }
  // The same decode, opaque to common-subexpression elimination: the exp pass
  // decodes again instead of keeping every decoded value of the max pass alive
  // (one VALU op per element, against 32 VGPRs of a batch of 4 chunks).
  __device__ __forceinline__ static float get_again(const raw& r, int e) {
    uint32_t out;
    if (e & 1)
      asm volatile("v_and_b32 %0, 0xffff0000, %1" : "=v"(out) : "v"(r[e >> 1]));
    else
      asm volatile("v_lshlrev_b32 %0, 16, %1" : "=v"(out) : "v"(r[e >> 1]));
    return __uint_as_float(out);
  }
  __device__ __forceinline__ static float scalar(const uint16_t* p) { return bf16_to_f32(*p); }
};

// Split of one row into scalar head, 16-byte-aligned vector body, scalar tail.
struct RowSplit {
  int head;    // elements before the first aligned chunk
  int nvec;    // aligned 16-byte chunks
  int tail;    // elements after the last chunk
};

template <typename T>
__device__ __forceinline__ RowSplit row_split(const T* row, int vocab) {
  constexpr int E = Vec<T>::kElems;
  const int mis = (int)(((uintptr_t)row & 15u) / sizeof(T));
  int head = mis ? (E - mis) : 0;
  head = head < vocab ? head : vocab;
  const int body = vocab - head;
  return {head, body / E, body % E};
}

// Pairwise sum of per-chunk sums part[U0..U) (keeps the fp32 error small).
template <int U, int U0>
__device__ __forceinline__ float sum_parts(float (&part)[U]) {
#pragma unroll
  for (int w = 1; w < U - U0; w <<= 1)
#pragma unroll
    for (int u = U0; u + w < U; u += 2 * w) part[u] += part[u + w];
  return part[U0];
}

// Two-pass fold of chunks [U0, U1) of a batch into the running state: the
// batch maximum first, then the sum of exponentials against the new maximum.
// Padding chunks hold -inf, which contributes 2^-inf = 0.
template <typename T, int U, int U0, int U1>
__device__ __forceinline__ void fold_two_pass(Lse& st, const typename Vec<T>::raw (&v)[U]) {
  static_assert(0 <= U0 && U0 < U1 && U1 <= U, "chunk range");
  constexpr int E = Vec<T>::kElems;
  float bm = kNegInf;
#pragma unroll
  for (int u = U0; u < U1; ++u)
#pragma unroll
    for (int e = 0; e < E; ++e) bm = fmaxf(bm, Vec<T>::get(v[u], e));
  const float mn = fmaxf(st.m, bm);
  if (mn == kNegInf) return;  // nothing but -inf so far
  const float Mn = mn * kLog2e;
  float part[U];
#pragma unroll
  for (int u = U0; u < U1; ++u) {
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc += exp2_fast(__builtin_fmaf(Vec<T>::get_again(v[u], e), kLog2e, -Mn));
    part[u] = acc;
  }
  // pairwise sum of the per-chunk sums keeps the fp32 error small
#pragma unroll
  for (int w = 1; w < U1 - U0; w <<= 1)
#pragma unroll
    for (int u = U0; u + w < U1; u += 2 * w) part[u] += part[u + w];
  st.s = st.s * lse_rescale(st.m, mn) + part[U0];
  st.m = mn;
}

// Rise of the running maximum (log2 units) up to which a batch's terms, taken
// against the old reference, are rescaled to the new one instead of taken
// again.  Rescaling carries two roundings of each term's exponent (the FMA's
// result and the difference of the references), each at most half an ulp of
// the rise: below 8 that is 2^-22, so the batch's largest term, which becomes
// the row's largest, is off by at most 2^-21 * ln 2 = 3.3e-7 relative.  Past
// the cut-off (and always before a term could overflow fp32) the exponentials
// are taken again against the new maximum.
constexpr float kRescaleRise = 8.0f;

// One-pass fold of chunks [U0, U) against the running maximum, which must be
// finite: each element is decoded once and feeds both the batch maximum and
// its exponential 2^(z*L - fp32(m*L)).  If the batch raised the maximum by at
// most kRescaleRise, the sum is rescaled to the new one afterwards; if it
// raised it further, the batch's exponentials are taken again against the new
// maximum.  Per element this is one decode, a third of a 3-input max, one FMA,
// one exponential and one add: one decode less than the two-pass fold.
template <typename T, int U, int U0>
__device__ __forceinline__ void fold_one_pass(Lse& st, const typename Vec<T>::raw (&v)[U]) {
  static_assert(0 <= U0 && U0 < U, "chunk range");
  constexpr int E = Vec<T>::kElems;
  const float M = st.m * kLog2e;
  float bm = kNegInf;
  float part[U];
#pragma unroll
  for (int u = U0; u < U; ++u) {
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float z = Vec<T>::get_again(v[u], e);
      bm = fmaxf(bm, z);
      acc += exp2_fast(__builtin_fmaf(z, kLog2e, -M));
    }
    part[u] = acc;
  }
  if (bm > st.m) {
    if (bm * kLog2e - M > kRescaleRise) {
      const float Mn = bm * kLog2e;
#pragma unroll
      for (int u = U0; u < U; ++u) {
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e)
          acc += exp2_fast(__builtin_fmaf(Vec<T>::get_again(v[u], e), kLog2e, -Mn));
        part[u] = acc;
      }
      st.s *= lse_rescale(st.m, bm);
    } else {
      st.s = (st.s + sum_parts<U, U0>(part)) * lse_rescale(st.m, bm);
      st.m = bm;
      return;
    }
    st.m = bm;
  }
  st.s += sum_parts<U, U0>(part);
}

// Fixed-reference fold of chunks [U0, U): the sum of 2^(z*L - M) against the
// state's M, which is left where it is even when a chunk holds a larger
// logit.  The state stays exact (s is still relative to fp32(m*L)), but s is
// no longer bounded by the element count: a logit d above the reference adds
// e^d.  Per element this is one decode, one FMA, one exponential and one add
// (no maximum).  Callers check the finished lane sums against kRefGuard and
// fold the row again with the tracked fold when any sum is not below it.
template <typename T, int U, int U0>
__device__ __forceinline__ void fold_fixed(Lse& st, const typename Vec<T>::raw (&v)[U]) {
  static_assert(0 <= U0 && U0 < U, "chunk range");
  constexpr int E = Vec<T>::kElems;
  const float M = st.m * kLog2e;
  float part[U];
#pragma unroll
  for (int u = U0; u < U; ++u) {
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc += exp2_fast(__builtin_fmaf(Vec<T>::get_again(v[u], e), kLog2e, -M));
    part[u] = acc;
  }
  st.s += sum_parts<U, U0>(part);
}

// Bound on a lane sum built by fold_fixed.  Below it, every later merge stays
// far from fp32 overflow (64 lanes, the waves of a workgroup and any number of
// split partials add at most a few powers of two, and rescaling only shrinks a
// sum); a sum at or above it, or one that is inf or NaN, sends the row to the
// tracked fold.  Only a logit about 44 above its lane's reference (the
// maximum of the lane's first finite chunk) can reach it.
constexpr float kRefGuard = 0x1p64f;

__device__ __forceinline__ bool lane_sum_unsafe(const Lse& st) { return !(st.s < kRefGuard); }

// Tag selecting the tracked (true) or fixed-reference (false) batch fold.
template <bool B>
struct TrackMax {
  static constexpr bool value = B;
};

// Fold a batch of loaded chunks into the running state.  A lane that has seen
// no finite logit yet (always so in the first batch, FIRST) takes its maximum
// from two passes over the first chunk, then folds the rest in one pass:
// max-tracking (TRACK) or against that fixed reference.
template <typename T, int U, bool FIRST = false, bool TRACK = true>
__device__ __forceinline__ void fold_batch(Lse& st, const typename Vec<T>::raw (&v)[U]) {
  if (FIRST || st.m == kNegInf) {
    fold_two_pass<T, U, 0, 1>(st, v);
    if constexpr (U > 1) {
      if (st.m == kNegInf)
        fold_two_pass<T, U, 1, U>(st, v);  // nothing but -inf so far
      else if constexpr (TRACK)
        fold_one_pass<T, U, 1>(st, v);
      else
        fold_fixed<T, U, 1>(st, v);
    }
  } else if constexpr (TRACK) {
    fold_one_pass<T, U, 0>(st, v);
  } else {
    fold_fixed<T, U, 0>(st, v);
  }
}

// Fold one scalar (or -inf) into the state.
__device__ __forceinline__ void fold_one(Lse& st, float z) {
  const float mn = fmaxf(st.m, z);
  if (mn == kNegInf) return;
  st.s = st.s * lse_rescale(st.m, mn) + exp2_fast(__builtin_fmaf(z, kLog2e, -(mn * kLog2e)));
  st.m = mn;
}

// Cache policy of the streaming loads: nt (each logit is read once).
constexpr int kStreamPolicy = 2;

// Load chunks c + u * step (u < U) through buffer resource `rs`; chunks at or
// past the resource's end read no memory and come back as zero.
template <typename T, int U>
__device__ __forceinline__ void load_batch(typename Vec<T>::raw (&v)[U], __amdgpu_buffer_rsrc_t rs,
                                           int c, int step) {
  typedef typename Vec<T>::raw raw;
#pragma unroll
  for (int u = 0; u < U; ++u)
    v[u] = (raw)__builtin_amdgcn_raw_buffer_load_b128(rs, (c + u * step) * 16, 0, kStreamPolicy);
}

// Chunks at or past chunk n become -inf, which folds as nothing.
template <typename T, int U>
__device__ __forceinline__ void mask_past(typename Vec<T>::raw (&v)[U], int c, int n, int step) {
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (c + u * step >= n) v[u] = Vec<T>::neg_inf();
}

// Stream chunks [c0, c1) of the aligned body: lane `first` of a group of
// `step` lanes takes chunks c0 + first + k * step, U per batch.  c0, c1 and
// step are uniform over the group.  Two batches live in registers and the
// next batch's loads are issued before the current one is folded, so up to
// 2 * U chunks per lane are in flight.  Every load is unconditional: loads
// past c1 (the lanes beyond a ragged end, and the batch after the last one)
// read nothing, and only the last batch of a ragged range is masked.
// `extra()` is called once, right after the first loads are issued (also
// for an empty range): the row's few scalar loads go there, so that their
// latency overlaps the stream instead of adding to it.
// TRACK selects the batch fold (fold_batch).  The caller keeps (c1 - c0) * 16
// below 2^31.
template <typename T, int U, bool TRACK = true, typename Extra>
__device__ __forceinline__ void stream_chunks(Lse& st, const typename Vec<T>::raw* body, int c0,
                                              int c1, int first, int step, Extra&& extra) {
  typedef typename Vec<T>::raw raw;
  const int n = wave_uniform(c1 - c0);
  if (n <= 0) {
    extra();
    return;
  }
  const int S = step * U;
  const int last = wave_uniform((n - 1) / S);  // index of the last batch
  const bool ragged = (n % S) != 0;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(body + c0, (uint32_t)n * 16u);
  int c = first;
  raw a[U], b[U];
  load_batch<T, U>(a, rs, c, step);
  __builtin_amdgcn_sched_barrier(0);
  extra();
  for (int k = 0;; k += 2) {
    load_batch<T, U>(b, rs, c + S, step);
    if (ragged && k == last) mask_past<T, U>(a, c, n, step);
    fold_batch<T, U, false, TRACK>(st, a);
    if (k == last) break;
    c += S;
    load_batch<T, U>(a, rs, c + S, step);
    if (ragged && k + 1 == last) mask_past<T, U>(b, c, n, step);
    fold_batch<T, U, false, TRACK>(st, b);
    if (k + 1 == last) break;
    c += S;
  }
}

// The same for ranges of at most MAXB batches, fully unrolled by template
// recursion (batch K is a compile-time constant, so the two register batches
// are never indexed at run time): with no loop back edge every fold waits for
// exactly its own batch (a loop header makes the compiler drain all loads).
struct ShortRange {
  __amdgpu_buffer_rsrc_t rs;
  int first, step, n, last;
  bool ragged;
};

template <typename T, int U, int MAXB, int K, bool TRACK, typename Extra>
__device__ __forceinline__ void short_step(Lse& st, typename Vec<T>::raw (&cur)[U],
                                           typename Vec<T>::raw (&nxt)[U], const ShortRange& r,
                                           Extra& extra) {
  const int c = r.first + K * r.step * U;
  if constexpr (K + 1 < MAXB) load_batch<T, U>(nxt, r.rs, c + r.step * U, r.step);
  if constexpr (K == 0) {
    __builtin_amdgcn_sched_barrier(0);
    extra();
  }
  if (r.ragged && K == r.last) mask_past<T, U>(cur, c, r.n, r.step);
  fold_batch<T, U, K == 0, TRACK>(st, cur);
  if constexpr (K + 1 < MAXB) {
    if (K != r.last) short_step<T, U, MAXB, K + 1, TRACK>(st, nxt, cur, r, extra);
  }
}

template <typename T, int U, int MAXB, bool TRACK = true, typename Extra>
__device__ __forceinline__ void stream_chunks_short(Lse& st, const typename Vec<T>::raw* body,
                                                    int c0, int c1, int first, int step,
                                                    Extra&& extra) {
  typedef typename Vec<T>::raw raw;
  const int n = wave_uniform(c1 - c0);
  if (n <= 0) {
    extra();
    return;
  }
  const int S = step * U;
  const ShortRange r{make_rsrc(body + c0, (uint32_t)n * 16u), first, step, n,
                     wave_uniform((n - 1) / S), (n % S) != 0};
  raw a[U], b[U];
  load_batch<T, U>(a, r.rs, first, step);
  short_step<T, U, MAXB, 0, TRACK>(st, a, b, r, extra);
}

// Index of the scalar head or tail element that lane `idx` folds when
// idx < head + tail; any in-row index (0) otherwise, so the load is always valid.
__device__ __forceinline__ int edge_index(const RowSplit& rs, int vocab, int idx) {
  if (idx >= rs.head + rs.tail) return 0;
  return (idx < rs.head) ? idx : (vocab - rs.tail + (idx - rs.head));
}

// Target index usable for a load: t itself when valid, else 0 (then the loss is NaN).
__device__ __forceinline__ int64_t safe_target(int64_t t, int vocab) {
  return (t >= 0 && t < (int64_t)vocab) ? t : 0;
}

// Index of the target within this row's columns: t - vocab_start when the row
// holds it, else -1 (a whole row has vocab_start = 0).
__device__ __forceinline__ int64_t local_target(int64_t t, int64_t vocab_start, int vocab) {
  return (t >= vocab_start && t - vocab_start < (int64_t)vocab) ? t - vocab_start : -1;
}

// Shard statistics of a row state: (m, sum of e^(z - m), target logit or NaN).
// The state's sum is relative to M = fp32(m*log2e); e^(z - m) = 2^(z*L - M) *
// 2^(M - m*L), and M - m*L is minus the exact residual fma(m, L, -M).
__device__ __forceinline__ void write_stats(float* dst, const Lse& r, bool holds_target, float zt) {
  const float s = (r.m == kNegInf) ? 0.0f
                                   : r.s * exp2_fast(-__builtin_fmaf(r.m, kLog2e, -(r.m * kLog2e)));
  dst[0] = r.m;
  dst[1] = s;
  dst[2] = holds_target ? zt : __builtin_nanf("");
}

// The target index, made opaque where this is called: code that uses the
// result cannot be hoisted above it, so the wait for the target's scalar load
// lands behind the first batch of logit loads instead of in front of them.
__device__ __forceinline__ int64_t target_here(int64_t t) {
  __asm__ volatile("" : "+s"(t));
  return t;
}

// Merge the 4 waves' states of a workgroup through LDS; every thread returns
// the workgroup's state.
__device__ __forceinline__ Lse block_lse(Lse st) {
  constexpr int kWaves = kRowThreads / 64;
  __shared__ float sm[kWaves], ss[kWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const Lse w = wave_lse(st);
  if (lane == 0) {
    sm[wave] = w.m;
    ss[wave] = w.s;
  }
  __syncthreads();
  float m = sm[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) m = fmaxf(m, sm[i]);
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) s += ss[i] * lse_rescale(sm[i], m);
  return {m, s};
}

}  // namespace lce
