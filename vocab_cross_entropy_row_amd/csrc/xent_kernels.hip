// Row cross-entropy kernels for gfx950.
//
// Computes, for every token row of a [tokens, vocab] logit matrix (fp32 or
// bf16), loss = ln(sum_j e^z_j) - z_target, and optionally their mean
// (KernelIndex "Cross-entropy loss" and "Vocab-parallel cross-entropy,
// Megatron layout": descriptions and Semantics blocks).
//
// The work is one pass over HBM: every logit is read once with 16-byte loads
// (4 fp32 or 8 bf16 per lane per load), consecutive lanes read consecutive
// 16-byte chunks, and each lane folds what it loaded into a running
// (max, sum-exp) state in fp32 (see lce_device.h).  Loads are issued in
// batches of U chunks per lane before any arithmetic, so each wave keeps
// U * 1 KiB in flight.
//
// Three layouts of work over rows:
//   wave_rows   one wavefront per row, 4 rows per workgroup (short rows);
//   block_rows  one 256-thread workgroup per row; the 4 waves stream the row
//               together and merge their states through LDS (long rows);
//   split       S workgroups per row write (max, sum-exp) partials, and a
//               merge kernel combines them (long rows, few tokens).
// Rows need not be 16-byte aligned: the few elements before the first
// aligned chunk and after the last one are loaded one by one.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lce_device.h"
#include "lce_internal.h"

namespace lce {

static_assert(kTicketBytes == (kTicketGroups + 1) * kTicketStride * sizeof(unsigned),
              "host scratch layout must match the device ticket layout");

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

// Fold a batch of loaded chunks into the running state.  Padding lanes hold
// -inf, which contributes 2^-inf = 0.
template <typename T, int U>
__device__ __forceinline__ void fold_batch(Lse& st, const typename Vec<T>::raw (&v)[U]) {
  constexpr int E = Vec<T>::kElems;
  float bm = kNegInf;
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int e = 0; e < E; ++e) bm = fmaxf(bm, Vec<T>::get(v[u], e));
  const float mn = fmaxf(st.m, bm);
  if (mn == kNegInf) return;  // nothing but -inf so far
  const float Mn = mn * kLog2e;
  float part[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc += exp2_fast(__builtin_fmaf(Vec<T>::get(v[u], e), kLog2e, -Mn));
    part[u] = acc;
  }
  // pairwise sum of the per-chunk sums keeps the fp32 error small
#pragma unroll
  for (int w = 1; w < U; w <<= 1)
#pragma unroll
    for (int u = 0; u + w < U; u += 2 * w) part[u] += part[u + w];
  st.s = st.s * lse_rescale(st.m, mn) + part[0];
  st.m = mn;
}

// Fold one scalar (or -inf) into the state.
__device__ __forceinline__ void fold_one(Lse& st, float z) {
  const float mn = fmaxf(st.m, z);
  if (mn == kNegInf) return;
  st.s = st.s * lse_rescale(st.m, mn) + exp2_fast(__builtin_fmaf(z, kLog2e, -(mn * kLog2e)));
  st.m = mn;
}

// Stream chunks [c0, c1) of the aligned body with stride `step` starting at
// chunk `c0 + first`, U chunks per lane per batch.
template <typename T, int U>
__device__ __forceinline__ void stream_chunks(Lse& st, const typename Vec<T>::raw* body, int c0,
                                              int c1, int first, int step) {
  typedef typename Vec<T>::raw raw;
  for (int base = c0 + first; base < c1; base += step * U) {
    raw v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = base + u * step;
      v[u] = (c < c1) ? __builtin_nontemporal_load(body + c) : Vec<T>::neg_inf();
    }
    fold_batch<T, U>(st, v);
  }
}

// Scalar head and tail elements of a row, one per lane (at most 2 * (E - 1)).
template <typename T>
__device__ __forceinline__ void fold_edges(Lse& st, const T* row, const RowSplit& rs, int vocab,
                                           int idx) {
  const int edges = rs.head + rs.tail;
  if (idx < edges) {
    const int j = (idx < rs.head) ? idx : (vocab - rs.tail + (idx - rs.head));
    fold_one(st, Vec<T>::scalar(row + j));
  }
}

// loss = ln(sum e^z) - z_t, or NaN when the target is out of range.  `t` is uniform.
template <typename T>
__device__ __forceinline__ float row_loss(const Lse& st, const T* row, int64_t t, int vocab) {
  if (t < 0 || t >= (int64_t)vocab) return __builtin_nanf("");
  return lse_minus(st, Vec<T>::scalar(row + t));
}

// ------------------------------------------------------------ one wave per row
// WAVES rows (one per wave) per workgroup.  With a mean, larger workgroups
// mean fewer partials and fewer ticket hand-offs.
template <typename T, int U, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void xent_wave_rows_kernel(
    const T* __restrict__ logits, int64_t tokens, int vocab, const int64_t* __restrict__ target,
    float* __restrict__ out, float* __restrict__ partials, unsigned* __restrict__ ticket,
    int reduce_mean) {
  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int64_t row = (int64_t)blockIdx.x * WAVES + wave;
  float loss = 0.0f;
  if (row < tokens) {
    const T* rp = logits + row * (int64_t)vocab;
    const int64_t t = target[row];
    const RowSplit rs = row_split(rp, vocab);
    const typename Vec<T>::raw* body =
        reinterpret_cast<const typename Vec<T>::raw*>(rp + rs.head);
    Lse st = lse_empty();
    fold_edges(st, rp, rs, vocab, lane);
    stream_chunks<T, U>(st, body, 0, rs.nvec, lane, 64);
    const Lse r = wave_lse(st);
    loss = row_loss(r, rp, t, vocab);
    if (!reduce_mean && lane == 0) out[row] = loss;
  }
  if (reduce_mean) {
    __shared__ float wl[WAVES];
    if (lane == 0) wl[wave] = loss;
    __syncthreads();
    float bsum = 0.0f;
    if (threadIdx.x == 0)
      for (int w = 0; w < WAVES; ++w) bsum += wl[w];
    finish_mean(bsum, partials, ticket, out, tokens);
  }
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

// ------------------------------------------------------------ one workgroup per row
template <typename T, int U>
__global__ __launch_bounds__(kRowThreads) void xent_block_rows_kernel(
    const T* __restrict__ logits, int64_t tokens, int vocab, const int64_t* __restrict__ target,
    float* __restrict__ out, float* __restrict__ partials, unsigned* __restrict__ ticket,
    int reduce_mean) {
  const int64_t row = blockIdx.x;
  const T* rp = logits + row * (int64_t)vocab;
  const int64_t t = target[row];
  const RowSplit rs = row_split(rp, vocab);
  const typename Vec<T>::raw* body = reinterpret_cast<const typename Vec<T>::raw*>(rp + rs.head);
  Lse st = lse_empty();
  fold_edges(st, rp, rs, vocab, threadIdx.x);
  stream_chunks<T, U>(st, body, 0, rs.nvec, threadIdx.x, kRowThreads);
  const Lse r = block_lse(st);
  const float loss = row_loss(r, rp, t, vocab);
  if (!reduce_mean) {
    if (threadIdx.x == 0) out[row] = loss;
  } else {
    finish_mean(loss, partials, ticket, out, tokens);
  }
}

// ------------------------------------------------------------ split rows
// grid = (S, tokens).  Workgroup (s, row) streams chunk slice s of the row and
// writes its state to part[row * S + s]; slice 0 also folds the scalar edges.
template <typename T, int U>
__global__ __launch_bounds__(kRowThreads) void xent_split_partial_kernel(
    const T* __restrict__ logits, int vocab, int chunks_per_slice, float2* __restrict__ part) {
  const int S = gridDim.x;
  const int s = blockIdx.x;
  const int64_t row = blockIdx.y;
  const T* rp = logits + row * (int64_t)vocab;
  const RowSplit rs = row_split(rp, vocab);
  const typename Vec<T>::raw* body = reinterpret_cast<const typename Vec<T>::raw*>(rp + rs.head);
  Lse st = lse_empty();
  if (s == 0) fold_edges(st, rp, rs, vocab, threadIdx.x);
  const int c0 = s * chunks_per_slice;
  int c1 = c0 + chunks_per_slice;
  c1 = c1 < rs.nvec ? c1 : rs.nvec;
  stream_chunks<T, U>(st, body, c0, c1, threadIdx.x, kRowThreads);
  const Lse r = block_lse(st);
  if (threadIdx.x == 0) part[row * S + s] = make_float2(r.m, r.s);
}

// One wave per row merges that row's S partials (lanes read them in order,
// then the wave reduction), then finishes the loss.
template <typename T>
__global__ __launch_bounds__(kRowThreads) void xent_split_merge_kernel(
    const T* __restrict__ logits, int64_t tokens, int vocab, int S,
    const float2* __restrict__ part, const int64_t* __restrict__ target, float* __restrict__ out,
    float* __restrict__ partials, unsigned* __restrict__ ticket, int reduce_mean) {
  constexpr int kWaves = kRowThreads / 64;
  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int64_t row = (int64_t)blockIdx.x * kWaves + wave;
  float loss = 0.0f;
  if (row < tokens) {
    Lse st = lse_empty();
    for (int i = lane; i < S; i += 64) {
      const float2 p = part[row * S + i];
      st = lse_merge(st, Lse{p.x, p.y});
    }
    const Lse r = wave_lse(st);
    const T* rp = logits + row * (int64_t)vocab;
    loss = row_loss(r, rp, target[row], vocab);
    if (!reduce_mean && lane == 0) out[row] = loss;
  }
  if (reduce_mean) {
    __shared__ float wl[kWaves];
    if (lane == 0) wl[wave] = loss;
    __syncthreads();
    float bsum = 0.0f;
    if (threadIdx.x == 0)
      for (int w = 0; w < kWaves; ++w) bsum += wl[w];
    finish_mean(bsum, partials, ticket, out, tokens);
  }
}

// ------------------------------------------------------------ small utilities
__global__ void fill_f32_kernel(float* p, int64_t n, float v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void zero_u32_kernel(unsigned* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// ------------------------------------------------------------ launchers
template <typename T, int U, int WAVES>
static hipError_t launch_wave_rows_w(const XentArgs& a, hipStream_t st) {
  const int64_t blocks = (a.tokens + WAVES - 1) / WAVES;
  hipLaunchKernelGGL((xent_wave_rows_kernel<T, U, WAVES>), dim3((unsigned)blocks), dim3(64 * WAVES),
                     0, st, (const T*)a.logits, a.tokens, (int)a.vocab, a.target, a.out,
                     a.mean_partials, a.ticket, a.reduce_mean);
  return hipGetLastError();
}

// Instantiated shapes: U in {4, 8, 16} with 4 waves; U in {4, 8} with 16 waves
// (16 waves with U = 16 would need more registers than 1024 threads can have).
template <typename T, int U>
static hipError_t launch_wave_rows(const XentArgs& a, hipStream_t st) {
  if (a.waves_per_block == 16) return launch_wave_rows_w<T, (U > 8 ? 8 : U), 16>(a, st);
  return launch_wave_rows_w<T, U, 4>(a, st);
}

template <typename T, int U>
static hipError_t launch_block_rows(const XentArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((xent_block_rows_kernel<T, U>), dim3((unsigned)a.tokens), dim3(kRowThreads), 0,
                     st, (const T*)a.logits, a.tokens, (int)a.vocab, a.target, a.out,
                     a.mean_partials, a.ticket, a.reduce_mean);
  return hipGetLastError();
}

template <typename T, int U>
static hipError_t launch_split(const XentArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((xent_split_partial_kernel<T, U>), dim3((unsigned)a.splits, (unsigned)a.tokens),
                     dim3(kRowThreads), 0, st, (const T*)a.logits, (int)a.vocab,
                     a.chunks_per_split, (float2*)a.split_partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t blocks = (a.tokens + kRowThreads / 64 - 1) / (kRowThreads / 64);
  hipLaunchKernelGGL((xent_split_merge_kernel<T>), dim3((unsigned)blocks), dim3(kRowThreads), 0, st,
                     (const T*)a.logits, a.tokens, (int)a.vocab, a.splits,
                     (const float2*)a.split_partials, a.target, a.out, a.mean_partials, a.ticket,
                     a.reduce_mean);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_xent_t(const XentArgs& a, hipStream_t st) {
  switch (a.path) {
    case XentPath::WaveRows:
      switch (a.unroll) {
        case 4: return launch_wave_rows<T, 4>(a, st);
        case 8: return launch_wave_rows<T, 8>(a, st);
        default: return launch_wave_rows<T, 16>(a, st);
      }
    case XentPath::BlockRows:
      return launch_block_rows<T, 8>(a, st);
    case XentPath::Split:
      return launch_split<T, 8>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_xent(const XentArgs& a, hipStream_t st) {
  return a.bf16 ? launch_xent_t<uint16_t>(a, st) : launch_xent_t<float>(a, st);
}

hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

hipError_t launch_zero_u32(unsigned* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace lce
