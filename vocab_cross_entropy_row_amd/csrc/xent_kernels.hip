// Row cross-entropy kernels for gfx950.
//
// Computes, for every token row of a [tokens, vocab] logit matrix (fp32 or
// bf16), loss = ln(sum_j e^z_j) - z_target, and optionally their mean
// (KernelIndex "Cross-entropy loss" and "Vocab-parallel cross-entropy,
// Megatron layout": descriptions and Semantics blocks).
//
// The work is one pass over HBM: every logit is read once with 16-byte loads
// (4 fp32 or 8 bf16 per lane per load), consecutive lanes read consecutive
// 16-byte chunks, and each lane folds what it loaded into a (max, sum-exp)
// state in fp32 (see lce_device.h).  For losses the sum is taken against a
// fixed per-lane reference (the maximum of the lane's first chunk) with no
// per-element maximum; a row whose lane sums are not safely bounded is folded
// again with a tracked maximum (row_stream.h).  Loads are buffer loads
// issued in batches of U chunks per lane, double-buffered, so each wave keeps
// up to 2 * U KiB in flight; the row's scalar loads (target logit, unaligned
// edges) are issued right behind the first batch.
//
// Four layouts of work over rows:
//   group_rows  2, 4 or 8 rows per wavefront, a group of lanes per row (rows
//               of at most 2 KiB without unaligned edges);
//   wave_rows   one wavefront per row, 4 or 16 rows per workgroup (rows of at
//               most 32 KiB);
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
#include "row_stream.h"

namespace lce {

static_assert(kMeanHeaderBytes >= (kEpochWord + 1) * sizeof(unsigned),
              "host mean-state layout must hold the device's epoch word");

// ------------------------------------------------------------ one wave per row
// WAVES rows (one per wave) per workgroup.  With a mean, larger workgroups
// mean fewer partials to hand off.
template <typename T, int U, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void xent_wave_rows_kernel(
    const T* __restrict__ logits, int64_t tokens, int vocab, const int64_t* __restrict__ target,
    int64_t vocab_start, float* __restrict__ stats, float* __restrict__ out,
    uint64_t* __restrict__ slots, unsigned* __restrict__ epoch, int reduce_mean) {
  const unsigned mean_tag = mean_begin(epoch, reduce_mean);
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
    float edge = 0.0f, zt = 0.0f;
    int64_t tt = -1;
    // Head and tail elements (rows not 16-byte aligned) are loaded first, and
    // only when the row has any: a load issued behind the logits would return
    // behind them all (measured: 0.36 us of the 8 KiB-row headline shape).
    // Issued before any other load, it leaves every later wait count exact.
    if (wave_uniform(rs.head + rs.tail) > 0) edge = Vec<T>::scalar(rp + edge_index(rs, vocab, lane));
    __builtin_amdgcn_sched_barrier(0);
    auto extra = [&]() {
      tt = local_target(target_here(t), vocab_start, vocab);
      zt = Vec<T>::scalar(rp + safe_target(tt, vocab));
    };
    Lse st = lse_empty();
    // Rows of at most kMaxB batches take the unrolled loop: 32 chunks per lane
    // for batches of 4 or more, two batches for batches of 1 or 2.
    constexpr int kMaxB = U >= 4 ? 32 / U : 2;
    auto stream = [&](auto track, auto&& ex) {
      constexpr bool kTrack = decltype(track)::value;
      if (wave_uniform(rs.nvec) <= 64 * U * kMaxB)
        stream_chunks_short<T, U, kMaxB, kTrack>(st, body, 0, rs.nvec, lane, 64, ex);
      else
        stream_chunks<T, U, kTrack>(st, body, 0, rs.nvec, lane, 64, ex);
    };
    // Shard statistics report the exact maximum, so they take the tracked
    // fold.  Losses take the fixed-reference fold, and the whole row again
    // through the tracked one if any lane's sum is not safely bounded.
    if (stats) {
      stream(TrackMax<true>{}, extra);
    } else {
      stream(TrackMax<false>{}, extra);
      if (__builtin_amdgcn_ballot_w64(lane_sum_unsafe(st))) {
        st = lse_empty();
        stream(TrackMax<true>{}, [] {});
      }
    }
    if (lane < rs.head + rs.tail) fold_one(st, edge);
    const Lse r = wave_lse(st);
    if (stats) {
      if (lane == 0) write_stats(stats + 3 * row, r, tt >= 0, zt);
    } else {
      loss = (tt >= 0) ? lse_minus(r, zt) : __builtin_nanf("");
      if (!reduce_mean && lane == 0) out[row] = loss;
    }
  }
  if (reduce_mean) {
    __shared__ float wl[WAVES];
    if (lane == 0) wl[wave] = loss;
    __syncthreads();
    float bsum = 0.0f;
    if (threadIdx.x == 0)
      for (int w = 0; w < WAVES; ++w) bsum += wl[w];
    finish_mean(bsum, slots, epoch, mean_tag, out, tokens);
  }
}

// ------------------------------------------------------------ several rows per wave
// Short rows (at most 4 * N 16-byte chunks, the rows' bytes a multiple of 16
// and the logits 16-byte aligned, so a row has no scalar edges): G rows per
// wave and N = 64 / G lanes per row, lane j of a row's group holding chunks
// j + N * u (u < U).  A wave's G rows are consecutive in memory, so one buffer
// resource covers them; a chunk past its row's end is loaded at an offset past
// the resource (no memory is read) and folds as -inf.  The group's lanes then
// merge their states (group_lse) and its first lane finishes the row.  Per row
// this is one group of lanes' worth of fixed work (target, reduction, store)
// instead of one wave's, and the target logit comes out of the registers.
template <typename T, int G, int U, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void xent_group_rows_kernel(
    const T* __restrict__ logits, int64_t tokens, int vocab, const int64_t* __restrict__ target,
    int64_t vocab_start, float* __restrict__ stats, float* __restrict__ out,
    uint64_t* __restrict__ slots, unsigned* __restrict__ epoch, int reduce_mean) {
  constexpr int N = 64 / G;
  typedef typename Vec<T>::raw raw;
  const unsigned mean_tag = mean_begin(epoch, reduce_mean);
  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int g = lane / N, j = lane % N;
  const int64_t r0 = ((int64_t)blockIdx.x * WAVES + wave) * G;  // this wave's first row
  const int64_t row = r0 + g;
  const bool have = row < tokens;
  float loss = 0.0f;
  if (r0 < tokens) {
    const int64_t left = tokens - r0;
    const uint32_t rows_here = (uint32_t)(left < G ? left : G);
    const uint32_t row_bytes = (uint32_t)vocab * (uint32_t)sizeof(T);
    const int nvec = (int)(row_bytes / 16u);
    // The target first: its wait then leaves the chunk loads in flight.
    const int64_t t = have ? target[row] : -1;
    __builtin_amdgcn_sched_barrier(0);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(logits + r0 * (int64_t)vocab, rows_here * row_bytes);
    raw v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = j + N * u;
      const uint32_t off = c < nvec ? (uint32_t)g * row_bytes + (uint32_t)c * 16u : 0x7ffffff0u;
      v[u] = (raw)__builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kStreamPolicy);
    }
    __builtin_amdgcn_sched_barrier(0);
    const int64_t tt = have ? local_target(t, vocab_start, vocab) : -1;
    // The target logit from the registers of the lane that holds it, spread over
    // the group with a max: no load that waits for the target index (bf16
    // [65536, 512] 13.31 -> 12.78 us, fp32 [65536, 256] 12.64 -> 12.01 us).
    constexpr int E = Vec<T>::kElems;
    const int tcg = tt >= 0 ? (int)(tt / E) : -1;
    const int teg = tt >= 0 ? (int)(tt % E) : -1;
    float zr = kNegInf;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (tcg == j + N * u) {
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (e == teg) zr = Vec<T>::get(v[u], e);
      }
    const float zt = group_allreduce<N>(zr, MaxOp{});
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (j + N * u >= nvec) v[u] = Vec<T>::neg_inf();
    // Shard statistics take the tracked fold (exact maximum); losses the
    // fixed-reference fold, and the tracked one if any lane's sum is not bounded.
    Lse st = lse_empty();
    if (stats) {
      fold_batch<T, U, true, true>(st, v);
    } else {
      fold_batch<T, U, true, false>(st, v);
      if (__builtin_amdgcn_ballot_w64(lane_sum_unsafe(st))) {
        st = lse_empty();
        fold_batch<T, U, true, true>(st, v);
      }
    }
    const Lse r = group_lse<N>(st);
    if (stats) {
      if (j == 0 && have) write_stats(stats + 3 * row, r, tt >= 0, zt);
    } else {
      loss = (tt >= 0) ? lse_minus(r, zt) : __builtin_nanf("");
      if (!reduce_mean && j == 0 && have) out[row] = loss;
    }
  }
  if (reduce_mean) {
    // The workgroup's rows in order (rows past the end add 0).
    __shared__ float wl[WAVES * G];
    if (j == 0) wl[wave * G + g] = have ? loss : 0.0f;
    __syncthreads();
    float bsum = 0.0f;
    if (threadIdx.x == 0)
      for (int i = 0; i < WAVES * G; ++i) bsum += wl[i];
    finish_mean(bsum, slots, epoch, mean_tag, out, tokens);
  }
}

// ------------------------------------------------------------ one workgroup per row
template <typename T, int U>
__global__ __launch_bounds__(kRowThreads) void xent_block_rows_kernel(
    const T* __restrict__ logits, int64_t tokens, int vocab, const int64_t* __restrict__ target,
    int64_t vocab_start, float* __restrict__ stats, float* __restrict__ out,
    uint64_t* __restrict__ slots, unsigned* __restrict__ epoch, int reduce_mean) {
  const unsigned mean_tag = mean_begin(epoch, reduce_mean);
  const int64_t row = blockIdx.x;
  const T* rp = logits + row * (int64_t)vocab;
  const int64_t t = target[row];
  const RowSplit rs = row_split(rp, vocab);
  const typename Vec<T>::raw* body = reinterpret_cast<const typename Vec<T>::raw*>(rp + rs.head);
  float edge = 0.0f, zt = 0.0f;
  int64_t tt = -1;
  auto extra = [&]() {
    edge = Vec<T>::scalar(rp + edge_index(rs, vocab, threadIdx.x));
    tt = local_target(target_here(t), vocab_start, vocab);
    zt = Vec<T>::scalar(rp + safe_target(tt, vocab));
  };
  Lse st = lse_empty();
  // As in the wave kernel: fixed-reference fold for losses, the tracked fold
  // for shard statistics and for rows where any lane's sum is not bounded.
  if (stats) {
    stream_chunks<T, U, true>(st, body, 0, rs.nvec, threadIdx.x, kRowThreads, extra);
  } else {
    stream_chunks<T, U, false>(st, body, 0, rs.nvec, threadIdx.x, kRowThreads, extra);
    if (__syncthreads_or(lane_sum_unsafe(st))) {
      st = lse_empty();
      stream_chunks<T, U, true>(st, body, 0, rs.nvec, threadIdx.x, kRowThreads, [] {});
    }
  }
  if ((int)threadIdx.x < rs.head + rs.tail) fold_one(st, edge);
  const Lse r = block_lse(st);
  if (stats) {
    if (threadIdx.x == 0) write_stats(stats + 3 * row, r, tt >= 0, zt);
    return;
  }
  const float loss = (tt >= 0) ? lse_minus(r, zt) : __builtin_nanf("");
  if (!reduce_mean) {
    if (threadIdx.x == 0) out[row] = loss;
  } else {
    finish_mean(loss, slots, epoch, mean_tag, out, tokens);
  }
}

// ------------------------------------------------------------ split rows
// grid = (S, tokens).  Workgroup (s, row) streams chunk slice s of the row and
// writes its state to part[s * tokens + row]; slice 0 also folds the scalar
// edges, and loads the target logit right behind its first batch (its latency
// hides under the stream) and writes it to zt[row], NaN when these columns do
// not hold the target.  The merge then needs no dependent load.
template <typename T, int U>
__global__ __launch_bounds__(kRowThreads) void xent_split_partial_kernel(
    const T* __restrict__ logits, int vocab, int chunks_per_slice, const int64_t* __restrict__ target,
    int64_t vocab_start, float2* __restrict__ part, float* __restrict__ zt_out, int exact) {
  const int s = blockIdx.x;
  const int64_t tokens = gridDim.y;
  const int64_t row = blockIdx.y;
  const T* rp = logits + row * (int64_t)vocab;
  const int64_t t = (s == 0) ? target[row] : -1;
  const RowSplit rs = row_split(rp, vocab);
  const typename Vec<T>::raw* body = reinterpret_cast<const typename Vec<T>::raw*>(rp + rs.head);
  float edge = 0.0f, zt = 0.0f;
  int64_t tt = -1;
  auto extra = [&]() {
    edge = Vec<T>::scalar(rp + edge_index(rs, vocab, threadIdx.x));
    if (s == 0) {
      tt = local_target(target_here(t), vocab_start, vocab);
      zt = Vec<T>::scalar(rp + safe_target(tt, vocab));
    }
  };
  Lse st = lse_empty();
  const int c0 = s * chunks_per_slice;
  int c1 = c0 + chunks_per_slice;
  c1 = c1 < rs.nvec ? c1 : rs.nvec;
  // Shard statistics (exact) report the exact maximum and take the tracked
  // fold; losses take the fixed-reference fold, and the slice again through the
  // tracked one if any thread's sum is not bounded.  Slices of up to kMaxB
  // batches per thread take the unrolled stream.
  constexpr int kMaxB = U >= 4 ? 32 / U : 2;
  const bool fits = (c1 - c0) <= kRowThreads * U * kMaxB;
  if (exact) {
    if (fits)
      stream_chunks_short<T, U, kMaxB, true>(st, body, c0, c1, threadIdx.x, kRowThreads, extra);
    else
      stream_chunks<T, U, true>(st, body, c0, c1, threadIdx.x, kRowThreads, extra);
  } else {
    if (fits)
      stream_chunks_short<T, U, kMaxB, false>(st, body, c0, c1, threadIdx.x, kRowThreads, extra);
    else
      stream_chunks<T, U, false>(st, body, c0, c1, threadIdx.x, kRowThreads, extra);
    if (__syncthreads_or(lane_sum_unsafe(st))) {
      st = lse_empty();
      stream_chunks<T, U, true>(st, body, c0, c1, threadIdx.x, kRowThreads, [] {});
    }
  }
  if (s == 0 && (int)threadIdx.x < rs.head + rs.tail) fold_one(st, edge);
  const Lse r = block_lse(st);
  if (threadIdx.x == 0) {
    part[s * tokens + row] = make_float2(r.m, r.s);
    if (s == 0) zt_out[row] = tt >= 0 ? zt : __builtin_nanf("");
  }
}

// One thread per row: merge its S partials in slice order (consecutive
// threads read consecutive rows of a slice; eight slices' loads in flight at
// once, padding entries merging as exact no-ops), then finish the loss (NaN
// for a NaN target logit: the target was invalid or outside these columns),
// the shard statistics, or the mean.  Every load is independent of the
// others, so the merge is one memory round trip before its stores.
__global__ __launch_bounds__(kRowThreads) void xent_split_merge_kernel(
    int64_t tokens, int S, const float2* __restrict__ part, const float* __restrict__ zt_in,
    float* __restrict__ stats, float* __restrict__ out, uint64_t* __restrict__ slots,
    unsigned* __restrict__ epoch, int reduce_mean) {
  const unsigned mean_tag = mean_begin(epoch, reduce_mean);
  const int64_t row = (int64_t)blockIdx.x * kRowThreads + threadIdx.x;
  float loss = 0.0f;
  if (row < tokens) {
    constexpr int kGroup = 8;
    Lse st = lse_empty();
    const float zt = zt_in[row];
    for (int s0 = 0; s0 < S; s0 += kGroup) {
      float2 p[kGroup];
#pragma unroll
      for (int j = 0; j < kGroup; ++j)
        p[j] = (s0 + j < S) ? part[(int64_t)(s0 + j) * tokens + row] : make_float2(kNegInf, 0.0f);
#pragma unroll
      for (int j = 0; j < kGroup; ++j) st = lse_merge(st, Lse{p[j].x, p[j].y});
    }
    if (stats) {
      write_stats(stats + 3 * row, st, true, zt);  // zt is NaN when these columns lack the target
    } else {
      loss = lse_minus(st, zt);
      if (!reduce_mean) out[row] = loss;
    }
  }
  if (reduce_mean) {
    __shared__ float red[kRowThreads];
    red[threadIdx.x] = loss;
    __syncthreads();
#pragma unroll
    for (int w = kRowThreads / 2; w > 0; w >>= 1) {
      if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
      __syncthreads();
    }
    finish_mean(red[0], slots, epoch, mean_tag, out, tokens);
  }
}

// ------------------------------------------------------------ merge of vocab-shard statistics
// One thread per token: fold the `shards` (m, s, zt) triples of its row in
// shard order into (M, S) with S relative to e^M (a shard of -inf only adds
// nothing), take the one target logit a shard reported, and finish the loss
// as (M - zt) + ln S.  Triples are loaded eight shards at a time.
__global__ __launch_bounds__(kRowThreads) void xent_stats_merge_kernel(
    const float* __restrict__ stats, int shards, int64_t tokens, const int64_t* __restrict__ target,
    int64_t vocab, float* __restrict__ out, uint64_t* __restrict__ slots,
    unsigned* __restrict__ epoch, int reduce_mean) {
  const unsigned mean_tag = mean_begin(epoch, reduce_mean);
  const int64_t row = (int64_t)blockIdx.x * kRowThreads + threadIdx.x;
  float loss = 0.0f;
  if (row < tokens) {
    const int64_t t = target[row];
    constexpr int kGroup = 8;
    float M = kNegInf, S = 0.0f, zt = __builtin_nanf("");
    for (int p0 = 0; p0 < shards; p0 += kGroup) {
      float q[kGroup][3];
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        const bool in = p0 + j < shards;
        const float* src = stats + 3 * ((int64_t)(in ? p0 + j : 0) * tokens + row);
        q[j][0] = in ? src[0] : kNegInf;
        q[j][1] = in ? src[1] : 0.0f;
        q[j][2] = in ? src[2] : __builtin_nanf("");
      }
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        const float m = q[j][0], s = q[j][1];
        if (m > M) {  // rescale the sum so far to the new maximum
          S = (M == kNegInf ? 0.0f : S * exp2_fast((M - m) * kLog2e)) + s;
          M = m;
        } else if (m != kNegInf) {  // (a NaN maximum lands here and makes S NaN)
          S += s * exp2_fast((m - M) * kLog2e);
        }
        if (q[j][2] == q[j][2]) zt = q[j][2];
      }
    }
    loss = (t >= 0 && t < vocab) ? (M - zt) + kLn2 * log2_fast(S) : __builtin_nanf("");
    if (!reduce_mean) out[row] = loss;
  }
  if (reduce_mean) {
    __shared__ float red[kRowThreads];
    red[threadIdx.x] = loss;
    __syncthreads();
#pragma unroll
    for (int w = kRowThreads / 2; w > 0; w >>= 1) {
      if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
      __syncthreads();
    }
    finish_mean(red[0], slots, epoch, mean_tag, out, tokens);
  }
}

hipError_t launch_stats_merge(const float* stats, int64_t shards, int64_t tokens,
                              const int64_t* target, int64_t vocab, float* out, int reduce_mean,
                              uint64_t* slots, unsigned* epoch, hipStream_t st) {
  const int64_t blocks = (tokens + kRowThreads - 1) / kRowThreads;
  if (!grid_fits(blocks, kRowThreads)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(xent_stats_merge_kernel, dim3((unsigned)blocks), dim3(kRowThreads), 0, st, stats,
                     (int)shards, tokens, target, vocab, out, slots, epoch, reduce_mean);
  return hipGetLastError();
}

// ------------------------------------------------------------ small utilities
// Grid-stride fills: any n (a zero-filled dweight can exceed 2^32 elements).
__global__ void fill_f32_kernel(float* p, int64_t n, float v) {
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += step) p[i] = v;
}

__global__ void zero_u32_kernel(unsigned* p, int64_t n) {
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += step) p[i] = 0u;
}

static unsigned fill_blocks(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return (unsigned)(b < 65536 ? b : 65536);
}

// ------------------------------------------------------------ launchers
template <typename T, int U, int WAVES>
static hipError_t launch_wave_rows_w(const XentArgs& a, hipStream_t st) {
  const int64_t blocks = (a.tokens + WAVES - 1) / WAVES;
  if (!grid_fits(blocks, 64 * WAVES)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((xent_wave_rows_kernel<T, U, WAVES>), dim3((unsigned)blocks), dim3(64 * WAVES),
                     0, st, (const T*)a.logits, a.tokens, (int)a.vocab, a.target, a.vocab_start,
                     a.stats, a.out, a.mean_slots, a.epoch, a.reduce_mean);
  return hipGetLastError();
}

// Instantiated shapes: U in {1, 2, 4, 8, 16} with 4 waves; U in {1, 2, 4, 8} with
// 16 waves (16 waves with U = 16 would need more registers than 1024 threads can
// have).
template <typename T, int U>
static hipError_t launch_wave_rows(const XentArgs& a, hipStream_t st) {
  if (a.waves_per_block == 16) return launch_wave_rows_w<T, (U > 8 ? 8 : U), 16>(a, st);
  return launch_wave_rows_w<T, U, 4>(a, st);
}

template <typename T, int G>
static hipError_t launch_group_rows(const XentArgs& a, hipStream_t st) {
  constexpr int W = 4;
  const int64_t blocks = (a.tokens + W * G - 1) / (W * G);
  if (!grid_fits(blocks, 64 * W)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((xent_group_rows_kernel<T, G, 4, W>), dim3((unsigned)blocks), dim3(64 * W), 0, st,
                     (const T*)a.logits, a.tokens, (int)a.vocab, a.target, a.vocab_start, a.stats,
                     a.out, a.mean_slots, a.epoch, a.reduce_mean);
  return hipGetLastError();
}

template <typename T, int U>
static hipError_t launch_block_rows(const XentArgs& a, hipStream_t st) {
  if (!grid_fits(a.tokens, kRowThreads)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((xent_block_rows_kernel<T, U>), dim3((unsigned)a.tokens), dim3(kRowThreads), 0,
                     st, (const T*)a.logits, a.tokens, (int)a.vocab, a.target, a.vocab_start,
                     a.stats, a.out, a.mean_slots, a.epoch, a.reduce_mean);
  return hipGetLastError();
}

template <typename T, int U>
static hipError_t launch_split(const XentArgs& a, hipStream_t st) {
  if (a.tokens > 65535 || !grid_fits(a.splits, kRowThreads)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((xent_split_partial_kernel<T, U>), dim3((unsigned)a.splits, (unsigned)a.tokens),
                     dim3(kRowThreads), 0, st, (const T*)a.logits, (int)a.vocab,
                     a.chunks_per_split, a.target, a.vocab_start, (float2*)a.split_partials,
                     a.split_zt, a.stats ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t blocks = (a.tokens + kRowThreads - 1) / kRowThreads;
  hipLaunchKernelGGL(xent_split_merge_kernel, dim3((unsigned)blocks), dim3(kRowThreads), 0, st,
                     a.tokens, a.splits, (const float2*)a.split_partials, (const float*)a.split_zt,
                     a.stats, a.out, a.mean_slots, a.epoch, a.reduce_mean);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_xent_t(const XentArgs& a, hipStream_t st) {
  switch (a.path) {
    case XentPath::WaveRows:
      switch (a.unroll) {
        case 1: return launch_wave_rows<T, 1>(a, st);
        case 2: return launch_wave_rows<T, 2>(a, st);
        case 4: return launch_wave_rows<T, 4>(a, st);
        case 8: return launch_wave_rows<T, 8>(a, st);
        default: return launch_wave_rows<T, 16>(a, st);
      }
    case XentPath::GroupRows:
      switch (a.rows_per_wave) {
        case 2: return launch_group_rows<T, 2>(a, st);
        case 4: return launch_group_rows<T, 4>(a, st);
        case 8: return launch_group_rows<T, 8>(a, st);
        default: return hipErrorInvalidValue;
      }
    case XentPath::BlockRows:
      return launch_block_rows<T, 8>(a, st);
    case XentPath::Split:
      // Batches of 4 chunks for bf16, 8 for fp32 (bf16 [400, 65536] mean 17.9 ->
      // 15.6 us, bf16 [256, 131072] 15.4 -> 14.8 us; fp32 rows 1-3% slower with 4).
      return launch_split<T, sizeof(T) == 2 ? 4 : 8>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_xent(const XentArgs& a, hipStream_t st) {
  return a.bf16 ? launch_xent_t<uint16_t>(a, st) : launch_xent_t<float>(a, st);
}

hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_f32_kernel, dim3(fill_blocks(n)), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

hipError_t launch_zero_u32(unsigned* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_u32_kernel, dim3(fill_blocks(n)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace lce
