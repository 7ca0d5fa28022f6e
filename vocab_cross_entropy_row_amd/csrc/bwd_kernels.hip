// Gradient of the row cross-entropy with respect to the logits, for gfx950.
//
// For row i with target t_i and loss-output gradient g_i (grad[i] for
// per-token losses, grad[0] / tokens for their mean):
//
//     dlogits_ij = g_i * (e^(z_ij - lse_i) - [j == t_i])
//
// The pages give the forward only; this is its derivative (softmax minus the
// one-hot target).  A row whose target is outside [0, vocab) has a NaN loss
// and gets a NaN gradient row.
//
// The softmax is taken against the row state the forward builds: with
// M = fp32(m*log2e) and s = sum_j 2^(z_j*log2e - M),
//     e^(z_j - lse) = 2^(fma(z_j, log2e, -M)) / s,
// so each element costs one decode, one FMA, one exponential and one multiply
// by the row constant g / s, and the target element subtracts g.
//
// Three layouts:
//   xent_bwd_group_kernel  rows of at most 2 KiB without unaligned edges: 2, 4
//                          or 8 rows per wave, each row in a group of lanes'
//                          registers;
//   xent_bwd_wave_kernel   rows of at most 64 * NCH 16-byte chunks: one wave
//                          per row holds the whole row in registers, so the
//                          logits are read once and the gradient written once;
//   xent_bwd_apply_kernel  longer rows: the row states come from the forward
//                          kernels' statistics mode (a first read), then S
//                          workgroups per row read the row again and write
//                          its gradient.
// dlogits may be the logits buffer itself (so neither pointer is restrict):
// every element is read before the same thread writes it.
//
// With a loss output (the forward and the backward in one call), the group and
// wave kernels also finish each row's loss from the state they built, with the
// target logit read out of the row's registers: per-token losses, or their
// deterministic mean (finish_mean).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lce_device.h"
#include "lce_internal.h"
#include "row_stream.h"

namespace lce {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Gradient values of one chunk -> the chunk's storage format (bf16: round to
// nearest even, v_cvt_pk_bf16_f32).
template <typename T>
struct Out;
template <>
struct Out<float> {
  template <int E>
  __device__ __forceinline__ static f32x4 pack(const float (&d)[E]) {
    return f32x4{d[0], d[1], d[2], d[3]};
  }
  __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
};
template <>
struct Out<uint16_t> {
  template <int E>
  __device__ __forceinline__ static u32x4 pack(const float (&d)[E]) {
    u32x4 r;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      r[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{d[2 * w], d[2 * w + 1]}), bf16x2));
    return r;
  }
  __device__ __forceinline__ static void store(uint16_t* p, float v) {
    *p = __builtin_bit_cast(uint16_t, (__bf16)v);
  }
};

// Row constants of the gradient: M = fp32(m*log2e) and c = g / s for the
// row state (m, s), or NaN when the row's target is invalid.
struct GradRow {
  float M, c, g;
};

__device__ __forceinline__ GradRow grad_row(const Lse& r, float g, bool valid) {
  if (!valid) g = __builtin_nanf("");
  return {r.m * kLog2e, g / r.s, g};
}

// Gradient of one chunk of logits.  `tsel` is the element index of the target
// in this chunk, or -1.
template <typename T>
__device__ __forceinline__ typename Vec<T>::raw grad_chunk(const typename Vec<T>::raw& v,
                                                           const GradRow& gr, int tsel) {
  constexpr int E = Vec<T>::kElems;
  float d[E];
#pragma unroll
  for (int e = 0; e < E; ++e)
    d[e] = exp2_fast(__builtin_fmaf(Vec<T>::get_again(v, e), kLog2e, -gr.M)) * gr.c;
  if (tsel >= 0) {
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (e == tsel) d[e] -= gr.g;
  }
  return Out<T>::template pack<E>(d);
}

template <typename T>
__device__ __forceinline__ void store_chunk(__amdgpu_buffer_rsrc_t rs, int c,
                                           const typename Vec<T>::raw& v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, c * 16, 0, 0);
}

__device__ __forceinline__ float row_grad_scale(const float* grad, int64_t row, int64_t tokens,
                                                int reduce_mean) {
  return reduce_mean ? grad[0] / (float)tokens : grad[row];
}

// Element `te` of chunk `k` in lane `ln` of a row held in registers (all three
// wave-uniform): one 32-bit word selected, read with one readlane, decoded.
template <typename T, int NCH>
__device__ __forceinline__ float row_element(const typename Vec<T>::raw (&v)[NCH], int k, int ln,
                                             int te) {
  constexpr int EW = Vec<T>::kElems / 4;  // elements per 32-bit word
  const int wi = te / EW;
  uint32_t w = 0;
#pragma unroll
  for (int kk = 0; kk < NCH; ++kk) {
    const u32x4 q = __builtin_bit_cast(u32x4, v[kk]);
    if (kk == k) w = wi == 0 ? q[0] : wi == 1 ? q[1] : wi == 2 ? q[2] : q[3];
  }
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)w, ln);
  if constexpr (EW == 1) return __uint_as_float(b);
  return __uint_as_float((te & 1) ? (b & 0xffff0000u) : (b << 16));
}

// ------------------------------------------------------------ one wave per row, row in registers
// Lane l holds chunks l + 64k (k < NCH) of the aligned body; loads past the
// body read nothing and stores past it are dropped (buffer resources).
// LOSS: also the row's loss into loss_out (per token, or their mean with
// reduce_mean; `slots` and `epoch` are then the mean state).
template <typename T, int NCH, int WAVES, bool LOSS>
__global__ __launch_bounds__(64 * WAVES) void xent_bwd_wave_kernel(
    const T* logits, int64_t tokens, int vocab, const int64_t* __restrict__ target,
    const float* __restrict__ grad, int reduce_mean, T* dlogits, float* __restrict__ loss_out,
    uint64_t* __restrict__ slots, unsigned* __restrict__ epoch) {
  typedef typename Vec<T>::raw raw;
  constexpr int E = Vec<T>::kElems;
  const unsigned mean_tag = LOSS ? mean_begin(epoch, reduce_mean) : 0u;
  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int64_t row = (int64_t)blockIdx.x * WAVES + wave;
  float loss = 0.0f;
  if (row < tokens) {
    const T* rp = logits + row * (int64_t)vocab;
    T* dp = dlogits + row * (int64_t)vocab;
    const int64_t t = target[row];
    const float g = row_grad_scale(grad, row, tokens, reduce_mean);
    const RowSplit rs = row_split(rp, vocab);
    const int n = wave_uniform(rs.nvec);
    const __amdgpu_buffer_rsrc_t src = make_rsrc(rp + rs.head, (uint32_t)n * 16u);
    const __amdgpu_buffer_rsrc_t dst = make_rsrc(dp + rs.head, (uint32_t)n * 16u);

    // Head and tail elements first, and only when the row has any (a load
    // issued behind the row's chunks would return behind them all).
    const int ei = edge_index(rs, vocab, lane);
    float edge = 0.0f;
    if (wave_uniform(rs.head + rs.tail) > 0) edge = Vec<T>::scalar(rp + ei);
    __builtin_amdgcn_sched_barrier(0);
    raw v[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k)
      v[k] = (raw)__builtin_amdgcn_raw_buffer_load_b128(src, (lane + 64 * k) * 16, 0, kStreamPolicy);
    const bool has_edge = lane < rs.head + rs.tail;

    // Row state.  Chunks past the body become -inf: they fold as nothing, and
    // their (zero) gradient is never stored.
#pragma unroll
    for (int k = 0; k < NCH; ++k)
      if (lane + 64 * k >= n) v[k] = Vec<T>::neg_inf();
    Lse st = lse_empty();
    fold_batch<T, NCH, true>(st, v);
    if (has_edge) fold_one(st, edge);
    const Lse r = wave_lse(st);
    const bool valid = t >= 0 && t < (int64_t)vocab;
    const GradRow gr = grad_row(r, g, valid);

    // Target position: aligned-body chunk and element, or an edge element.
    const int64_t tb = valid ? t - rs.head : -1;
    const int tc = (tb >= 0 && tb < (int64_t)n * E) ? (int)(tb / E) : -1;
    const int te = (tc >= 0) ? (int)(tb % E) : -1;
    if constexpr (LOSS) {
      // The target logit: from its chunk's lane, or from the edge lane that
      // holds it (head element t is lane t, tail element t lane head + t -
      // (vocab - tail)).
      float zt = 0.0f;
      if (tc >= 0) {
        zt = row_element<T, NCH>(v, tc >> 6, tc & 63, te);
      } else if (valid) {
        const int el = t < rs.head ? (int)t : rs.head + (int)(t - (vocab - rs.tail));
        zt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(edge), el));
      }
      loss = valid ? lse_minus(r, zt) : __builtin_nanf("");
    }
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int c = lane + 64 * k;
      store_chunk<T>(dst, c, grad_chunk<T>(v[k], gr, c == tc ? te : -1));
    }
    if (has_edge) {
      float d = exp2_fast(__builtin_fmaf(edge, kLog2e, -gr.M)) * gr.c;
      if ((int64_t)ei == t) d -= gr.g;
      Out<T>::store(dp + ei, d);
    }
  }
  if constexpr (LOSS) {
    if (!reduce_mean) {
      if (row < tokens && lane == 0) loss_out[row] = loss;
    } else {
      __shared__ float wl[WAVES];
      if (lane == 0) wl[wave] = loss;
      __syncthreads();
      float bsum = 0.0f;
      if (threadIdx.x == 0)
        for (int w = 0; w < WAVES; ++w) bsum += wl[w];
      finish_mean(bsum, slots, epoch, mean_tag, loss_out, tokens);
    }
  }
}

// ------------------------------------------------------------ several short rows per wave
// Rows of at most 4 * N chunks with no scalar edges (as the forward's
// several-rows-per-wave kernel): G rows per wave, N = 64 / G lanes per row, lane
// j of a row's group holding chunks j + N * u (u < U) of the row, all in
// registers; one buffer resource covers the wave's G consecutive rows for the
// loads and one for the stores (chunks past a row's end are loaded and stored
// past the resource: no memory is touched).  The row state is merged over the
// group's lanes (group_lse).  With LOSS the group also finishes the row's loss
// (the target logit taken by the lane that holds it and spread over the group
// with a max), per token or into the deterministic mean.
template <typename T, int G, int U, int WAVES, bool LOSS>
__global__ __launch_bounds__(64 * WAVES) void xent_bwd_group_kernel(
    const T* logits, int64_t tokens, int vocab, const int64_t* __restrict__ target,
    const float* __restrict__ grad, int reduce_mean, T* dlogits, float* __restrict__ loss_out,
    uint64_t* __restrict__ slots, unsigned* __restrict__ epoch) {
  typedef typename Vec<T>::raw raw;
  constexpr int E = Vec<T>::kElems;
  constexpr int N = 64 / G;
  const unsigned mean_tag = LOSS ? mean_begin(epoch, reduce_mean) : 0u;
  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int g = lane / N, j = lane % N;
  const int64_t r0 = ((int64_t)blockIdx.x * WAVES + wave) * G;
  const int64_t row = r0 + g;
  const bool have = row < tokens;
  float loss = 0.0f;
  if (r0 < tokens) {
    const int64_t left = tokens - r0;
    const uint32_t rows_here = (uint32_t)(left < G ? left : G);
    const uint32_t row_bytes = (uint32_t)vocab * (uint32_t)sizeof(T);
    const int nvec = (int)(row_bytes / 16u);
    const int64_t t = have ? target[row] : -1;
    const float gs = have ? row_grad_scale(grad, row, tokens, reduce_mean) : 0.0f;
    __builtin_amdgcn_sched_barrier(0);
    const __amdgpu_buffer_rsrc_t src = make_rsrc(logits + r0 * (int64_t)vocab, rows_here * row_bytes);
    const __amdgpu_buffer_rsrc_t dst = make_rsrc(dlogits + r0 * (int64_t)vocab, rows_here * row_bytes);
    uint32_t off[U];
    raw v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = j + N * u;
      off[u] = c < nvec ? (uint32_t)g * row_bytes + (uint32_t)c * 16u : 0x7ffffff0u;
      v[u] = (raw)__builtin_amdgcn_raw_buffer_load_b128(src, off[u], 0, kStreamPolicy);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (j + N * u >= nvec) v[u] = Vec<T>::neg_inf();
    Lse st = lse_empty();
    fold_batch<T, U, true>(st, v);
    const Lse r = group_lse<N>(st);
    const bool valid = t >= 0 && t < (int64_t)vocab;
    const GradRow gr = grad_row(r, gs, valid);
    // The target's chunk and element within the row (all lanes of the group agree).
    const int tc = valid ? (int)(t / E) : -1;
    const int te = valid ? (int)(t % E) : -1;
    if constexpr (LOSS) {
      float zt = kNegInf;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (tc == j + N * u) {
#pragma unroll
          for (int e = 0; e < E; ++e)
            if (e == te) zt = Vec<T>::get(v[u], e);
        }
      zt = group_allreduce<N>(zt, MaxOp{});
      loss = valid ? lse_minus(r, zt) : __builtin_nanf("");
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = j + N * u;
      const raw d = grad_chunk<T>(v[u], gr, c == tc ? te : -1);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, d), dst, off[u], 0, 0);
    }
  }
  if constexpr (LOSS) {
    if (!reduce_mean) {
      if (have && j == 0) loss_out[row] = loss;
    } else {
      __shared__ float wl[WAVES * G];
      if (j == 0) wl[wave * G + g] = have ? loss : 0.0f;
      __syncthreads();
      float bsum = 0.0f;
      if (threadIdx.x == 0)
        for (int i = 0; i < WAVES * G; ++i) bsum += wl[i];
      finish_mean(bsum, slots, epoch, mean_tag, loss_out, tokens);
    }
  }
}

// ------------------------------------------------------------ long rows: apply from row states
// grid = S * tokens workgroups; workgroup b rewrites chunk slice s = b % S of
// row b / S, and slice 0 also the row's scalar edges.  stats[3*row ..] = (m, sum e^(z - m), .) from
// the forward kernels' statistics mode.
template <typename T, int U>
__global__ __launch_bounds__(kRowThreads) void xent_bwd_apply_kernel(
    const T* logits, int64_t tokens, int vocab, const int64_t* __restrict__ target,
    const float* __restrict__ grad, int reduce_mean, const float* __restrict__ stats, int slices,
    int chunks_per_slice, T* dlogits) {
  typedef typename Vec<T>::raw raw;
  constexpr int E = Vec<T>::kElems;
  const int s = (int)(blockIdx.x % (unsigned)slices);
  const int64_t row = blockIdx.x / (unsigned)slices;
  const T* rp = logits + row * (int64_t)vocab;
  T* dp = dlogits + row * (int64_t)vocab;
  const int64_t t = target[row];
  const bool valid = t >= 0 && t < (int64_t)vocab;
  float g = row_grad_scale(grad, row, tokens, reduce_mean);
  if (!valid) g = __builtin_nanf("");
  // e^(z - m) / s_nat = 2^(fma(z, L, -M)) * 2^(M - m*L) / s_nat
  const float m = stats[3 * row], s_nat = stats[3 * row + 1];
  const float M = m * kLog2e;
  const GradRow gr{M, g * exp2_fast(-__builtin_fmaf(m, kLog2e, -M)) / s_nat, g};

  const RowSplit rsplit = row_split(rp, vocab);
  const int c0 = s * chunks_per_slice;
  int c1 = c0 + chunks_per_slice;
  c1 = c1 < rsplit.nvec ? c1 : rsplit.nvec;
  const int n = c1 - c0;
  if (s == 0 && (int)threadIdx.x < rsplit.head + rsplit.tail) {
    const int ei = edge_index(rsplit, vocab, threadIdx.x);
    float d = exp2_fast(__builtin_fmaf(Vec<T>::scalar(rp + ei), kLog2e, -gr.M)) * gr.c;
    if ((int64_t)ei == t) d -= gr.g;
    Out<T>::store(dp + ei, d);
  }
  if (n <= 0) return;
  const __amdgpu_buffer_rsrc_t src = make_rsrc(rp + rsplit.head + (int64_t)c0 * E, (uint32_t)n * 16u);
  const __amdgpu_buffer_rsrc_t dst = make_rsrc(dp + rsplit.head + (int64_t)c0 * E, (uint32_t)n * 16u);
  const int64_t tb = valid ? t - rsplit.head - (int64_t)c0 * E : -1;
  const int tc = (tb >= 0 && tb < (int64_t)n * E) ? (int)(tb / E) : -1;
  const int te = (tc >= 0) ? (int)(tb % E) : -1;
  // Batches of U chunks per thread, loads of the next batch in flight while the
  // current one is rewritten (stores past the slice are dropped).
  const int S = kRowThreads * U;
  raw a[U];
#pragma unroll
  for (int u = 0; u < U; ++u)
    a[u] = (raw)__builtin_amdgcn_raw_buffer_load_b128(src, ((int)threadIdx.x + u * kRowThreads) * 16, 0,
                                                      kStreamPolicy);
  for (int base = threadIdx.x; base < n; base += S) {
    raw b[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      b[u] = (raw)__builtin_amdgcn_raw_buffer_load_b128(src, (base + S + u * kRowThreads) * 16, 0,
                                                        kStreamPolicy);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = base + u * kRowThreads;
      store_chunk<T>(dst, c, grad_chunk<T>(a[u], gr, c == tc ? te : -1));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = b[u];
  }
}

// ------------------------------------------------------------ launchers
template <typename T, int NCH, int W, bool LOSS>
hipError_t launch_bwd_wave_w(const BwdArgs& a, hipStream_t st) {
  const int64_t blocks = (a.tokens + W - 1) / W;
  if (!grid_fits(blocks, 64 * W)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((xent_bwd_wave_kernel<T, NCH, W, LOSS>), dim3((unsigned)blocks), dim3(64 * W), 0, st,
                     (const T*)a.logits, a.tokens, (int)a.vocab, a.target, a.grad, a.reduce_mean,
                     (T*)a.dlogits, a.loss_out, a.mean_slots, a.epoch);
  return hipGetLastError();
}

// Rows per workgroup: 4, and for a mean of the losses 16 (a quarter of the
// workgroups hand a partial to the mean's finisher), or 8 for rows of 32 chunks
// per lane (about 176 VGPRs: a 1024-thread workgroup would allow 128).
int bwd_wave_rows(const BwdArgs& a) {
  if (!(a.loss_out && a.reduce_mean)) return 4;
  return a.wave_chunks >= 32 ? 8 : 16;
}

template <typename T, int NCH>
hipError_t launch_bwd_wave_t(const BwdArgs& a, hipStream_t st) {
  if (!a.loss_out) return launch_bwd_wave_w<T, NCH, 4, false>(a, st);
  if (!a.reduce_mean) return launch_bwd_wave_w<T, NCH, 4, true>(a, st);
  if constexpr (NCH >= 32)
    return launch_bwd_wave_w<T, NCH, 8, true>(a, st);
  else
    return launch_bwd_wave_w<T, NCH, 16, true>(a, st);
}

template <typename T, int G>
hipError_t launch_bwd_group_t(const BwdArgs& a, hipStream_t st) {
  constexpr int W = 4;
  const int64_t blocks = (a.tokens + W * G - 1) / (W * G);
  if (!grid_fits(blocks, 64 * W)) return hipErrorInvalidConfiguration;
  if (a.loss_out)
    hipLaunchKernelGGL((xent_bwd_group_kernel<T, G, 4, W, true>), dim3((unsigned)blocks), dim3(64 * W), 0, st,
                       (const T*)a.logits, a.tokens, (int)a.vocab, a.target, a.grad, a.reduce_mean,
                       (T*)a.dlogits, a.loss_out, a.mean_slots, a.epoch);
  else
    hipLaunchKernelGGL((xent_bwd_group_kernel<T, G, 4, W, false>), dim3((unsigned)blocks), dim3(64 * W), 0, st,
                       (const T*)a.logits, a.tokens, (int)a.vocab, a.target, a.grad, a.reduce_mean,
                       (T*)a.dlogits, nullptr, nullptr, nullptr);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t st) {
  switch (a.rows_per_wave) {
    case 2: return launch_bwd_group_t<T, 2>(a, st);
    case 4: return launch_bwd_group_t<T, 4>(a, st);
    case 8: return launch_bwd_group_t<T, 8>(a, st);
    default: break;
  }
  if (a.wave_chunks > 0) {
    switch (a.wave_chunks) {
      case 1: return launch_bwd_wave_t<T, 1>(a, st);
      case 2: return launch_bwd_wave_t<T, 2>(a, st);
      case 4: return launch_bwd_wave_t<T, 4>(a, st);
      case 8: return launch_bwd_wave_t<T, 8>(a, st);
      case 16: return launch_bwd_wave_t<T, 16>(a, st);
      case 32: return launch_bwd_wave_t<T, 32>(a, st);
      default: return hipErrorInvalidValue;
    }
  }
  if (!grid_fits((int64_t)a.splits * a.tokens, kRowThreads)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((xent_bwd_apply_kernel<T, 4>), dim3((unsigned)(a.splits * a.tokens)),
                     dim3(kRowThreads), 0, st, (const T*)a.logits, a.tokens, (int)a.vocab, a.target,
                     a.grad, a.reduce_mean, a.stats, a.splits, a.chunks_per_split, (T*)a.dlogits);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t st) {
  return a.bf16 ? launch_bwd_t<uint16_t>(a, st) : launch_bwd_t<float>(a, st);
}

}  // namespace lce
