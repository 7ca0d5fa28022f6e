// Fused projection + generalized Jensen-Shannon divergence for gfx950.
//
// KernelIndex "Fused linear + JSD" (description and Semantics block): student
// and teacher activations (tokens x hidden) projected through their own
// vocab x hidden heads, then a generalized JSD between the two distributions,
// averaged over tokens ("batchmean"), with the logits never stored.  The page
// names the divergence without printing it; with P = softmax(student logits),
// Q = softmax(teacher logits) and M = beta P + (1 - beta) Q, per token
//
//     JSD = beta KL(P || M) + (1 - beta) KL(Q || M),  KL(A || B) = sum_j A_j ln(A_j / B_j).
//
// Each term needs both distributions normalised, so the work is two passes:
//   1. the log-sum-exp of each head's logits per token: the cross-entropy
//      kernel in its log-sum-exp mode, once per head;
//   2. this kernel: both heads' logit tiles again, side by side, and per
//      element  beta P (lp - ln M) + (1 - beta) Q (lq - ln M)  with
//      lp = z_s - lse_s, lq = z_t - lse_t, summed per token over the vocab.
//      Every such term is >= 0 (log-sum inequality), so the sum does not
//      cancel; the term is evaluated relative to max(lp, lq), so that a
//      probability below the fp32 range gives 0 and never 0 * infinity.
//
// Tile: 128 vocab x 128 tokens per head.  Eight waves (2 along vocab x 4
// along tokens) each own 64 vocab x 32 tokens of both heads (2 x 1 blocks of
// 32 x 32 per head, 64 fp32 accumulators per lane).  Slabs of 64 hidden
// elements of the four operands (W_s, W_t, x_s, x_t; 16 KiB each) go global ->
// LDS directly (buffer_load ... lds, XOR-swizzled rows) in two stages: the
// next slab's DMAs are issued right after the barrier and land while the
// current slab multiplies.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lce_device.h"
#include "lce_internal.h"
#include "mfma_common.h"

namespace lce {

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

namespace {
constexpr int kJV = 128;                  // vocab rows per tile
constexpr int kJT = 128;                  // tokens per tile
constexpr int kJK = 64;                   // hidden elements per slab
constexpr int kJWaves = 8;
constexpr int kJThreads = 64 * kJWaves;
constexpr int kJWV = 2;                   // waves along vocab (64 rows each)
constexpr int kJBVB = 2;                  // 32-row blocks per wave along vocab
constexpr int kJOpElems = 128 * kJK;      // one operand slab (128 rows of 64)
constexpr int kJStageElems = 4 * kJOpElems;
constexpr int kJStages = 2;
constexpr int kJDmas = 128 / 8 / kJWaves; // 1 KiB DMAs per wave per operand per slab
static_assert(kJDmas == 2, "DMA plan");
}  // namespace

__global__ __launch_bounds__(kJThreads) void fused_jsd_partial_kernel(
    const uint16_t* __restrict__ xs, const uint16_t* __restrict__ ws,
    const uint16_t* __restrict__ xt, const uint16_t* __restrict__ wt, int64_t tokens,
    int64_t hidden, int64_t vocab, const float* __restrict__ lse_s,
    const float* __restrict__ lse_t, float beta, int segments, float* __restrict__ part) {
  __shared__ __attribute__((aligned(1024))) uint16_t lds[kJStages * kJStageElems];

  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int wv = wave % kJWV;
  const int wt_ = wave / kJWV;
  const int half = lane >> 5;

  // Placement as in the cross-entropy kernel: the token blocks of one vocab
  // segment run on one XCD and share its L2 for the W slabs.
  const int G = gridDim.x;
  const int bid = blockIdx.x;
  const int L = (G % 8 == 0) ? ((bid % 8) * (G / 8) + bid / 8) : bid;
  const int n_tok_tiles = (int)((tokens + kJT - 1) / kJT);
  const int tb = L % n_tok_tiles;
  const int seg = L / n_tok_tiles;
  const int n_v_tiles = (int)((vocab + kJV - 1) / kJV);
  const int tile0 = (int)(((int64_t)seg * n_v_tiles) / segments);
  const int tile1 = (int)(((int64_t)(seg + 1) * n_v_tiles) / segments);
  const int64_t t0 = (int64_t)tb * kJT;

  const int64_t tok = t0 + wt_ * 32 + (lane & 31);
  const bool tok_ok = tok < tokens;
  const float As = tok_ok ? lse_s[tok] : 0.0f;
  const float At = tok_ok ? lse_t[tok] : 0.0f;

  // DMA plan: DMA i of this wave fills rows 8 * (wave + 8 i) .. + 7 of an
  // operand slab; lane l lands on physical chunk l & 7 of row 8 (wave + 8 i) +
  // (l >> 3).  With 8 waves the swizzled chunk is the same for both DMAs.
  const uint32_t row_bytes = (uint32_t)hidden * 2u;
  const int r0 = 8 * wave + (lane >> 3);
  const uint32_t kch = (uint32_t)swz(r0, lane & 7) * 8u;
  const uint32_t voff0 = (uint32_t)r0 * row_bytes + kch * 2u;
  const uint32_t voff_step = 64u * row_bytes;
  const uint32_t x_rows = (uint32_t)((tokens - t0) < kJT ? (tokens - t0) : kJT);
  const __amdgpu_buffer_rsrc_t xs_r = make_rsrc(xs + t0 * hidden, x_rows * row_bytes);
  const __amdgpu_buffer_rsrc_t xt_r = make_rsrc(xt + t0 * hidden, x_rows * row_bytes);
  auto w_rsrc = [&](const uint16_t* w, int tile) {
    const int64_t v0 = (int64_t)tile * kJV;
    const int64_t left = vocab - v0;
    const uint32_t w_rows = (uint32_t)(left < kJV ? left : kJV);
    return make_rsrc(w + v0 * hidden, w_rows * row_bytes);
  };
  const int nk = (int)((hidden + kJK - 1) / kJK);
  const bool k_ragged = (hidden % kJK) != 0;
  auto issue = [&](__amdgpu_buffer_rsrc_t r, uint16_t* op, int kk) {
    const uint32_t k0 = (uint32_t)kk * kJK;
    const bool tail = k_ragged && kk == nk - 1;
#pragma unroll
    for (int i = 0; i < kJDmas; ++i) {
      uint32_t vo = voff0 + (uint32_t)i * voff_step;
      if (tail && k0 + kch >= (uint32_t)hidden) vo = 0x7ffffff0u;  // past the end: reads zero
      lds_ptr_t dst = (lds_ptr_t)(op + (wave + kJWaves * i) * 8 * kJK);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, vo, k0 * 2u, 0, 0);
    }
  };
  // Stage layout: W_s, W_t, x_s, x_t.
  auto issue_slab = [&](int tile, int kk, int stage) {
    uint16_t* base = lds + stage * kJStageElems;
    issue(w_rsrc(ws, tile), base, kk);
    issue(w_rsrc(wt, tile), base + kJOpElems, kk);
    issue(xs_r, base + 2 * kJOpElems, kk);
    issue(xt_r, base + 3 * kJOpElems, kk);
  };

  int a_row[kJBVB];
#pragma unroll
  for (int a = 0; a < kJBVB; ++a) a_row[a] = wv * (kJBVB * 32) + a * 32 + (lane & 31);
  const int b_row = wt_ * 32 + (lane & 31);

  float jsd = 0.0f;  // this lane's share of its token's divergence
  const int n_iter = (tile1 - tile0) * nk;
  if (n_iter > 0) issue_slab(tile0, 0, 0);
  int it = 0;
  for (int tile = tile0; tile < tile1; ++tile) {
    f32x16 acc_s[kJBVB], acc_t[kJBVB];
#pragma unroll
    for (int a = 0; a < kJBVB; ++a) {
      acc_s[a] = (f32x16)(0.0f);
      acc_t[a] = (f32x16)(0.0f);
    }
    for (int kk = 0; kk < nk; ++kk, ++it) {
      wait_vmcnt<0>();  // this wave's DMAs of slab `it` have landed
      lds_barrier();    // everyone's have; every read of slab it - 1 is done
      if (it + 1 < n_iter) {
        const bool next_tile = kk + 1 == nk;
        issue_slab(next_tile ? tile + 1 : tile, next_tile ? 0 : kk + 1, (it + 1) & 1);
      }
      const uint16_t* base = lds + (it & 1) * kJStageElems;
#pragma unroll
      for (int ks = 0; ks < kJK / 16; ++ks) {
        const int c = 2 * ks + half;
        bf16x8 as[kJBVB], at[kJBVB];
#pragma unroll
        for (int a = 0; a < kJBVB; ++a) {
          as[a] = *reinterpret_cast<const bf16x8*>(base + a_row[a] * kJK + swz(a_row[a], c) * 8);
          at[a] = *reinterpret_cast<const bf16x8*>(base + kJOpElems + a_row[a] * kJK +
                                                   swz(a_row[a], c) * 8);
        }
        const bf16x8 bs = *reinterpret_cast<const bf16x8*>(base + 2 * kJOpElems + b_row * kJK +
                                                           swz(b_row, c) * 8);
        const bf16x8 bt = *reinterpret_cast<const bf16x8*>(base + 3 * kJOpElems + b_row * kJK +
                                                           swz(b_row, c) * 8);
#pragma unroll
        for (int a = 0; a < kJBVB; ++a) {
          acc_s[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as[a], bs, acc_s[a], 0, 0, 0);
          acc_t[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(at[a], bt, acc_t[a], 0, 0, 0);
        }
      }
    }
    // Divergence terms of the finished tile.  acc[a][v] is vocab row
    // vbase + a*32 + 8*(v/4) + 4*half + v%4 of token `tok`.
    const int64_t vbase = (int64_t)tile * kJV + wv * (kJBVB * 32);
#pragma unroll
    for (int a = 0; a < kJBVB; ++a)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t j = vbase + a * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
        const float term = jsd_term(acc_s[a][v] - As, acc_t[a][v] - At, beta);
        jsd += j < vocab ? term : 0.0f;
      }
  }

  // Sum the two lane halves (same token, different vocab rows), then the
  // kJWV waves that share the token, through LDS (free once every wave passed
  // its last slab).
  jsd += half_swap(jsd);
  lds_barrier();
  float* red = reinterpret_cast<float*>(lds);  // [kJWV][kJT]
  const int tl = wt_ * 32 + (lane & 31);
  if (half == 0) red[wv * kJT + tl] = jsd;
  lds_barrier();
  if (wv == 0 && half == 0 && tok_ok) {
    float s = red[tl];
#pragma unroll
    for (int q = 1; q < kJWV; ++q) s += red[q * kJT + tl];
    part[(int64_t)seg * tokens + tok] = s;
  }
}

// Divergence of token rows whose logits are stored: zs and zt are [rows, z_ld]
// fp32 (the first vocab columns of each row are the logits), lse_s / lse_t the
// rows' log-sum-exp.  One workgroup per row streams both rows with 16-byte
// buffer loads (kJRU chunks of each per lane in flight) and writes the row's
// sum to dst[row].  Summation order is fixed: per lane in chunk order, then
// the wave and workgroup reductions.
namespace {
constexpr int kJRThreads = 256;
constexpr int kJRU = 4;
constexpr int kJRPolicy = 2;  // nontemporal: each stored logit is read once
}  // namespace

__global__ __launch_bounds__(kJRThreads) void jsd_stored_rows_kernel(
    const float* __restrict__ zs, const float* __restrict__ zt, int64_t z_ld, int64_t vocab,
    const float* __restrict__ lse_s, const float* __restrict__ lse_t, float beta,
    float* __restrict__ dst) {
  const int64_t row = blockIdx.x;
  const float As = lse_s[row];
  const float At = lse_t[row];
  const uint32_t bytes = (uint32_t)vocab * 4u;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(zs + row * z_ld, bytes);
  const __amdgpu_buffer_rsrc_t rt = make_rsrc(zt + row * z_ld, bytes);
  const int nch = (int)((vocab + 3) / 4);
  float acc = 0.0f;
  for (int c0 = threadIdx.x; c0 < nch; c0 += kJRThreads * kJRU) {
    f32x4 a[kJRU], b[kJRU];
#pragma unroll
    for (int u = 0; u < kJRU; ++u) {
      const uint32_t off = (uint32_t)(c0 + u * kJRThreads) * 16u;  // past the row: reads 0
      a[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kJRPolicy));
      b[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rt, off, 0, kJRPolicy));
    }
#pragma unroll
    for (int u = 0; u < kJRU; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t j = (int64_t)(c0 + u * kJRThreads) * 4 + e;
        const float t = jsd_term(a[u][e] - As, b[u][e] - At, beta);
        acc += j < vocab ? t : 0.0f;
      }
  }
  acc = wave_sum(acc);
  __shared__ float red[kJRThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float tot = red[0];
#pragma unroll
    for (int q = 1; q < kJRThreads / 64; ++q) tot += red[q];
    dst[row] = tot;
  }
}

// One thread per token: the segments' sums in segment order, then the
// per-token divergence or the deterministic batch mean.
__global__ __launch_bounds__(kRowThreads) void fused_jsd_merge_kernel(
    int64_t tokens, int segments, const float* __restrict__ part, float* __restrict__ out,
    uint64_t* __restrict__ slots, unsigned* __restrict__ ticket, int reduce_mean) {
  const int64_t row = (int64_t)blockIdx.x * kRowThreads + threadIdx.x;
  float v = 0.0f;
  if (row < tokens) {
    for (int s = 0; s < segments; ++s) v += part[(int64_t)s * tokens + row];
    if (!reduce_mean) out[row] = v;
  }
  if (reduce_mean) {
    __shared__ float red[kRowThreads];
    red[threadIdx.x] = v;
    __syncthreads();
#pragma unroll
    for (int w = kRowThreads / 2; w > 0; w >>= 1) {
      if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
      __syncthreads();
    }
    finish_mean(red[0], slots, ticket, out, tokens);
  }
}

int jsd_segments(int64_t tokens, int64_t vocab, int num_cus) {
  const int64_t n_tok = (tokens + kJT - 1) / kJT;
  const int64_t n_voc = (vocab + kJV - 1) / kJV;
  int64_t s = num_cus / (n_tok > 0 ? n_tok : 1);
  if (s < 1) s = 1;
  if (s > n_voc) s = n_voc;
  return (int)s;
}

hipError_t launch_jsd(const JsdArgs& a, hipStream_t stream) {
  const int64_t n_tok = (a.tokens + kJT - 1) / kJT;
  if (!grid_fits(n_tok * a.segments, kJThreads) ||
      !grid_fits((a.tokens + kRowThreads - 1) / kRowThreads, kRowThreads))
    return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(fused_jsd_partial_kernel, dim3((unsigned)(n_tok * a.segments)), dim3(kJThreads),
                     0, stream, (const uint16_t*)a.xs, (const uint16_t*)a.ws, (const uint16_t*)a.xt,
                     (const uint16_t*)a.wt, a.tokens, a.hidden, a.vocab, a.lse_s, a.lse_t, a.beta,
                     a.segments, a.partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t blocks = (a.tokens + kRowThreads - 1) / kRowThreads;
  hipLaunchKernelGGL(fused_jsd_merge_kernel, dim3((unsigned)blocks), dim3(kRowThreads), 0, stream,
                     a.tokens, a.segments, (const float*)a.partials, a.out, a.mean_slots, a.ticket,
                     a.reduce_mean);
  return hipGetLastError();
}

hipError_t launch_jsd_rows(const JsdRowsArgs& a, hipStream_t stream) {
  if (!grid_fits(a.rows, kJRThreads)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(jsd_stored_rows_kernel, dim3((unsigned)a.rows), dim3(kJRThreads), 0, stream,
                     a.zs, a.zt, a.z_ld, a.vocab, a.lse_s, a.lse_t, a.beta, a.dst);
  return hipGetLastError();
}

hipError_t launch_jsd_mean(int64_t tokens, const float* per_token, float* out, uint64_t* slots,
                           unsigned* ticket, hipStream_t stream) {
  const int64_t blocks = (tokens + kRowThreads - 1) / kRowThreads;
  if (!grid_fits(blocks, kRowThreads)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(fused_jsd_merge_kernel, dim3((unsigned)blocks), dim3(kRowThreads), 0, stream,
                     tokens, 1, per_token, out, slots, ticket, 1);
  return hipGetLastError();
}

}  // namespace lce
