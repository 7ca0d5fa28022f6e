// Fused LM-head projection + cross-entropy for gfx950 (bf16 MFMA).
//
// KernelIndex "Fused linear + CPO loss" (description and Semantics): tokens x
// hidden activations projected through a vocab x hidden head, reduced against
// integer targets chunk by chunk, so the [tokens, vocab] logits never exist
// in memory.  Here the reduction is the per-token softmax cross-entropy.
//
// Work decomposition.  The logit matrix z = x W^T is cut into tiles of
// kBV vocab rows x kBT tokens.  A workgroup owns one token block and a
// contiguous segment of vocab tiles; it walks the segment tile by tile, and
// for each tile runs the K loop over `hidden` in slabs of 64:
//   global (16-byte loads, W and x tiles) -> registers -> LDS (double
//   buffered, 16-byte chunks XOR-swizzled per row) -> ds_read_b128 ->
//   v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
// W is the MFMA "A" operand (rows = vocab) and x the "B" operand
// (columns = tokens), so each lane's 32x32 accumulator block holds 16 vocab
// entries of a single token.  After the last slab of a tile every lane folds
// its values straight into that token's running (max, sum-exp) state and, if
// the token's target falls in the tile, records z_target.  At the end of the
// segment the states of the two lane halves and of the waves that share a
// token are merged, and one (max, sum-exp) pair per (segment, token) is
// written.  A small merge kernel combines the segments and finishes the loss
// and, optionally, the deterministic mean.
//
// Placement.  Consecutive workgroup ids are dealt round-robin to the 8 XCDs
// (each with its own L2).  Workgroup ids are remapped so that the token
// blocks of the same vocab segment run on the same XCD at the same time and
// share each W slab through that XCD's L2; W then crosses HBM about once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lce_device.h"
#include "lce_internal.h"

namespace lce {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Tile shape: WV x WT waves; each wave owns BVB x BTB blocks of 32 x 32.
template <int WV, int WT, int BVB, int BTB>
struct Tile {
  static constexpr int kWaves = WV * WT;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kBV = WV * BVB * 32;   // vocab rows per tile
  static constexpr int kBT = WT * BTB * 32;   // tokens per tile
  static constexpr int kBK = 64;              // hidden elements per slab (128 B per row)
  static constexpr int kRowsLds = kBV + kBT;  // W rows, then x rows
  static constexpr int kGroups = kRowsLds / 8;          // 1 KiB (8-row) LDS groups per slab
  static constexpr int kGroupsW = kBV / 8;
  static constexpr int kGroupsPerWave = kGroups / kWaves;
  static_assert(kGroups % kWaves == 0, "slab groups per wave");
  static_assert(kGroupsW % kWaves == 0, "W groups per wave");
};

typedef Tile<2, 2, 4, 4> FusedTile;  // 256 vocab x 256 tokens, 4 waves of 128 x 128

// Physical 16-byte chunk of logical chunk `c` in LDS row `r`: conflict-free
// ds_read_b128 for 8 or 16 consecutive rows read at the same logical chunk.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r & 7) ^ ((r >> 3) & 1)); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Buffer resource over `bytes` bytes at `base` (raw, unswizzled; loads past the
// end return zero).  gfx9 word 3: 32-bit data format, no swizzle.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Fold one token column of a finished tile into that token's running state and
// capture its target logit.  acc[a][v] is the logit of vocab row
// vbase + a*32 + 8*(v/4) + 4*half + v%4.  RAGGED masks rows >= vocab.
template <int BVB, bool RAGGED>
__device__ __forceinline__ void fold_tile_column(Lse& st, const f32x16 (&acc)[BVB], int64_t vbase,
                                                 int64_t vocab, int half, int tgt, float* zt_dst) {
  float bm = kNegInf;
#pragma unroll
  for (int a = 0; a < BVB; ++a)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const bool ok = !RAGGED || (vbase + a * 32 + 8 * (v >> 2) + 4 * half + (v & 3) < vocab);
      bm = fmaxf(bm, ok ? acc[a][v] : kNegInf);
    }
  const float mn = fmaxf(st.m, bm);
  if (mn != kNegInf) {
    const float Mn = mn * kLog2e;
    float tsum = 0.0f;
#pragma unroll
    for (int a = 0; a < BVB; ++a) {
      float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const bool ok0 = !RAGGED || (vbase + a * 32 + 8 * (v >> 2) + 4 * half + (v & 3) < vocab);
        const bool ok1 = !RAGGED || (vbase + a * 32 + 8 * (v >> 2) + 4 * half + ((v + 1) & 3) < vocab);
        const float e0 = exp2_fast(__builtin_fmaf(acc[a][v], kLog2e, -Mn));
        const float e1 = exp2_fast(__builtin_fmaf(acc[a][v + 1], kLog2e, -Mn));
        s0 += ok0 ? e0 : 0.0f;
        s1 += ok1 ? e1 : 0.0f;
      }
      tsum += s0 + s1;
    }
    st.s = st.s * lse_rescale(st.m, mn) + tsum;
    st.m = mn;
  }
  // Target logit: only the one lane holding (token, target) writes it.
  const int64_t rel = (int64_t)tgt - vbase;
  if (tgt >= 0 && rel >= 0 && rel < BVB * 32) {
    const int r = (int)rel & 31;
    if (((r >> 2) & 1) == half) {
      const int ai = (int)rel >> 5;
      const int vi = ((r >> 3) << 2) | (r & 3);
      float z = 0.0f;
#pragma unroll
      for (int a = 0; a < BVB; ++a)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (a == ai && v == vi) z = acc[a][v];
      *zt_dst = z;
    }
  }
}

template <int WV, int WT, int BVB, int BTB>
__global__ __launch_bounds__(64 * WV * WT) void fused_xent_partial_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int64_t tokens, int64_t hidden,
    int64_t vocab, const int64_t* __restrict__ target, int segments, float2* __restrict__ part,
    float* __restrict__ zt_out) {
  typedef Tile<WV, WT, BVB, BTB> TL;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2][TL::kRowsLds * 64];

  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int wv = wave % WV;  // wave position along vocab
  const int wt = wave / WV;  // wave position along tokens
  const int half = lane >> 5;

  // XCD-aware placement: logical index L keeps one XCD's workgroups together.
  const int G = gridDim.x;
  const int bid = blockIdx.x;
  const int L = (G % 8 == 0) ? ((bid % 8) * (G / 8) + bid / 8) : bid;
  const int n_tok_tiles = (int)((tokens + TL::kBT - 1) / TL::kBT);
  const int tb = L % n_tok_tiles;
  const int seg = L / n_tok_tiles;
  const int n_v_tiles = (int)((vocab + TL::kBV - 1) / TL::kBV);
  const int tile0 = (int)(((int64_t)seg * n_v_tiles) / segments);
  const int tile1 = (int)(((int64_t)(seg + 1) * n_v_tiles) / segments);
  const int64_t t0 = (int64_t)tb * TL::kBT;

  // This lane's tokens and their targets (-1 when outside [0, vocab)).
  int64_t tok[BTB];
  int tgt[BTB];
#pragma unroll
  for (int j = 0; j < BTB; ++j) {
    tok[j] = t0 + wt * (BTB * 32) + j * 32 + (lane & 31);
    const int64_t t = (tok[j] < tokens) ? target[tok[j]] : -1;
    tgt[j] = (t >= 0 && t < vocab) ? (int)t : -1;
  }

  // Global -> LDS plan.  A slab is kRowsLds rows of 64 bf16 (128 B); one wave
  // instruction (64 lanes x 16 B) fills LDS group g = rows [8g, 8g + 8).  Wave
  // `wave` issues groups g = wave + kWaves * i.  Lane l lands on physical chunk
  // l & 7 of row 8g + (l >> 3), so it loads the logical chunk that the swizzle
  // maps there.  Offsets are relative to the tile's W or x block; the slab's
  // hidden offset is the uniform soffset.
  const uint32_t row_bytes = (uint32_t)hidden * 2u;
  uint32_t voff[TL::kGroupsPerWave];
  uint32_t kchunk[TL::kGroupsPerWave];
#pragma unroll
  for (int i = 0; i < TL::kGroupsPerWave; ++i) {
    const int g = wave + TL::kWaves * i;
    const int r = 8 * g + (lane >> 3);
    const int c = swz(r, lane & 7);  // swz is an involution in its chunk argument
    const int rr = (i < TL::kGroupsW / TL::kWaves) ? r : r - TL::kBV;
    voff[i] = (uint32_t)rr * row_bytes + (uint32_t)c * 16u;
    kchunk[i] = (uint32_t)c * 8u;
  }
  const bool k_ragged = (hidden % TL::kBK) != 0;

  Lse st[BTB];
#pragma unroll
  for (int j = 0; j < BTB; ++j) st[j] = lse_empty();

  const int nk = (int)((hidden + TL::kBK - 1) / TL::kBK);
  const int n_iter = (tile1 - tile0) * nk;
  const uint32_t x_rows = (uint32_t)((tokens - t0) < TL::kBT ? (tokens - t0) : TL::kBT);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + t0 * hidden, x_rows * row_bytes);

  auto issue_slab = [&](int tile, int kk, int buf) {
    const int64_t v0 = (int64_t)tile * TL::kBV;
    const uint32_t w_rows = (uint32_t)((vocab - v0) < TL::kBV ? (vocab - v0) : TL::kBV);
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(w + v0 * hidden, w_rows * row_bytes);
    const uint32_t k0 = (uint32_t)kk * TL::kBK;
    const uint32_t soff = k0 * 2u;
#pragma unroll
    for (int i = 0; i < TL::kGroupsPerWave; ++i) {
      const int g = wave + TL::kWaves * i;
      uint32_t vo = voff[i];
      if (k_ragged && k0 + kchunk[i] >= (uint32_t)hidden) vo = 0x7ffffff0u;  // past the end: zeros
      lds_ptr_t dst = (lds_ptr_t)(&lds[buf][g * 8 * 64]);
      if (i < TL::kGroupsW / TL::kWaves)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, dst, 16, vo, soff, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, dst, 16, vo, soff, 0, 0);
    }
  };

  if (n_iter > 0) issue_slab(tile0, 0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's slab is in LDS
  __syncthreads();

  // LDS read addresses (bf16 elements) of this lane's fragments at k-step 0;
  // k-step ks adds the swizzled chunk offset, computed per lane below.
  int a_row[BVB], b_row[BTB];
#pragma unroll
  for (int a = 0; a < BVB; ++a) a_row[a] = wv * (BVB * 32) + a * 32 + (lane & 31);
#pragma unroll
  for (int b = 0; b < BTB; ++b) b_row[b] = TL::kBV + wt * (BTB * 32) + b * 32 + (lane & 31);

  int it = 0;
  for (int tile = tile0; tile < tile1; ++tile) {
    f32x16 acc[BTB][BVB];
#pragma unroll
    for (int b = 0; b < BTB; ++b)
#pragma unroll
      for (int a = 0; a < BVB; ++a) acc[b][a] = (f32x16)(0.0f);

    for (int kk = 0; kk < nk; ++kk, ++it) {
      const int cur = it & 1;
      if (it + 1 < n_iter) {
        const bool next_tile = (kk + 1 == nk);
        issue_slab(next_tile ? tile + 1 : tile, next_tile ? 0 : kk + 1, cur ^ 1);
      }
      const uint16_t* S = lds[cur];
      // Fragments of k-step ks+1 are read while k-step ks is multiplied.
      bf16x8 af[2][BVB], bfr[2][BTB];
#pragma unroll
      for (int a = 0; a < BVB; ++a)
        af[0][a] = *reinterpret_cast<const bf16x8*>(S + a_row[a] * 64 + swz(a_row[a], half) * 8);
#pragma unroll
      for (int b = 0; b < BTB; ++b)
        bfr[0][b] = *reinterpret_cast<const bf16x8*>(S + b_row[b] * 64 + swz(b_row[b], half) * 8);
#pragma unroll
      for (int ks = 0; ks < TL::kBK / 16; ++ks) {
        const int p = ks & 1;
        if (ks + 1 < TL::kBK / 16) {
          const int c = 2 * (ks + 1) + half;
#pragma unroll
          for (int a = 0; a < BVB; ++a)
            af[p ^ 1][a] = *reinterpret_cast<const bf16x8*>(S + a_row[a] * 64 + swz(a_row[a], c) * 8);
#pragma unroll
          for (int b = 0; b < BTB; ++b)
            bfr[p ^ 1][b] = *reinterpret_cast<const bf16x8*>(S + b_row[b] * 64 + swz(b_row[b], c) * 8);
        }
        // Keep the reads above ahead of this k-step's MFMAs (the scheduler would
        // otherwise sink each read next to its first use and expose LDS latency).
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < BTB; ++b)
#pragma unroll
          for (int a = 0; a < BVB; ++a)
            acc[b][a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[p][a], bfr[p][b], acc[b][a], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): next slab landed in LDS
      __syncthreads();
    }

    // Epilogue of the finished tile, one token column at a time.
    const int64_t vbase = (int64_t)tile * TL::kBV + wv * (BVB * 32);
    if (vbase + BVB * 32 > vocab) {
#pragma unroll
      for (int b = 0; b < BTB; ++b)
        fold_tile_column<BVB, true>(st[b], acc[b], vbase, vocab, half, tgt[b], zt_out + tok[b]);
    } else {
#pragma unroll
      for (int b = 0; b < BTB; ++b)
        fold_tile_column<BVB, false>(st[b], acc[b], vbase, vocab, half, tgt[b], zt_out + tok[b]);
    }
  }

  // Merge the two lane halves (same tokens, different vocab rows) ...
#pragma unroll
  for (int b = 0; b < BTB; ++b) {
    const Lse o{half_swap(st[b].m), half_swap(st[b].s)};
    st[b] = (half == 0) ? lse_merge(st[b], o) : lse_merge(o, st[b]);
  }
  // ... then the WV waves that share these tokens, through LDS.
  float* red = reinterpret_cast<float*>(&lds[0][0]);  // [WV][kBT][2]
  if (half == 0) {
#pragma unroll
    for (int b = 0; b < BTB; ++b) {
      const int tl = wt * (BTB * 32) + b * 32 + (lane & 31);
      red[(wv * TL::kBT + tl) * 2 + 0] = st[b].m;
      red[(wv * TL::kBT + tl) * 2 + 1] = st[b].s;
    }
  }
  __syncthreads();
  if (wv == 0 && half == 0) {
#pragma unroll
    for (int b = 0; b < BTB; ++b) {
      const int tl = wt * (BTB * 32) + b * 32 + (lane & 31);
      Lse acc_st{red[tl * 2 + 0], red[tl * 2 + 1]};
#pragma unroll
      for (int q = 1; q < WV; ++q)
        acc_st = lse_merge(acc_st, Lse{red[(q * TL::kBT + tl) * 2 + 0], red[(q * TL::kBT + tl) * 2 + 1]});
      if (tok[b] < tokens) part[(int64_t)seg * tokens + tok[b]] = make_float2(acc_st.m, acc_st.s);
    }
  }
}

// One thread per token: merge its `segments` partials in segment order
// (consecutive threads read consecutive tokens of a segment), subtract z_target.
__global__ __launch_bounds__(kRowThreads) void fused_xent_merge_kernel(
    int64_t tokens, int64_t vocab, int segments, const float2* __restrict__ part,
    const float* __restrict__ zt, const int64_t* __restrict__ target, float* __restrict__ out,
    float* __restrict__ partials, unsigned* __restrict__ ticket, int reduce_mean) {
  const int64_t row = (int64_t)blockIdx.x * kRowThreads + threadIdx.x;
  float loss = 0.0f;
  if (row < tokens) {
    Lse st = lse_empty();
    for (int s = 0; s < segments; ++s) {
      const float2 p = part[(int64_t)s * tokens + row];
      st = lse_merge(st, Lse{p.x, p.y});
    }
    const int64_t t = target[row];
    loss = (t >= 0 && t < vocab) ? lse_minus(st, zt[row]) : __builtin_nanf("");
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
    finish_mean(red[0], partials, ticket, out, tokens);
  }
}

FusedGeometry fused_geometry() { return {FusedTile::kBT, FusedTile::kBV}; }

int fused_segments(int64_t tokens, int64_t vocab, int num_cus) {
  const int64_t n_tok = (tokens + FusedTile::kBT - 1) / FusedTile::kBT;
  const int64_t n_voc = (vocab + FusedTile::kBV - 1) / FusedTile::kBV;
  int64_t s = num_cus / (n_tok > 0 ? n_tok : 1);
  if (s < 1) s = 1;
  if (s > n_voc) s = n_voc;
  return (int)s;
}

hipError_t launch_fused(const FusedArgs& a, hipStream_t stream) {
  const int64_t n_tok = (a.tokens + FusedTile::kBT - 1) / FusedTile::kBT;
  const int64_t grid = n_tok * a.segments;
  hipLaunchKernelGGL((fused_xent_partial_kernel<2, 2, 4, 4>), dim3((unsigned)grid),
                     dim3(FusedTile::kThreads), 0, stream, (const uint16_t*)a.x,
                     (const uint16_t*)a.w, a.tokens, a.hidden, a.vocab, a.target, a.segments,
                     (float2*)a.seg_partials, a.target_logit);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t blocks = (a.tokens + kRowThreads - 1) / kRowThreads;
  hipLaunchKernelGGL(fused_xent_merge_kernel, dim3((unsigned)blocks), dim3(kRowThreads), 0, stream,
                     a.tokens, a.vocab, a.segments, (const float2*)a.seg_partials,
                     (const float*)a.target_logit, a.target, a.out, a.mean_partials, a.ticket,
                     a.reduce_mean);
  return hipGetLastError();
}

}  // namespace lce
