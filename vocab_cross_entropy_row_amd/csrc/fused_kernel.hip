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
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Tile shape: WV x WT waves; each wave owns BVB x BTB blocks of 32 x 32.
template <int WV, int WT, int BVB, int BTB>
struct Tile {
  static constexpr int kWaves = WV * WT;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kBV = WV * BVB * 32;  // vocab rows per tile
  static constexpr int kBT = WT * BTB * 32;  // tokens per tile
  static constexpr int kBK = 64;             // hidden elements per slab
  static constexpr int kRowsLds = kBV + kBT; // W rows then x rows
  static constexpr int kChunks = kRowsLds * 8;        // 16-byte chunks per slab
  static constexpr int kChunksW = kBV * 8;
  static constexpr int kPerThread = kChunks / kThreads;
  static constexpr int kPerThreadW = kChunksW / kThreads;
  static_assert(kChunks % kThreads == 0 && kChunksW % kThreads == 0, "slab split");
};

typedef Tile<2, 4, 4, 2> FusedTile;  // 256 vocab x 256 tokens, 8 waves

// Physical 16-byte chunk of logical chunk `c` in LDS row `r`: conflict-free
// ds_read_b128 for 8 or 16 consecutive rows read at the same logical chunk.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r & 7) ^ ((r >> 3) & 1)); }

template <class TL>
__device__ __forceinline__ void load_slab(u32x4_t (&reg)[TL::kPerThread], const uint16_t* __restrict__ x,
                                          const uint16_t* __restrict__ w, int64_t tokens,
                                          int64_t hidden, int64_t vocab, int64_t v0, int64_t t0,
                                          int64_t k0) {
#pragma unroll
  for (int i = 0; i < TL::kPerThread; ++i) {
    const int c = threadIdx.x + i * TL::kThreads;
    const bool is_w = i < TL::kPerThreadW;
    const int r = is_w ? (c >> 3) : ((c - TL::kChunksW) >> 3);
    const int kc = c & 7;
    const int64_t k = k0 + kc * 8;
    const int64_t g = is_w ? (v0 + r) : (t0 + r);
    const bool ok = (g < (is_w ? vocab : tokens)) && (k < hidden);
    const uint16_t* src = (is_w ? w : x) + g * hidden + k;
    reg[i] = ok ? *reinterpret_cast<const u32x4_t*>(src) : (u32x4_t)(0u);
  }
}

template <class TL>
__device__ __forceinline__ void store_slab(uint16_t* lds, const u32x4_t (&reg)[TL::kPerThread]) {
#pragma unroll
  for (int i = 0; i < TL::kPerThread; ++i) {
    const int c = threadIdx.x + i * TL::kThreads;
    const int row = c >> 3;  // W rows first, then x rows, in one array
    const int kc = c & 7;
    *reinterpret_cast<u32x4_t*>(lds + row * 64 + swz(row, kc) * 8) = reg[i];
  }
}

template <int WV, int WT, int BVB, int BTB>
__global__ __launch_bounds__(64 * WV * WT) void fused_xent_partial_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int64_t tokens, int64_t hidden,
    int64_t vocab, const int64_t* __restrict__ target, int segments, float2* __restrict__ part,
    float* __restrict__ zt_out) {
  typedef Tile<WV, WT, BVB, BTB> TL;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][TL::kRowsLds * 64];

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
    int64_t t = (tok[j] < tokens) ? target[tok[j]] : -1;
    tgt[j] = (t >= 0 && t < vocab) ? (int)t : -1;
  }

  Lse st[BTB];
#pragma unroll
  for (int j = 0; j < BTB; ++j) st[j] = lse_empty();

  const int nk = (int)((hidden + TL::kBK - 1) / TL::kBK);
  const int n_iter = (tile1 - tile0) * nk;

  // Slab pipeline over the flattened (tile, k) sequence: slab it+1 is loaded
  // from global memory while slab it is multiplied out of LDS.
  u32x4_t reg[TL::kPerThread];
  if (n_iter > 0) {
    load_slab<TL>(reg, x, w, tokens, hidden, vocab, (int64_t)tile0 * TL::kBV, t0, 0);
    store_slab<TL>(lds[0], reg);
  }
  __syncthreads();

  int it = 0;
  for (int tile = tile0; tile < tile1; ++tile) {
    f32x16 acc[BVB][BTB];
#pragma unroll
    for (int a = 0; a < BVB; ++a)
#pragma unroll
      for (int b = 0; b < BTB; ++b) acc[a][b] = (f32x16)(0.0f);

    for (int kk = 0; kk < nk; ++kk, ++it) {
      const int cur = it & 1;
      const bool more = (it + 1) < n_iter;
      if (more) {
        const bool next_tile = (kk + 1 == nk);
        load_slab<TL>(reg, x, w, tokens, hidden, vocab,
                      (int64_t)(next_tile ? tile + 1 : tile) * TL::kBV, t0,
                      (int64_t)(next_tile ? 0 : kk + 1) * TL::kBK);
      }
      const uint16_t* Ws = lds[cur];
      const uint16_t* Xs = lds[cur] + TL::kBV * 64;
#pragma unroll
      for (int ks = 0; ks < TL::kBK / 16; ++ks) {
        const int c = 2 * ks + half;
        bf16x8 af[BVB], bfr[BTB];
#pragma unroll
        for (int a = 0; a < BVB; ++a) {
          const int r = wv * (BVB * 32) + a * 32 + (lane & 31);
          af[a] = *reinterpret_cast<const bf16x8*>(Ws + r * 64 + swz(r, c) * 8);
        }
#pragma unroll
        for (int b = 0; b < BTB; ++b) {
          const int r = wt * (BTB * 32) + b * 32 + (lane & 31);
          bfr[b] = *reinterpret_cast<const bf16x8*>(Xs + r * 64 + swz(TL::kBV + r, c) * 8);
        }
#pragma unroll
        for (int a = 0; a < BVB; ++a)
#pragma unroll
          for (int b = 0; b < BTB; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
      }
      if (more) store_slab<TL>(lds[cur ^ 1], reg);
      __syncthreads();
    }

    // Epilogue of the finished tile.  acc[a][b][v] is the logit of token
    // tok[b] and vocab row vbase + a*32 + 8*(v/4) + 4*half + v%4.
    const int64_t vbase = (int64_t)tile * TL::kBV + wv * (BVB * 32);
    const bool ragged = vbase + BVB * 32 > vocab;
#pragma unroll
    for (int b = 0; b < BTB; ++b) {
      if (ragged) {
#pragma unroll
        for (int a = 0; a < BVB; ++a)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int64_t vi = vbase + a * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
            if (vi >= vocab) acc[a][b][v] = kNegInf;
          }
      }
      float bm = kNegInf;
#pragma unroll
      for (int a = 0; a < BVB; ++a)
#pragma unroll
        for (int v = 0; v < 16; ++v) bm = fmaxf(bm, acc[a][b][v]);
      const float mn = fmaxf(st[b].m, bm);
      const float Mn = mn * kLog2e;
      float tsum = 0.0f;
#pragma unroll
      for (int a = 0; a < BVB; ++a) {
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          s0 += exp2_fast(__builtin_fmaf(acc[a][b][v], kLog2e, -Mn));
          s1 += exp2_fast(__builtin_fmaf(acc[a][b][v + 1], kLog2e, -Mn));
        }
        tsum += s0 + s1;
      }
      if (mn != kNegInf) {
        st[b].s = st[b].s * lse_rescale(st[b].m, mn) + tsum;
        st[b].m = mn;
      }
      // Target logit: only the one lane holding (tok, target) writes it.
      const int64_t rel = (int64_t)tgt[b] - vbase;
      if (tgt[b] >= 0 && rel >= 0 && rel < BVB * 32) {
        const int r = (int)rel & 31;
        if (((r >> 2) & 1) == half) {
          const int ai = (int)rel >> 5;
          const int vi = ((r >> 3) << 2) | (r & 3);
          float z = 0.0f;
#pragma unroll
          for (int a = 0; a < BVB; ++a)
#pragma unroll
            for (int v = 0; v < 16; ++v)
              if (a == ai && v == vi) z = acc[a][b][v];
          zt_out[tok[b]] = z;
        }
      }
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

// One wave per token: merge its `segments` partials, subtract z_target.
__global__ __launch_bounds__(kRowThreads) void fused_xent_merge_kernel(
    int64_t tokens, int64_t vocab, int segments, const float2* __restrict__ part,
    const float* __restrict__ zt, const int64_t* __restrict__ target, float* __restrict__ out,
    float* __restrict__ partials, unsigned* __restrict__ ticket, int reduce_mean) {
  constexpr int kWaves = kRowThreads / 64;
  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int64_t row = (int64_t)blockIdx.x * kWaves + wave;
  float loss = 0.0f;
  if (row < tokens) {
    Lse st = lse_empty();
    for (int s = lane; s < segments; s += 64) {
      const float2 p = part[(int64_t)s * tokens + row];
      st = lse_merge(st, Lse{p.x, p.y});
    }
    const Lse r = wave_lse(st);
    const int64_t t = target[row];
    loss = (t >= 0 && t < vocab) ? lse_minus(r, zt[row]) : __builtin_nanf("");
    if (!reduce_mean && lane == 0) out[row] = loss;
  }
  if (reduce_mean) {
    __shared__ float wl[kWaves];
    if (lane == 0) wl[wave] = loss;
    __syncthreads();
    float bsum = 0.0f;
    if (threadIdx.x == 0)
      for (int i = 0; i < kWaves; ++i) bsum += wl[i];
    finish_mean<kRowThreads>(bsum, partials, ticket, out, tokens);
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
  hipLaunchKernelGGL((fused_xent_partial_kernel<2, 4, 4, 2>), dim3((unsigned)grid),
                     dim3(FusedTile::kThreads), 0, stream, (const uint16_t*)a.x,
                     (const uint16_t*)a.w, a.tokens, a.hidden, a.vocab, a.target, a.segments,
                     (float2*)a.seg_partials, a.target_logit);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t blocks = (a.tokens + kRowThreads / 64 - 1) / (kRowThreads / 64);
  hipLaunchKernelGGL(fused_xent_merge_kernel, dim3((unsigned)blocks), dim3(kRowThreads), 0, stream,
                     a.tokens, a.vocab, a.segments, (const float2*)a.seg_partials,
                     (const float*)a.target_logit, a.target, a.out, a.mean_partials, a.ticket,
                     a.reduce_mean);
  return hipGetLastError();
}

}  // namespace lce
