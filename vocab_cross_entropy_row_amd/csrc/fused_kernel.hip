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
//   global -> LDS directly (16-byte buffer loads into LDS, no registers;
//   W slabs rotate through three stages and x slabs through two, 16-byte
//   chunks XOR-swizzled per row) -> ds_read_b128 ->
//   v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
// W is the MFMA "A" operand (rows = vocab) and x the "B" operand
// (columns = tokens), so each lane's 32x32 accumulator block holds 16 vocab
// entries of a single token.  After the last slab of a tile every lane folds
// its values straight into that token's running (max, sum-exp) state and, if
// the token's target falls in the tile, records z_target.  At the end of the
// segment the states of the two lane halves and of the waves that share a
// token are merged, and one (max, sum-exp) pair per (segment, token) is
// written.  A small merge kernel combines the segments and finishes the loss
// and, optionally, the deterministic mean.  The same pipeline serves the
// kernel's other modes (stored logits, the logit gradient, and the
// generalized JSD of two projections: KernelIndex "Fused linear + JSD",
// description), which differ only in the epilogue and, for the JSD, in
// running each tile's K loop once per head.
//
// Placement.  Consecutive workgroup ids are dealt round-robin to the 8 XCDs
// (each with its own L2).  Workgroup ids are remapped so that the token
// blocks of the same vocab segment run on the same XCD at the same time and
// share each W slab through that XCD's L2; W then crosses HBM about once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lce_device.h"
#include "lce_internal.h"
#include "mfma_common.h"

namespace lce {


// Tile shape: WV x WT waves, each owning BVB x BTB blocks of 32 x 32; K-slabs
// of 64 hidden elements (one 128-byte LDS row per W row and per token).  W
// slabs rotate through WST stages, x slabs through XST stages.
template <int WV, int WT, int BVB, int BTB, int WST, int XST>
struct Tile {
  static constexpr int kWaves = WV * WT;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kBV = WV * BVB * 32;   // vocab rows per tile
  static constexpr int kBT = WT * BTB * 32;   // tokens per tile
  static constexpr int kBK = 64;              // hidden elements per slab
  static constexpr int kKSteps = kBK / 16;    // MFMA k-steps per slab
  static constexpr int kWStages = WST;
  static constexpr int kXStages = XST;
  static constexpr int kWStageElems = kBV * kBK;
  static constexpr int kXStageElems = kBT * kBK;
  static constexpr int kLdsElems = WST * kWStageElems + XST * kXStageElems;
  static constexpr int kWPerWave = kBV / 8 / kWaves;  // 1 KiB W DMAs per wave per slab
  static constexpr int kXPerWave = kBT / 8 / kWaves;  // 1 KiB x DMAs per wave per slab
  static_assert((kBV / 8) % kWaves == 0 && (kBT / 8) % kWaves == 0, "slab groups per wave");
  static_assert(kWPerWave <= 63, "vmcnt range");
};

// 256 vocab x 256 tokens (8 waves of 128 vocab x 64 tokens); 3 W + 2 x stages
// of 32 KiB fill the 160 KiB of LDS.
typedef Tile<2, 4, 4, 2, 3, 2> FusedTile;

// JSD mode: 256 vocab x 128 tokens (8 waves of 64 x 64) per head, so that both
// heads' accumulators fit (2 x 64 per lane); 3 W stages of 32 KiB and 2 x
// stages of 16 KiB.
typedef Tile<4, 2, 2, 2, 3, 2> JsdTile;


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

// Store the logits of a finished tile into z [tokens, z_ld] fp32 (token
// rows): for each (a, v/4) the lane's four consecutive vocab rows of its token
// are one 16-byte store.  `zr` covers the rows of this token tile that exist,
// so stores for tokens past the end are dropped; z_ld is a multiple of the
// tile's vocab extent, so columns past vocab land in the row's padding.
template <int BVB>
__device__ __forceinline__ void store_tile_column(__amdgpu_buffer_rsrc_t zr, const f32x16 (&acc)[BVB],
                                                  uint32_t voff) {
#pragma unroll
  for (int a = 0; a < BVB; ++a)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 q = {acc[a][4 * g], acc[a][4 * g + 1], acc[a][4 * g + 2], acc[a][4 * g + 3]};
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, q), zr,
                                             voff + (uint32_t)(a * 32 + 8 * g) * 4u, 0, 0);
    }
}

// Store the logit gradient of a finished tile into dz [tokens, dz_ld] bf16
// (token rows): dz_j = g * e^(z_j - lse) - [j == t] * g for the lane's token,
// with L = lse * log2e, rounded to nearest even; for each (a, v/4) the lane's
// four consecutive vocab rows are one 8-byte store.  Same addressing as
// store_tile_column.
template <int BVB>
__device__ __forceinline__ void store_tile_grad(__amdgpu_buffer_rsrc_t dr, const f32x16 (&acc)[BVB],
                                                uint32_t voff, int64_t vbase, int half, float L,
                                                float g, int tgt) {
  // Target row relative to this lane's first row of the tile (-1: not here).
  const int64_t rel64 = (int64_t)tgt - vbase - 4 * half;
  const int rel = (tgt >= 0 && rel64 >= 0 && rel64 < BVB * 32) ? (int)rel64 : -1;
#pragma unroll
  for (int a = 0; a < BVB; ++a)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float d[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        d[e] = g * exp2_fast(__builtin_fmaf(acc[a][4 * q + e], kLog2e, -L));
        if (rel == a * 32 + 8 * q + e) d[e] -= g;
      }
      const u32x2 packed = {
          __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{d[0], d[1]}), bf16x2)),
          __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{d[2], d[3]}), bf16x2))};
      __builtin_amdgcn_raw_buffer_store_b64(packed, dr, voff + (uint32_t)(a * 32 + 8 * q) * 2u, 0, 0);
    }
}

// MODE: kFusedXent (per-token (max, sum-exp) partials and the target logit),
// kFusedStoreLogits (the same, and the fp32 logits into z_out), kFusedGrad
// (only the bf16 logit gradient into dz_out, from the log-sum-exp `lse` and
// the loss-output gradient: grad[0] / grad_tokens with grad_mean, else
// grad[token]; NaN rows for targets outside [0, vocab)), kFusedJsd (two
// projections, x W^T and x2 W2^T, each tile's K loop run once per head into
// its own accumulators, then per element the generalized JSD term from the
// heads' log-sum-exps `lse` and `lse2`; per (segment, token) sums into
// jsd_part).
constexpr int kFusedXent = 0;
constexpr int kFusedStoreLogits = 1;
constexpr int kFusedGrad = 2;
constexpr int kFusedJsd = 3;

template <class TL, int BVB, int BTB, int WV, int MODE>
__global__ __launch_bounds__(TL::kThreads) void fused_xent_partial_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int64_t tokens, int64_t hidden,
    int64_t vocab, const int64_t* __restrict__ target, int segments, float2* __restrict__ part,
    float* __restrict__ zt_out, float* __restrict__ z_out, int64_t z_ld,
    const float* __restrict__ lse, const float* __restrict__ grad, int grad_mean,
    int64_t grad_tokens, uint16_t* __restrict__ dz_out, const uint16_t* __restrict__ x2,
    const uint16_t* __restrict__ w2, const float* __restrict__ lse2, float beta,
    float* __restrict__ jsd_part) {
  constexpr bool STORE = MODE == kFusedStoreLogits;
  constexpr bool GRAD = MODE == kFusedGrad;
  constexpr bool JSD = MODE == kFusedJsd;
  constexpr int kHeads = JSD ? 2 : 1;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[TL::kLdsElems];
  constexpr int kXBase = TL::kWStages * TL::kWStageElems;  // x stages follow the W stages

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
    const int64_t t = (target && tok[j] < tokens) ? target[tok[j]] : -1;
    tgt[j] = (t >= 0 && t < vocab) ? (int)t : -1;
  }
  // Gradient mode: L = lse * log2e and the row's output gradient (NaN for an
  // invalid target) of each of this lane's tokens.
  float gL[BTB], gg[BTB];
  if constexpr (GRAD) {
#pragma unroll
    for (int j = 0; j < BTB; ++j) {
      const bool in = tok[j] < tokens;
      gL[j] = in ? lse[tok[j]] * kLog2e : 0.0f;
      const float g = grad_mean ? grad[0] / (float)grad_tokens : (in ? grad[tok[j]] : 0.0f);
      gg[j] = (!in || tgt[j] >= 0) ? g : __builtin_nanf("");
    }
  }

  // JSD mode: both heads' log-sum-exps of each of this lane's tokens.
  float lA[BTB], lB[BTB];
  if constexpr (JSD) {
#pragma unroll
    for (int j = 0; j < BTB; ++j) {
      const bool in = tok[j] < tokens;
      lA[j] = in ? lse[tok[j]] : 0.0f;
      lB[j] = in ? lse2[tok[j]] : 0.0f;
    }
  }

  // Global -> LDS plan.  One wave instruction (64 lanes x 16 B) fills 8 LDS
  // rows; W DMA i of this wave fills W-stage rows 8g .. 8g+7, g = wave + kWaves*i,
  // and likewise for x.  Lane l lands on physical chunk l & 7 of row
  // 8g + (l >> 3), so it loads the logical chunk the swizzle maps there.
  // Offsets are relative to the tile's W or x block; the slab's hidden offset
  // is the uniform soffset.
  // With an even number of waves, the swizzled chunk of every row a lane fills
  // is the same ((r >> 3) & 1 is the wave's parity for all its DMAs), so DMA i
  // differs from DMA 0 only by 8 * kWaves rows.
  static_assert(TL::kWaves % 2 == 0, "one swizzled chunk per lane");
  const uint32_t row_bytes = (uint32_t)hidden * 2u;
  const int r0 = 8 * wave + (lane >> 3);
  const uint32_t kch = (uint32_t)swz(r0, lane & 7) * 8u;  // hidden offset of the lane's chunk
  const uint32_t voff0 = (uint32_t)r0 * row_bytes + kch * 2u;
  const uint32_t voff_step = 8u * TL::kWaves * row_bytes;
  Lse st[BTB];
#pragma unroll
  for (int j = 0; j < BTB; ++j) st[j] = lse_empty();

  const int nk = (int)((hidden + TL::kBK - 1) / TL::kBK);
  const int n_iter = (tile1 - tile0) * nk * kHeads;
  const uint32_t x_rows = (uint32_t)((tokens - t0) < TL::kBT ? (tokens - t0) : TL::kBT);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + t0 * hidden, x_rows * row_bytes);
  const __amdgpu_buffer_rsrc_t xr2 = make_rsrc(JSD ? x2 + t0 * hidden : x, JSD ? x_rows * row_bytes : 0u);
  // Logit rows of this token tile (STORE only); byte offset of this lane's
  // first row and column, relative to vocab tile 0.
  // (GRAD: the same for dz_out, bf16 elements, leading dimension z_ld.)
  constexpr uint32_t kZBytes = GRAD ? 2u : 4u;
  const __amdgpu_buffer_rsrc_t zr =
      GRAD ? make_rsrc(dz_out + t0 * z_ld, x_rows * (uint32_t)z_ld * kZBytes)
           : make_rsrc(z_out + t0 * z_ld, STORE ? x_rows * (uint32_t)z_ld * kZBytes : 0u);
  uint32_t z_voff[BTB];
  if constexpr (STORE || GRAD) {
#pragma unroll
    for (int b = 0; b < BTB; ++b)
      z_voff[b] = ((uint32_t)(wt * (BTB * 32) + b * 32 + (lane & 31)) * (uint32_t)z_ld +
                   (uint32_t)(wv * (BVB * 32) + 4 * half)) * kZBytes;
  }

  // W block of vocab tile `tile` of head `head` (W2 for head 1, JSD mode) as a
  // buffer resource (rows past vocab read 0).
  auto w_rsrc = [&](int tile, int head) {
    const int64_t v0 = (int64_t)tile * TL::kBV;
    const int64_t left = vocab - v0;  // <= 0 only for a tile past the end, never loaded
    const uint32_t w_rows = (uint32_t)(left < 0 ? 0 : (left < TL::kBV ? left : TL::kBV));
    const uint16_t* wh = (JSD && head) ? w2 : w;
    return make_rsrc(wh + (left < 0 ? 0 : v0 * hidden), w_rows * row_bytes);
  };
  // DMA i of this wave for a slab at hidden offset k0 into a W or x stage.
  // `tail` marks the last slab of a hidden size that is not a multiple of 64:
  // chunks past the end read zeros.
  auto issue_w = [&](int i, __amdgpu_buffer_rsrc_t wr, uint32_t k0, bool tail, uint16_t* stage) {
    uint32_t vo = voff0 + (uint32_t)i * voff_step;
    if (tail && k0 + kch >= (uint32_t)hidden) vo = 0x7ffffff0u;
    lds_ptr_t dst = (lds_ptr_t)(stage + (wave + TL::kWaves * i) * 8 * TL::kBK);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, dst, 16, vo, k0 * 2u, 0, 0);
  };
  auto issue_x = [&](int i, __amdgpu_buffer_rsrc_t xres, uint32_t k0, bool tail, uint16_t* stage) {
    uint32_t vo = voff0 + (uint32_t)i * voff_step;
    if (tail && k0 + kch >= (uint32_t)hidden) vo = 0x7ffffff0u;
    lds_ptr_t dst = (lds_ptr_t)(stage + (wave + TL::kWaves * i) * 8 * TL::kBK);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xres, dst, 16, vo, k0 * 2u, 0, 0);
  };
  constexpr int kWPerGroup = TL::kWPerWave / BTB;  // spread over one k-step's MFMA groups
  constexpr int kXPerGroup = TL::kXPerWave / BTB;
  static_assert(kWPerGroup * BTB == TL::kWPerWave && kXPerGroup * BTB == TL::kXPerWave, "DMA spread");

  // LDS rows of this lane's fragments.
  int a_row[BVB], b_row[BTB];
#pragma unroll
  for (int a = 0; a < BVB; ++a) a_row[a] = wv * (BVB * 32) + a * 32 + (lane & 31);
#pragma unroll
  for (int b = 0; b < BTB; ++b) b_row[b] = wt * (BTB * 32) + b * 32 + (lane & 31);

  const bool k_ragged = (hidden % TL::kBK) != 0;
  auto slab_is_tail = [&](int kk) { return k_ragged && kk == nk - 1; };

  // Fragment loads of k-step ks of slab stages (Ws, Xs) into fragment buffer p.
  bf16x8 af[2][BVB], bfr[2][BTB];
  auto read_frags = [&](const uint16_t* Ws, const uint16_t* Xs, int ks, int p) {
    const int c = 2 * ks + half;
#pragma unroll
    for (int a = 0; a < BVB; ++a)
      af[p][a] = *reinterpret_cast<const bf16x8*>(Ws + a_row[a] * TL::kBK + swz(a_row[a], c) * 8);
#pragma unroll
    for (int b = 0; b < BTB; ++b)
      bfr[p][b] = *reinterpret_cast<const bf16x8*>(Xs + b_row[b] * TL::kBK + swz(b_row[b], c) * 8);
  };

  // Pipeline.  W slabs (the operand that misses to HBM) rotate through
  // kWStages stages and x slabs through kXStages.  The barrier of slab `it`
  // sits before its last k-step: by then its last fragments are in registers
  // and its stages are free.  Right after it, the x slab it+kXStages goes into
  // the freed x stage (spread over the last k-step's MFMAs), and during the
  // next slab's first k-step the W slab it+kWStages goes into the freed W
  // stage.  Every x slab is issued before the newer W slab, so at the next
  // barrier "all but the newest W slab landed" is exactly what is needed.
  int wq = 0;                  // it % kWStages
  int xq = 0;                  // it % kXStages
  // W cursor (next W slab to issue) and x cursor (next x slab to issue).
  // In JSD mode each tile's slabs run head 0 (x, W) then head 1 (x2, W2).
  int w_kk = 0, w_tile = tile0, w_head = 0, w_left = n_iter;
  __amdgpu_buffer_rsrc_t w_cur = w_rsrc(tile0, 0);
  int x_kk = 0, x_head = 0, x_left = n_iter;
  auto w_issue_part = [&](int stage, int group) {  // this wave's W DMAs for MFMA group `group`
#pragma unroll
    for (int d = 0; d < kWPerGroup; ++d) {
      const int i = group * kWPerGroup + d;
      issue_w(i, w_cur, (uint32_t)w_kk * TL::kBK, slab_is_tail(w_kk), lds + stage * TL::kWStageElems);
    }
  };
  auto w_advance = [&]() {
    --w_left;
    if (++w_kk == nk) {
      w_kk = 0;
      if (JSD && w_head == 0) {
        w_head = 1;
      } else {
        w_head = 0;
        ++w_tile;
      }
      w_cur = w_rsrc(w_tile, w_head);
    }
  };
  auto x_issue_part = [&](int stage, int group) {
    const __amdgpu_buffer_rsrc_t xres = (JSD && x_head) ? xr2 : xr;
#pragma unroll
    for (int d = 0; d < kXPerGroup; ++d) {
      const int i = group * kXPerGroup + d;
      issue_x(i, xres, (uint32_t)x_kk * TL::kBK, slab_is_tail(x_kk),
              lds + kXBase + stage * TL::kXStageElems);
    }
  };
  auto x_advance = [&]() {
    --x_left;
    if (++x_kk == nk) {
      x_kk = 0;
      if constexpr (JSD) x_head ^= 1;
    }
  };

  // Prologue: x slabs 0 .. kXStages-1 and W slabs 0 .. kWStages-1, in the
  // order x0 W0 x1 W1 W2: slab 0 landed, then at slab 0's barrier everything
  // but W2 must have landed.
  for (int j = 0; j < TL::kWStages; ++j) {
    if (j < TL::kXStages && x_left > 0) {
#pragma unroll
      for (int g = 0; g < BTB; ++g) x_issue_part(j, g);
      x_advance();
    }
    if (w_left > 0) {
#pragma unroll
      for (int g = 0; g < BTB; ++g) w_issue_part(j, g);
      w_advance();
    }
    if (j == 0) {
      wait_vmcnt<0>();  // only the first x and W slabs have been issued
      __syncthreads();
    }
  }
  if (n_iter > 0) read_frags(lds, lds + kXBase, 0, 0);

  int it = 0;
  float jsd[BTB];  // JSD mode: this lane's share of each token's divergence
#pragma unroll
  for (int b = 0; b < BTB; ++b) jsd[b] = 0.0f;
  for (int tile = tile0; tile < tile1; ++tile) {
    // Each head's K loop (one head except in JSD mode) into its accumulators:
    // nk slabs per head.  The head loop is unrolled, so `A` names a fixed array.
    f32x16 acc[BTB][BVB], acc2[BTB][BVB];
#pragma unroll
    for (int h = 0; h < kHeads; ++h) {
      f32x16 (&A)[BTB][BVB] = h == 0 ? acc : acc2;
#pragma unroll
      for (int b = 0; b < BTB; ++b)
#pragma unroll
        for (int a = 0; a < BVB; ++a) A[b][a] = (f32x16)(0.0f);

      for (int kk = 0; kk < nk; ++kk, ++it) {
        const uint16_t* Ws = lds + wq * TL::kWStageElems;
        const uint16_t* Xs = lds + kXBase + xq * TL::kXStageElems;
        // W slab issued in this slab's first k-step (into the stage freed at the
        // previous barrier), if any is left.
        const int w_stage_free = (wq + TL::kWStages - 1) % TL::kWStages;
        const bool w_now = (it > 0) && (w_left > 0);
#pragma unroll
        for (int ks = 0; ks < TL::kKSteps - 1; ++ks) {
          const int p = ks & 1;
          read_frags(Ws, Xs, ks + 1, p ^ 1);
#pragma unroll
          for (int b = 0; b < BTB; ++b) {
#pragma unroll
            for (int a = 0; a < BVB; ++a)
              A[b][a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[p][a], bfr[p][b], A[b][a], 0, 0, 0);
            if (ks == 0 && w_now) w_issue_part(w_stage_free, b);
          }
        }
        if (w_now) w_advance();
        // The next slab's x and W have landed for every wave (only the newest W
        // slab may still be in flight); every read of this slab is done.
        if (w_now) wait_vmcnt<TL::kWPerWave>(); else wait_vmcnt<0>();
        lds_barrier();
        const int wq1 = (wq + 1 == TL::kWStages) ? 0 : wq + 1;
        const int xq1 = (xq + 1 == TL::kXStages) ? 0 : xq + 1;
        const bool x_now = x_left > 0;
        if (it + 1 < n_iter)
          read_frags(lds + wq1 * TL::kWStageElems, lds + kXBase + xq1 * TL::kXStageElems, 0, 0);
        constexpr int pl = (TL::kKSteps - 1) & 1;
#pragma unroll
        for (int b = 0; b < BTB; ++b) {
#pragma unroll
          for (int a = 0; a < BVB; ++a)
            A[b][a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[pl][a], bfr[pl][b], A[b][a], 0, 0, 0);
          if (x_now) x_issue_part(xq, b);  // x slab it + kXStages into this slab's x stage
        }
        if (x_now) x_advance();
        wq = wq1;
        xq = xq1;
      }
    }
    if constexpr (JSD) {
      // Head 1's logits of the same tile, then the divergence terms:
      // acc[b][a][v] is vocab row vbase + a*32 + 8*(v/4) + 4*half + v%4 of token tok[b].
      const int64_t vbase = (int64_t)tile * TL::kBV + wv * (BVB * 32);
#pragma unroll
      for (int b = 0; b < BTB; ++b)
#pragma unroll
        for (int a = 0; a < BVB; ++a)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int64_t j = vbase + a * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
            const float term = jsd_term(acc[b][a][v] - lA[b], acc2[b][a][v] - lB[b], beta);
            jsd[b] += j < vocab ? term : 0.0f;
          }
      continue;
    }

    // Epilogue of the finished tile, one token column at a time.
    const int64_t vbase = (int64_t)tile * TL::kBV + wv * (BVB * 32);
    if constexpr (STORE) {
#pragma unroll
      for (int b = 0; b < BTB; ++b)
        store_tile_column<BVB>(zr, acc[b], z_voff[b] + (uint32_t)tile * (uint32_t)TL::kBV * 4u);
    }
    if constexpr (GRAD) {
#pragma unroll
      for (int b = 0; b < BTB; ++b)
        store_tile_grad<BVB>(zr, acc[b], z_voff[b] + (uint32_t)tile * (uint32_t)TL::kBV * 2u, vbase,
                             half, gL[b], gg[b], tgt[b]);
      continue;  // no (max, sum-exp) state in this mode
    }
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

  if constexpr (GRAD) return;
  if constexpr (JSD) {
    // Sum the two lane halves (same tokens, different vocab rows), then the WV
    // waves that share these tokens, in wave order, through LDS (free: every
    // wave passed the barrier after its last slab).
    float* red = reinterpret_cast<float*>(lds);  // [WV][kBT]
#pragma unroll
    for (int b = 0; b < BTB; ++b) {
      const float v = jsd[b] + half_swap(jsd[b]);
      if (half == 0) red[wv * TL::kBT + wt * (BTB * 32) + b * 32 + (lane & 31)] = v;
    }
    __syncthreads();
    if (wv == 0 && half == 0) {
#pragma unroll
      for (int b = 0; b < BTB; ++b) {
        const int tl = wt * (BTB * 32) + b * 32 + (lane & 31);
        float sum = red[tl];
#pragma unroll
        for (int q = 1; q < WV; ++q) sum += red[q * TL::kBT + tl];
        if (tok[b] < tokens) jsd_part[(int64_t)seg * tokens + tok[b]] = sum;
      }
    }
    return;
  }
  // Merge the two lane halves (same tokens, different vocab rows) ...
#pragma unroll
  for (int b = 0; b < BTB; ++b) {
    const Lse o{half_swap(st[b].m), half_swap(st[b].s)};
    st[b] = (half == 0) ? lse_merge(st[b], o) : lse_merge(o, st[b]);
  }
  // ... then the WV waves that share these tokens, through LDS (the slab
  // stages are free: every wave passed the barrier after its last slab).
  float* red = reinterpret_cast<float*>(lds);  // [WV][kBT][2]
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
// Writes ln sum_j e^z_j per token into lse_out when it is set, and the loss
// (or the mean) into out when that is set; at least one of them is.
// The partials are loaded 32 segments at a time (the default segment count
// of the benchmark shapes), so the loads of a group are in flight together
// instead of one memory latency per segment or per group of eight; padding
// entries past `segments` merge as exact no-ops.
__global__ __launch_bounds__(kRowThreads) void fused_xent_merge_kernel(
    int64_t tokens, int64_t vocab, int segments, const float2* __restrict__ part,
    const float* __restrict__ zt, const int64_t* __restrict__ target, float* __restrict__ out,
    float* __restrict__ lse_out, uint64_t* __restrict__ slots, unsigned* __restrict__ epoch,
    int reduce_mean) {
  const unsigned mean_tag = mean_begin(epoch, reduce_mean);
  const int64_t row = (int64_t)blockIdx.x * kRowThreads + threadIdx.x;
  float loss = 0.0f;
  if (row < tokens) {
    const int64_t t = out ? target[row] : -1;
    const float z = out ? zt[row] : 0.0f;
    constexpr int kGroup = 32;
    Lse st = lse_empty();
    for (int s0 = 0; s0 < segments; s0 += kGroup) {
      float2 p[kGroup];
#pragma unroll
      for (int j = 0; j < kGroup; ++j)
        p[j] = (s0 + j < segments) ? part[(int64_t)(s0 + j) * tokens + row] : make_float2(kNegInf, 0.0f);
#pragma unroll
      for (int j = 0; j < kGroup; ++j) st = lse_merge(st, Lse{p[j].x, p[j].y});
    }
    if (lse_out)  // ln sum_j e^z_j = m + ln2 * (log2 s - (m*log2e - fp32(m*log2e)))
      lse_out[row] = st.m + kLn2 * (log2_fast(st.s) - __builtin_fmaf(st.m, kLog2e, -(st.m * kLog2e)));
    if (!out) return;  // (no mean without out)
    loss = (t >= 0 && t < vocab) ? lse_minus(st, z) : __builtin_nanf("");
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

FusedGeometry fused_geometry() { return {FusedTile::kBT, FusedTile::kBV}; }
FusedGeometry jsd_geometry() { return {JsdTile::kBT, JsdTile::kBV}; }

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
  if (!grid_fits(grid, FusedTile::kThreads) ||
      !grid_fits((a.tokens + kRowThreads - 1) / kRowThreads, kRowThreads))
    return hipErrorInvalidConfiguration;
  if (a.z_out)
    hipLaunchKernelGGL((fused_xent_partial_kernel<FusedTile, 4, 2, 2, kFusedStoreLogits>),
                       dim3((unsigned)grid), dim3(FusedTile::kThreads), 0, stream,
                       (const uint16_t*)a.x, (const uint16_t*)a.w, a.tokens, a.hidden, a.vocab,
                       a.target, a.segments, (float2*)a.seg_partials, a.target_logit, a.z_out,
                       a.z_ld, nullptr, nullptr, 0, (int64_t)0, nullptr, nullptr, nullptr, nullptr,
                       0.0f, nullptr);
  else
    hipLaunchKernelGGL((fused_xent_partial_kernel<FusedTile, 4, 2, 2, kFusedXent>),
                       dim3((unsigned)grid), dim3(FusedTile::kThreads), 0, stream,
                       (const uint16_t*)a.x, (const uint16_t*)a.w, a.tokens, a.hidden, a.vocab,
                       a.target, a.segments, (float2*)a.seg_partials, a.target_logit, nullptr,
                       (int64_t)0, nullptr, nullptr, 0, (int64_t)0, nullptr, nullptr, nullptr,
                       nullptr, 0.0f, nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t blocks = (a.tokens + kRowThreads - 1) / kRowThreads;
  hipLaunchKernelGGL(fused_xent_merge_kernel, dim3((unsigned)blocks), dim3(kRowThreads), 0, stream,
                     a.tokens, a.vocab, a.segments, (const float2*)a.seg_partials,
                     (const float*)a.target_logit, a.target, a.out, a.lse_out, a.mean_slots, a.epoch,
                     a.reduce_mean);
  return hipGetLastError();
}

hipError_t launch_fused_grad(const FusedGradArgs& a, hipStream_t stream) {
  const int64_t n_tok = (a.tokens + FusedTile::kBT - 1) / FusedTile::kBT;
  const int64_t grid = n_tok * a.segments;
  if (!grid_fits(grid, FusedTile::kThreads)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fused_xent_partial_kernel<FusedTile, 4, 2, 2, kFusedGrad>),
                     dim3((unsigned)grid), dim3(FusedTile::kThreads), 0, stream,
                     (const uint16_t*)a.x, (const uint16_t*)a.w, a.tokens, a.hidden, a.vocab,
                     a.target, a.segments, nullptr, nullptr, nullptr, a.dz_ld, a.lse, a.grad,
                     a.grad_mean, a.grad_tokens, (uint16_t*)a.dz, nullptr, nullptr, nullptr, 0.0f,
                     nullptr);
  return hipGetLastError();
}

int jsd_segments(int64_t tokens, int64_t vocab, int num_cus) {
  const int64_t n_tok = (tokens + JsdTile::kBT - 1) / JsdTile::kBT;
  const int64_t n_voc = (vocab + JsdTile::kBV - 1) / JsdTile::kBV;
  int64_t s = num_cus / (n_tok > 0 ? n_tok : 1);
  if (s < 1) s = 1;
  if (s > n_voc) s = n_voc;
  return (int)s;
}

hipError_t launch_fused_jsd_partial(const JsdArgs& a, hipStream_t stream) {
  const int64_t n_tok = (a.tokens + JsdTile::kBT - 1) / JsdTile::kBT;
  const int64_t grid = n_tok * a.segments;
  if (!grid_fits(grid, JsdTile::kThreads)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fused_xent_partial_kernel<JsdTile, 2, 2, 4, kFusedJsd>), dim3((unsigned)grid),
                     dim3(JsdTile::kThreads), 0, stream, (const uint16_t*)a.xs, (const uint16_t*)a.ws,
                     a.tokens, a.hidden, a.vocab, nullptr, a.segments, nullptr, nullptr, nullptr,
                     (int64_t)0, a.lse_s, nullptr, 0, (int64_t)0, nullptr, (const uint16_t*)a.xt,
                     (const uint16_t*)a.wt, a.lse_t, a.beta, a.partials);
  return hipGetLastError();
}

}  // namespace lce
