// Internal interface between liblce's host dispatch (lce_api.cpp) and its
// kernel launchers (xent_kernels.hip, fused_kernel.hip).  Not installed.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace lce {

constexpr int kRowThreads = 256;  // threads per workgroup of the row kernels

// Bytes of the mean state's header at the start of its buffer: the epoch
// word on a 256-byte line of its own (see finish_mean in lce_device.h).
constexpr size_t kMeanHeaderBytes = 256;

// A dispatch counts its work-items in 32 bits, so blocks * threads must stay
// below 2^32.  Launchers check it (hipErrorInvalidConfiguration); the entry
// points refuse such sizes first, with LCE_ERR_UNSUPPORTED.
constexpr int64_t kMaxGridItems = (int64_t(1) << 32) - 1;
inline bool grid_fits(int64_t blocks, int64_t threads) {
  return blocks >= 0 && blocks <= kMaxGridItems / threads;
}

enum class XentPath : int { WaveRows = 0, BlockRows = 1, Split = 2, GroupRows = 3 };

struct XentArgs {
  const void* logits;
  bool bf16;
  int64_t tokens;
  int64_t vocab;
  const int64_t* target;
  float* out;
  int reduce_mean;
  int64_t vocab_start;      // first full-vocab column of these rows (0 for whole rows)
  float* stats;             // non-null: write (m, s, zt) per row instead of losses
  XentPath path;
  int unroll;               // chunks per lane per batch (wave_rows: 4, 8 or 16)
  int waves_per_block;      // WaveRows: rows (waves) per workgroup, 4 or 16 (then unroll <= 8)
  int rows_per_wave;        // GroupRows: 2, 4 or 8 rows per wave (4 waves per workgroup)
  int splits;               // Split: workgroups per row
  int chunks_per_split;     // Split: 16-byte chunks per workgroup
  float* split_partials;    // Split: splits * tokens (max, sum-exp) pairs, slice-major
  float* split_zt;          // Split: tokens target logits (NaN where not held)
  uint64_t* mean_slots;     // one 64-bit (tag, partial) slot per workgroup of the last kernel
  unsigned* epoch;          // the mean state's epoch word (advanced by every launch with a mean)
};

hipError_t launch_xent(const XentArgs& a, hipStream_t stream);

// Gradient with respect to the logits.
struct BwdArgs {
  const void* logits;
  bool bf16;
  int64_t tokens;
  int64_t vocab;
  const int64_t* target;
  const float* grad;        // 1 (mean) or tokens (none) fp32
  int reduce_mean;
  void* dlogits;            // same dtype and layout as logits; may be logits itself
  int rows_per_wave;        // 2, 4 or 8: several short rows per wave (no scalar edges); else 0
  int wave_chunks;          // > 0: one wave per row holding <= 64 * wave_chunks chunks
  const float* stats;       // otherwise: (m, s, .) per row from the statistics mode
  int splits;               //   workgroups per row
  int chunks_per_split;     //   16-byte chunks per workgroup
  float* loss_out;          // wave_chunks > 0: also the losses (or their mean) here; else null
  uint64_t* mean_slots;     //   with reduce_mean: the mean state
  unsigned* epoch;
};

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);
// Rows per workgroup of the one-wave-per-row gradient kernel for these arguments.
int bwd_wave_rows(const BwdArgs& a);

// Losses (or their mean) from [shards][tokens][3] vocab-shard statistics.
hipError_t launch_stats_merge(const float* stats, int64_t shards, int64_t tokens,
                              const int64_t* target, int64_t vocab, float* out, int reduce_mean,
                              uint64_t* slots, unsigned* epoch, hipStream_t stream);

// Fused projection + cross-entropy.
struct FusedArgs {
  const void* x;          // bf16 [tokens, hidden]
  const void* w;          // bf16 [vocab, hidden]
  int64_t tokens;
  int64_t hidden;
  int64_t vocab;
  const int64_t* target;
  float* out;
  int reduce_mean;
  float* lse_out;         // non-null: write ln sum_j e^z_j per token; losses (or the mean)
                          // go to out only when out is non-null (target may then be null)
  float* z_out;           // non-null: also store the fp32 logits as [tokens, z_ld] rows
  int64_t z_ld;           // multiple of block_vocab, >= vocab; z_ld * block_tokens * 4 < 2^32
  int segments;           // vocab segments (workgroups per token block)
  float* seg_partials;    // segments * tokens (max, sum-exp) pairs
  float* target_logit;    // tokens fp32
  uint64_t* mean_slots;
  unsigned* epoch;
};

// Logit gradient of the fused projection for a block of tokens, written as
// bf16 rows dz [tokens, dz_ld]: dz_ij = g_i (e^(z_ij - lse_i) - [j == t_i]),
// g_i = grad[0] / grad_tokens (grad_mean) or grad[i]; NaN rows for targets
// outside [0, vocab).  Columns in [vocab, dz_ld) receive values for zero
// logits and are never meaningful.
struct FusedGradArgs {
  const void* x;          // bf16 [tokens, hidden]
  const void* w;          // bf16 [vocab, hidden]
  int64_t tokens;
  int64_t hidden;
  int64_t vocab;
  const int64_t* target;  // [tokens]
  const float* lse;       // [tokens] ln sum_j e^z_ij
  const float* grad;      // [1] or [tokens]
  int grad_mean;
  int64_t grad_tokens;    // divisor of grad[0] with grad_mean
  void* dz;               // bf16 [tokens, dz_ld]
  int64_t dz_ld;          // multiple of block_vocab, >= vocab; dz_ld * block_tokens * 2 < 2^32
  int segments;
};
hipError_t launch_fused_grad(const FusedGradArgs& a, hipStream_t stream);

// Geometry of the fused kernel, needed by the host to size scratch.
struct FusedGeometry {
  int block_tokens;   // tokens per workgroup tile
  int block_vocab;    // vocab rows per workgroup tile
};
FusedGeometry fused_geometry();
// The JSD mode's tile (its token tiles size the recompute path's grid).
FusedGeometry jsd_geometry();
int fused_segments(int64_t tokens, int64_t vocab, int num_cus);
hipError_t launch_fused(const FusedArgs& a, hipStream_t stream);

// out[b] = -sum of loss[b * seq .. b * seq + seq - 1] (per-sequence log-prob sums).
hipError_t launch_seq_logprob_sums(const float* loss, int64_t batch, int64_t seq, float* out,
                                   hipStream_t stream);

// Fused projection + generalized JSD between a student and a teacher head.
struct JsdArgs {
  const void* xs;           // bf16 [tokens, hidden], student activations
  const void* ws;           // bf16 [vocab, hidden], student head
  const void* xt;           // teacher activations
  const void* wt;           // teacher head
  int64_t tokens;
  int64_t hidden;
  int64_t vocab;
  float beta;
  const float* lse_s;       // [tokens] ln sum_j e^(student logits)
  const float* lse_t;       // [tokens] the same for the teacher
  float* out;
  int reduce_mean;
  int segments;
  float* partials;          // [segments, tokens]
  uint64_t* mean_slots;
  unsigned* epoch;
};
int jsd_segments(int64_t tokens, int64_t vocab, int num_cus);
// The fused kernel's JSD mode alone (per-segment sums into partials).
hipError_t launch_fused_jsd_partial(const JsdArgs& a, hipStream_t stream);
// That, then the merge into per-token divergences or their mean.
hipError_t launch_jsd(const JsdArgs& a, hipStream_t stream);

// Divergence of rows whose logits were stored by the fused kernel (z_out).
struct JsdRowsArgs {
  const float* zs;          // [rows, z_ld] student logits
  const float* zt;          // [rows, z_ld] teacher logits
  int64_t z_ld;
  int64_t rows;
  int64_t vocab;            // < 2^30
  const float* lse_s;       // [rows]
  const float* lse_t;       // [rows]
  float beta;
  float* dst;               // [rows] per-token divergence
};
hipError_t launch_jsd_rows(const JsdRowsArgs& a, hipStream_t stream);
// Deterministic mean of `tokens` per-token values into out[0].
hipError_t launch_jsd_mean(int64_t tokens, const float* per_token, float* out, uint64_t* slots,
                           unsigned* epoch, hipStream_t stream);

hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t stream);
hipError_t launch_zero_u32(unsigned* p, int64_t n, hipStream_t stream);

}  // namespace lce
