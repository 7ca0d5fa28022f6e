// liblce entry points of the row cross-entropy (forward, backward, vocab-shard
// statistics and merge) and of the fused projection + cross-entropy forward,
// with their path selection.  Every entry point validates its arguments on the
// host before it makes any HIP call, so argument errors never touch the device.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "lce.h"
#include "lce_host.h"
#include "lce_internal.h"

namespace lce {
namespace host {

// Row kernels for `tokens` rows of `vocab` columns: per-token losses or their
// mean into `out`, or (stats != nullptr) per-row vocab-shard statistics, with
// targets read relative to `vocab_start`.  Arguments are validated; tokens > 0.
// The first `reserved` bytes of scratch regions belong to the caller.
lce_status run_rows(const void* logits, int dtype, int64_t tokens, int64_t vocab,
                    const int64_t* target, bool mean, float* out, int64_t vocab_start,
                    float* stats, hipStream_t stream, size_t reserved, const RowWorkspace* ws) {
  lce_status s = LCE_OK;
  int cus = 0;
  if ((s = num_cus(&cus)) != LCE_OK) return s;

  lce::XentArgs a{};
  a.logits = logits;
  a.bf16 = dtype == LCE_BF16;
  a.vocab_start = vocab_start;
  a.stats = stats;
  a.tokens = tokens;
  a.vocab = vocab;
  a.target = target;
  a.out = out;
  a.reduce_mean = mean ? 1 : 0;

  // Path selection (measured on MI355X):
  //  - rows up to 2 KiB without scalar edges: several rows per wave;
  //  - rows up to 32 KiB: one wave per row; 4 waves per workgroup without a
  //    mean, 16 with a mean (a quarter of the partials to hand off);
  //  - longer rows: without a mean, one workgroup per row; with a mean, one
  //    wave per row in 16-wave workgroups; with few rows, several workgroups
  //    per row (split).
  const int64_t esize = a.bf16 ? 2 : 4;
  const int64_t row_bytes = vocab * esize;
  const int64_t nvec = row_bytes / 16;
  // Chunks per lane per batch (two batches are in flight at once).  Rows of
  // up to 8 chunks per lane take batches of 4 when there is a mean or the
  // logits are bf16.  With a mean, the 16-wave workgroups end at a barrier, and
  // at the register count of 8-chunk batches only one such workgroup fits on a
  // CU, which then idles until its slowest row is done; with 4-chunk batches
  // two fit (bf16 [8192, 4096] mean 16.4 -> 14.6 us, fp32 [16384, 2048] mean
  // 26.7 -> 24.5 us).  Without a mean, bf16 rows gain a little (bf16
  // [8192, 4096] 12.01-12.07 -> 11.94 us) and fp32 rows lose (fp32
  // [16384, 2048] 20.83 -> 21.10 us); fp32 rows of 16 chunks per lane with a
  // mean are slower with 4 as well (45.2 vs 44.3 us).  Rows of one or two
  // chunks per lane take batches of exactly that size: larger batches would be
  // mostly loads past the row (bf16 [65536, 512] 30.8 -> 18.6 us per token,
  // 46.3 -> 34.2 us with a mean; fp32 [65536, 256] 23.2 -> 16.9 us).
  // Rows longer than 32 KiB with a mean (one wave per row, 16-wave
  // workgroups) take batches of 4 as well: fp32 [16384, 131072] mean
  // 1236 -> 1231 us, the same in three interleaved rounds (51 instead of 87
  // VGPRs: two 16-wave workgroups fit on a CU instead of one).
  const int64_t per_lane = (nvec + 63) / 64;
  a.unroll = (per_lane <= 4 || (per_lane <= 8 && (mean || a.bf16))) ? 4 : 8;
  if (mean && row_bytes > 32 * 1024) a.unroll = 4;
  if (per_lane <= 2) a.unroll = per_lane < 1 ? 1 : (int)per_lane;
  a.waves_per_block = 4;
  if (row_bytes <= 32 * 1024) {
    a.path = lce::XentPath::WaveRows;
    if (mean) a.waves_per_block = 16;
  } else if (tokens >= 2 * (int64_t)cus) {
    if (mean) {
      a.path = lce::XentPath::WaveRows;
      a.waves_per_block = 16;
    } else {
      a.path = lce::XentPath::BlockRows;
    }
  } else {
    a.path = lce::XentPath::Split;
  }
  // Rows of at most 128 chunks (2 KiB) with no scalar edges (the logits
  // 16-byte aligned and the row bytes a multiple of 16): several rows per wave,
  // N = 64 / G lanes per row with up to 4 chunks each, so a row's fixed work is
  // one lane group's, not one wave's (bf16 [65536, 512] 18.9 -> 13.3 us per
  // token, 25.0 -> 15.6 us with a mean; bf16 [131072, 128] 32.1 -> 10.8 us).
  const bool edgeless = row_bytes % 16 == 0 && ((uintptr_t)logits % 16) == 0;
  if (a.path == lce::XentPath::WaveRows && edgeless && nvec <= 128) {
    a.path = lce::XentPath::GroupRows;
    a.rows_per_wave = nvec <= 32 ? 8 : nvec <= 64 ? 4 : 2;
  }
  // Overrides for tuning and tests.
  const char* forced = getenv("LCE_PATH");
  if (forced && !strcmp(forced, "wave")) a.path = lce::XentPath::WaveRows;
  else if (forced && !strcmp(forced, "block")) a.path = lce::XentPath::BlockRows;
  else if (forced && !strcmp(forced, "split")) a.path = lce::XentPath::Split;
  const int forced_unroll = env_int("LCE_UNROLL", 0);
  if (forced_unroll == 1 || forced_unroll == 2 || forced_unroll == 4 || forced_unroll == 8 ||
      forced_unroll == 16)
    a.unroll = forced_unroll;
  const int forced_waves = env_int("LCE_WAVES_PER_BLOCK", 0);
  if (forced_waves == 4 || forced_waves == 16) a.waves_per_block = forced_waves;
  if (a.waves_per_block == 16 && a.unroll > 8) a.unroll = 8;
  // The kernels address a row (or a split slice) with 32-bit buffer offsets.
  if (a.path != lce::XentPath::Split && row_bytes > kMaxStreamBytes) a.path = lce::XentPath::Split;

  size_t need_split = 0;
  if (a.path == lce::XentPath::Split) {
    if (tokens > 65535) return fail(LCE_ERR_UNSUPPORTED, "split path needs tokens <= 65535");
    // Enough workgroups for ~4 per CU, but at least one 256-thread batch of 8
    // chunks per workgroup.
    // A forced count (LCE_SPLITS) may go down to one chunk per thread.
    const int64_t forced_s = env_int("LCE_SPLITS", 0);
    int64_t S = forced_s > 0 ? forced_s : (4 * (int64_t)cus + tokens - 1) / tokens;
    const int64_t per_split = forced_s > 0 ? lce::kRowThreads : lce::kRowThreads * 8;
    const int64_t max_s = (nvec + per_split - 1) / per_split;
    if (S > max_s) S = max_s;
    if (S < 1) S = 1;
    if (S > 65535) S = 65535;
    const int64_t min_s = (nvec * 16 + kMaxStreamBytes - 1) / kMaxStreamBytes;
    if (S < min_s) S = min_s;
    a.splits = (int)S;
    a.chunks_per_split = (int)((nvec + S - 1) / S);
    need_split = (size_t)tokens * (size_t)S * 8u;
  }
  // The split path's target logits follow its partials.
  const size_t off_zt_rel = round_up(need_split, kAlign);
  if (need_split) need_split = off_zt_rel + (size_t)tokens * 4u;
  const int64_t mean_blocks =
      (a.path == lce::XentPath::BlockRows) ? tokens
      : (a.path == lce::XentPath::WaveRows) ? (tokens + a.waves_per_block - 1) / a.waves_per_block
      : (a.path == lce::XentPath::GroupRows) ? (tokens + 4 * a.rows_per_wave - 1) / (4 * a.rows_per_wave)
                                              : (tokens + lce::kRowThreads - 1) / lce::kRowThreads;

  if (ws) {  // the caller's memory: nothing is allocated
    if (need_split > ws->general_bytes)
      return fail(LCE_ERR_UNSUPPORTED,
                  "the split path needs %zu bytes of partials; the workspace holds %zu", need_split,
                  ws->general_bytes);
    if (mean && mean_blocks > ws->max_slots)
      return fail(LCE_ERR_UNSUPPORTED, "the mean needs %lld workgroup slots; the workspace holds %lld",
                  (long long)mean_blocks, (long long)ws->max_slots);
    a.split_partials = (float*)ws->general;
    a.split_zt = (float*)(ws->general + off_zt_rel);
    a.epoch = ws->epoch;
    a.mean_slots = ws->slots;
  } else {
    Carve cv;
    if (reserved) cv.take(reserved);
    const size_t off_split = cv.take(need_split);
    char* base = nullptr;
    if ((s = get_scratch(stream, cv.off, &base)) != LCE_OK) return s;
    a.split_partials = (float*)(base + off_split);
    a.split_zt = (float*)(base + off_split + off_zt_rel);
    if (mean) {
      MeanState ms;
      if ((s = get_mean_state(stream, mean_blocks, &ms)) != LCE_OK) return s;
      a.epoch = ms.epoch;
      a.mean_slots = ms.slots;
    }
  }

  hipError_t e = lce::launch_xent(a, stream);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  // Template arguments as a demangler prints them (T is float or unsigned short).
  const char* tn = a.bf16 ? "unsigned short" : "float";
  if (a.path == lce::XentPath::WaveRows)
    note_launch("xent_wave_rows_kernel<%s, %d, %d> grid %lld x %d", tn, a.unroll, a.waves_per_block,
                (long long)((tokens + a.waves_per_block - 1) / a.waves_per_block), 64 * a.waves_per_block);
  else if (a.path == lce::XentPath::GroupRows)
    note_launch("xent_group_rows_kernel<%s, %d, 4, 4> grid %lld x 256", tn, a.rows_per_wave,
                (long long)((tokens + 4 * a.rows_per_wave - 1) / (4 * a.rows_per_wave)));
  else if (a.path == lce::XentPath::BlockRows)
    note_launch("xent_block_rows_kernel<%s, 8> grid %lld x %d", tn, (long long)tokens, lce::kRowThreads);
  else
    note_launch("xent_split_partial_kernel<%s, %d> grid (%d, %lld) x %d + xent_split_merge_kernel "
                "grid %lld x %d", tn, a.bf16 ? 4 : 8, a.splits, (long long)tokens, lce::kRowThreads,
                (long long)((tokens + lce::kRowThreads - 1) / lce::kRowThreads), lce::kRowThreads);
  return LCE_OK;
}

FusedPlan plan_fused(int64_t tokens, int64_t vocab, int cus, size_t reserved) {
  FusedPlan p;
  p.segments = lce::fused_segments(tokens, vocab, cus);
  const int forced = env_int("LCE_FUSED_SEGMENTS", 0);
  if (forced > 0) {
    const lce::FusedGeometry g = lce::fused_geometry();
    const int64_t n_voc = (vocab + g.block_vocab - 1) / g.block_vocab;
    p.segments = (int)(forced < n_voc ? forced : n_voc);
  }
  Carve cv;
  if (reserved) cv.take(reserved);
  p.off_seg = cv.take((size_t)p.segments * (size_t)tokens * 8u);
  p.off_zt = cv.take((size_t)tokens * 4u);
  p.end = cv.off;
  return p;
}

// The fused projection + cross-entropy for validated arguments, tokens > 0.
// The first `reserved` bytes of scratch regions belong to the caller.  With
// lse_out set, writes ln sum_j e^(z_j) per token there; with out set (and
// target), the losses or their mean; at least one of the two.  With z_out
// set, the logits are also stored there as [tokens, z_ld] fp32 rows.
lce_status run_fused(const void* x, const void* weight, int64_t tokens, int64_t hidden, int64_t vocab,
                     const int64_t* target, bool mean, float* out, hipStream_t stream,
                     size_t reserved, float* lse_out, float* z_out, int64_t z_ld) {
  lce_status s = LCE_OK;
  int cus = 0;
  if ((s = num_cus(&cus)) != LCE_OK) return s;
  const FusedPlan p = plan_fused(tokens, vocab, cus, reserved);

  lce::FusedArgs a{};
  a.x = x;
  a.w = weight;
  a.tokens = tokens;
  a.hidden = hidden;
  a.vocab = vocab;
  a.target = out ? target : nullptr;
  a.out = out;
  a.lse_out = lse_out;
  a.z_out = z_out;
  a.z_ld = z_ld;
  a.reduce_mean = (mean && out) ? 1 : 0;
  a.segments = p.segments;

  char* base = nullptr;
  if ((s = get_scratch(stream, p.end, &base)) != LCE_OK) return s;
  a.seg_partials = (float*)(base + p.off_seg);
  a.target_logit = (float*)(base + p.off_zt);
  if (a.reduce_mean) {
    MeanState ms;
    if ((s = get_mean_state(stream, (tokens + lce::kRowThreads - 1) / lce::kRowThreads, &ms)) != LCE_OK)
      return s;
    a.epoch = ms.epoch;
    a.mean_slots = ms.slots;
  }

  hipError_t e = lce::launch_fused(a, stream);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  const lce::FusedGeometry g = lce::fused_geometry();
  note_launch("fused_xent_partial_kernel (%s) grid %lld x 512 + fused_xent_merge_kernel grid %lld x %d",
              z_out ? (out ? "loss and log-sum-exp, logits stored" : "log-sum-exp, logits stored")
                    : lse_out ? (out ? "loss and log-sum-exp" : "log-sum-exp") : "loss",
              (long long)((tokens + g.block_tokens - 1) / g.block_tokens * p.segments),
              (long long)((tokens + lce::kRowThreads - 1) / lce::kRowThreads), lce::kRowThreads);
  return LCE_OK;
}

}  // namespace host
}  // namespace lce

using namespace lce::host;

extern "C" {

const char* lce_status_string(lce_status status) {
  switch (status) {
    case LCE_OK: return "LCE_OK";
    case LCE_ERR_INVALID_ARG: return "LCE_ERR_INVALID_ARG";
    case LCE_ERR_UNSUPPORTED: return "LCE_ERR_UNSUPPORTED";
    case LCE_ERR_ALIAS: return "LCE_ERR_ALIAS";
    case LCE_ERR_OOM: return "LCE_ERR_OOM";
    case LCE_ERR_HIP: return "LCE_ERR_HIP";
  }
  return "LCE_ERR_UNKNOWN";
}

const char* lce_last_error(void) { return last_error().c_str(); }

const char* lce_last_launch(void) { return last_launch().c_str(); }

int lce_version(void) { return LCE_VERSION_MAJOR * 10000 + LCE_VERSION_MINOR * 100 + LCE_VERSION_PATCH; }

lce_status lce_xent_fwd(const void* logits, lce_dtype dtype, int64_t tokens, int64_t vocab,
                        const int64_t* target, lce_reduction reduction, float* out,
                        hipStream_t stream) {
  begin_call();
  lce_status s = validate_xent(logits, (int)dtype, tokens, vocab, target, (int)reduction, out);
  if (s != LCE_OK) return s;
  const bool mean = reduction == LCE_REDUCTION_MEAN;
  if (tokens == 0) {
    if (!mean) return LCE_OK;
    hipError_t e = lce::launch_fill_f32(out, 1, __builtin_nanf(""), stream);
    return e == hipSuccess ? LCE_OK : hip_fail(e, "launch");
  }
  return run_rows(logits, (int)dtype, tokens, vocab, target, mean, out, 0, nullptr, stream);
}

lce_status lce_xent_partial_fwd(const void* logits, lce_dtype dtype, int64_t tokens,
                                int64_t shard_vocab, int64_t vocab_start, const int64_t* target,
                                float* partial, hipStream_t stream) {
  begin_call();
  // Same checks as lce_xent_fwd with a per-token output of 3 floats.
  lce_status s = validate_xent(logits, (int)dtype, tokens, shard_vocab, target,
                               LCE_REDUCTION_NONE, partial, "partial", 3);
  if (s != LCE_OK) return s;
  if (vocab_start < 0)
    return fail(LCE_ERR_INVALID_ARG, "vocab_start must be >= 0 (got %lld)", (long long)vocab_start);
  if (vocab_start > INT64_MAX - shard_vocab)
    return fail(LCE_ERR_INVALID_ARG, "vocab_start + shard_vocab overflows");
  if (tokens == 0) return LCE_OK;
  return run_rows(logits, (int)dtype, tokens, shard_vocab, target, false, nullptr, vocab_start,
                  partial, stream);
}

lce_status lce_xent_merge(const float* partials, int64_t shards, int64_t tokens,
                          const int64_t* target, int64_t vocab, lce_reduction reduction,
                          float* out, hipStream_t stream) {
  begin_call();
  lce_status s = validate_common(tokens, target, (int)reduction, out);
  if (s != LCE_OK) return s;
  if (shards < 1) return fail(LCE_ERR_INVALID_ARG, "shards must be >= 1 (got %lld)", (long long)shards);
  if (shards >= (int64_t(1) << 31))
    return fail(LCE_ERR_UNSUPPORTED, "shards must be < 2^31 (got %lld)", (long long)shards);
  if (vocab < 1) return fail(LCE_ERR_INVALID_ARG, "vocab must be >= 1 (got %lld)", (long long)vocab);
  if (tokens > 0 && !partials) return fail(LCE_ERR_INVALID_ARG, "partials is NULL");
  if (partials && !aligned(partials, 4)) return fail(LCE_ERR_INVALID_ARG, "partials is not 4-byte aligned");
  if (tokens > INT64_MAX / 12 / shards) return fail(LCE_ERR_INVALID_ARG, "shards * tokens overflows");
  const bool mean = reduction == LCE_REDUCTION_MEAN;
  const uint64_t ob = out_bytes(tokens, (int)reduction);
  if (overlaps(out, ob, partials, (uint64_t)(shards * tokens * 12)))
    return fail(LCE_ERR_ALIAS, "out overlaps partials");
  if (overlaps(out, ob, target, (uint64_t)tokens * 8u)) return fail(LCE_ERR_ALIAS, "out overlaps target");
  if (tokens == 0) {
    if (!mean) return LCE_OK;
    hipError_t e = lce::launch_fill_f32(out, 1, __builtin_nanf(""), stream);
    return e == hipSuccess ? LCE_OK : hip_fail(e, "launch");
  }
  MeanState ms;
  if (mean && (s = get_mean_state(stream, (tokens + lce::kRowThreads - 1) / lce::kRowThreads, &ms)) != LCE_OK)
    return s;
  hipError_t e = lce::launch_stats_merge(partials, shards, tokens, target, vocab, out, mean ? 1 : 0,
                                         ms.slots, ms.epoch, stream);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  note_launch("xent_stats_merge_kernel grid %lld x %d",
              (long long)((tokens + lce::kRowThreads - 1) / lce::kRowThreads), lce::kRowThreads);
  return LCE_OK;
}

// The row gradient for a call whose logits, target and reduction are already
// validated (tokens > 0); with `out` also the forward's losses (or their mean).
static lce_status run_xent_bwd(const void* logits, lce_dtype dtype, int64_t tokens, int64_t vocab,
                               const int64_t* target, bool mean, const float* grad, void* dlogits,
                               float* out, hipStream_t stream) {
  lce_status s = LCE_OK;
  const int64_t esize = dtype == LCE_F32 ? 4 : 2;
  if (!grad) return fail(LCE_ERR_INVALID_ARG, "grad is NULL");
  if (!dlogits) return fail(LCE_ERR_INVALID_ARG, "dlogits is NULL");
  if (!aligned(grad, 4)) return fail(LCE_ERR_INVALID_ARG, "grad is not 4-byte aligned");
  if (!aligned(dlogits, (uint64_t)esize))
    return fail(LCE_ERR_INVALID_ARG, "dlogits is not aligned to its element size");
  // Each row is cut into scalar edges and 16-byte chunks by the logits' address;
  // the gradient rows are written with the same cut.
  if (((uintptr_t)dlogits - (uintptr_t)logits) % 16u != 0)
    return fail(LCE_ERR_UNSUPPORTED, "dlogits must start at the same offset modulo 16 bytes as logits");
  const uint64_t zb = (uint64_t)(tokens * vocab * esize);
  const uint64_t gb = mean ? 4u : (uint64_t)tokens * 4u;
  // In place (dlogits == logits) is allowed; any other overlap is not.
  if (dlogits != logits && overlaps(dlogits, zb, logits, zb))
    return fail(LCE_ERR_ALIAS, "dlogits overlaps logits without being the same buffer");
  if (overlaps(dlogits, zb, target, (uint64_t)tokens * 8u))
    return fail(LCE_ERR_ALIAS, "dlogits overlaps target");
  if (overlaps(dlogits, zb, grad, gb)) return fail(LCE_ERR_ALIAS, "dlogits overlaps grad");
  if (out) {
    const uint64_t ob = out_bytes(tokens, mean ? LCE_REDUCTION_MEAN : LCE_REDUCTION_NONE);
    if (overlaps(out, ob, dlogits, zb)) return fail(LCE_ERR_ALIAS, "out overlaps dlogits");
    if (overlaps(out, ob, grad, gb)) return fail(LCE_ERR_ALIAS, "out overlaps grad");
  }

  lce::BwdArgs a{};
  a.logits = logits;
  a.bf16 = dtype == LCE_BF16;
  a.tokens = tokens;
  a.vocab = vocab;
  a.target = target;
  a.grad = grad;
  a.reduce_mean = mean ? 1 : 0;
  a.dlogits = dlogits;
  // Rows of at most 32 chunks per lane stay in one wave's registers (read once,
  // written once); longer rows take the row states from a statistics pass first.
  // Rows of one or two chunks per lane hold exactly that many (with 4, most of
  // the loads would fall past the row: bf16 [65536, 512] mean 54.3 -> 30.4 us,
  // fp32 [65536, 256] 34.5 -> 26.6 us).
  const int64_t nvec = vocab * esize / 16;
  const int64_t per_lane = (nvec + 63) / 64;
  a.wave_chunks = per_lane <= 1   ? 1
                  : per_lane <= 2  ? 2
                  : per_lane <= 4  ? 4
                  : per_lane <= 8  ? 8
                  : per_lane <= 16 ? 16
                  : per_lane <= 32 ? 32
                                   : 0;
  const char* forced = getenv("LCE_BWD_PATH");
  if (forced && !strcmp(forced, "apply")) a.wave_chunks = 0;
  // Rows of at most 128 chunks with no scalar edges: several rows per wave, as
  // in the forward (LCE_BWD_PATH=wave keeps one wave per row).
  const bool edgeless = (vocab * esize) % 16 == 0 && ((uintptr_t)logits % 16) == 0;
  if (a.wave_chunks > 0 && a.wave_chunks <= 2 && edgeless && !(forced && !strcmp(forced, "wave")))
    a.rows_per_wave = nvec <= 32 ? 8 : nvec <= 64 ? 4 : 2;
  MeanState ms;
  if (a.wave_chunks == 0) {
    int cus = 0;
    if ((s = num_cus(&cus)) != LCE_OK) return s;
    int64_t S = (4 * (int64_t)cus + tokens - 1) / tokens;
    const int64_t max_s = (nvec + lce::kRowThreads * 4 - 1) / (lce::kRowThreads * 4);
    if (S > max_s) S = max_s;
    const int64_t min_s = (nvec * 16 + kMaxStreamBytes - 1) / kMaxStreamBytes;
    if (S < min_s) S = min_s;
    if (S < 1) S = 1;
    if (!lce::grid_fits(S * tokens, lce::kRowThreads))
      return fail(LCE_ERR_UNSUPPORTED, "tokens * slices * 256 work-items must be < 2^32 (got %lld slices)",
                  (long long)(S * tokens));
    a.splits = (int)S;
    a.chunks_per_split = (int)((nvec + S - 1) / S);
    // Row states (m, sum e^(z - m), z_target) into scratch, then the gradient
    // pass; the losses (with `out`) come from the same states.
    Carve cv;
    const size_t off_stats = cv.take((size_t)tokens * 12u);
    char* base = nullptr;
    if ((s = get_scratch(stream, cv.off, &base)) != LCE_OK) return s;
    float* stats = (float*)(base + off_stats);
    if ((s = run_rows(logits, (int)dtype, tokens, vocab, target, false, nullptr, 0, stats, stream,
                      (size_t)tokens * 12u)) != LCE_OK)
      return s;
    a.stats = stats;
    if (out) {
      if (mean && (s = get_mean_state(stream, (tokens + lce::kRowThreads - 1) / lce::kRowThreads, &ms)) != LCE_OK)
        return s;
      hipError_t e = lce::launch_stats_merge(stats, 1, tokens, target, vocab, out, mean ? 1 : 0, ms.slots,
                                             ms.epoch, stream);
      if (e != hipSuccess) return hip_fail(e, "kernel launch");
      note_launch("xent_stats_merge_kernel grid %lld x %d",
                  (long long)((tokens + lce::kRowThreads - 1) / lce::kRowThreads), lce::kRowThreads);
    }
  } else if (out) {
    a.loss_out = out;
    const int rows = a.rows_per_wave ? 4 * a.rows_per_wave : lce::bwd_wave_rows(a);
    if (mean && (s = get_mean_state(stream, (tokens + rows - 1) / rows, &ms)) != LCE_OK) return s;
    a.mean_slots = ms.slots;
    a.epoch = ms.epoch;
  }
  hipError_t e = lce::launch_bwd(a, stream);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  const char* tn = a.bf16 ? "unsigned short" : "float";
  if (a.rows_per_wave) {
    note_launch("xent_bwd_group_kernel<%s, %d, 4, 4, %s> grid %lld x 256", tn, a.rows_per_wave,
                out ? "true" : "false", (long long)((tokens + 4 * a.rows_per_wave - 1) / (4 * a.rows_per_wave)));
  } else if (a.wave_chunks > 0) {
    const int rows = lce::bwd_wave_rows(a);
    note_launch("xent_bwd_wave_kernel<%s, %d, %d, %s> grid %lld x %d", tn, a.wave_chunks, rows,
                out ? "true" : "false", (long long)((tokens + rows - 1) / rows), 64 * rows);
  }
  else
    note_launch("xent_bwd_apply_kernel<%s, 4> grid %lld x %d", tn, (long long)(a.splits * tokens),
                lce::kRowThreads);
  return LCE_OK;
}

lce_status lce_xent_bwd(const void* logits, lce_dtype dtype, int64_t tokens, int64_t vocab,
                        const int64_t* target, lce_reduction reduction, const float* grad,
                        void* dlogits, hipStream_t stream) {
  begin_call();
  lce_status s = validate_xent(logits, (int)dtype, tokens, vocab, target, LCE_REDUCTION_NONE, nullptr,
                               nullptr);
  if (s != LCE_OK) return s;
  if (reduction != LCE_REDUCTION_MEAN && reduction != LCE_REDUCTION_NONE)
    return fail(LCE_ERR_INVALID_ARG, "reduction must be LCE_REDUCTION_MEAN or LCE_REDUCTION_NONE (got %d)",
                (int)reduction);
  if (tokens == 0) return LCE_OK;
  return run_xent_bwd(logits, dtype, tokens, vocab, target, reduction == LCE_REDUCTION_MEAN, grad,
                      dlogits, nullptr, stream);
}

lce_status lce_xent_fwd_bwd(const void* logits, lce_dtype dtype, int64_t tokens, int64_t vocab,
                            const int64_t* target, lce_reduction reduction, const float* grad,
                            float* out, void* dlogits, hipStream_t stream) {
  begin_call();
  lce_status s = validate_xent(logits, (int)dtype, tokens, vocab, target, (int)reduction, out);
  if (s != LCE_OK) return s;
  const bool mean = reduction == LCE_REDUCTION_MEAN;
  if (tokens == 0) {
    if (!mean) return LCE_OK;
    hipError_t e = lce::launch_fill_f32(out, 1, __builtin_nanf(""), stream);
    return e == hipSuccess ? LCE_OK : hip_fail(e, "launch");
  }
  return run_xent_bwd(logits, dtype, tokens, vocab, target, mean, grad, dlogits, out, stream);
}

lce_status lce_fused_linear_xent_fwd(const void* x, const void* weight, int64_t tokens,
                                     int64_t hidden, int64_t vocab, const int64_t* target,
                                     lce_reduction reduction, float* out, hipStream_t stream) {
  begin_call();
  lce_status s = validate_fused(x, weight, tokens, hidden, vocab, target, (int)reduction, out);
  if (s != LCE_OK) return s;
  const bool mean = reduction == LCE_REDUCTION_MEAN;
  if (tokens == 0) {
    if (!mean) return LCE_OK;
    hipError_t e = lce::launch_fill_f32(out, 1, __builtin_nanf(""), stream);
    return e == hipSuccess ? LCE_OK : hip_fail(e, "launch");
  }
  return run_fused(x, weight, tokens, hidden, vocab, target, mean, out, stream);
}

lce_status lce_fused_linear_logprob_sums(const void* x, const void* weight, int64_t batch,
                                         int64_t seq, int64_t hidden, int64_t vocab,
                                         const int64_t* target, float* out, hipStream_t stream) {
  begin_call();
  if (batch < 0 || seq < 0)
    return fail(LCE_ERR_INVALID_ARG, "batch and seq must be >= 0 (got %lld, %lld)", (long long)batch,
                (long long)seq);
  if (seq > 0 && batch > INT64_MAX / seq) return fail(LCE_ERR_INVALID_ARG, "batch * seq overflows");
  const int64_t tokens = batch * seq;
  // Same checks as the fused call with per-token output; out holds `batch` floats.
  if (batch > 0 && !out) return fail(LCE_ERR_INVALID_ARG, "out is NULL");
  lce_status s = validate_fused(x, weight, tokens, hidden, vocab, target, LCE_REDUCTION_NONE,
                                batch > 0 ? out : nullptr, batch);
  if (s != LCE_OK) return s;
  if (batch == 0) return LCE_OK;
  if (seq == 0) {  // empty sequences: a sum of nothing
    hipError_t e = lce::launch_fill_f32(out, batch, 0.0f, stream);
    return e == hipSuccess ? LCE_OK : hip_fail(e, "launch");
  }
  // Per-token losses into the front of scratch, then one wave per sequence.
  Carve cv;
  const size_t off_loss = cv.take((size_t)tokens * 4u);
  char* base = nullptr;
  if ((s = get_scratch(stream, cv.off, &base)) != LCE_OK) return s;
  float* loss = (float*)(base + off_loss);
  if ((s = run_fused(x, weight, tokens, hidden, vocab, target, false, loss, stream,
                     (size_t)tokens * 4u)) != LCE_OK)
    return s;
  hipError_t e = lce::launch_seq_logprob_sums(loss, batch, seq, out, stream);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  note_launch("seq_logprob_sum_kernel grid %lld x %d", (long long)((batch + 3) / 4), lce::kRowThreads);
  return LCE_OK;
}
}  // extern "C"
