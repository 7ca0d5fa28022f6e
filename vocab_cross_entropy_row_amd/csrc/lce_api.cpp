// liblce host API: argument validation, path selection, scratch management
// and error reporting.  Every entry point validates its arguments on the host
// before it makes any HIP call, so argument errors never touch the device.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <vector>
#include <mutex>
#include <string>
#include <tuple>
#include <utility>

#include "fused_grad.h"
#include "lce.h"
#include "lce_internal.h"

namespace {

thread_local std::string g_last_error;

lce_status fail(lce_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

lce_status hip_fail(hipError_t e, const char* what) {
  return fail(LCE_ERR_HIP, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
}

// [a, a + an) and [b, b + bn) overlap (byte ranges).
bool overlaps(const void* a, uint64_t an, const void* b, uint64_t bn) {
  if (!a || !b || an == 0 || bn == 0) return false;
  const uint64_t a0 = (uint64_t)(uintptr_t)a, b0 = (uint64_t)(uintptr_t)b;
  return a0 < b0 + bn && b0 < a0 + an;
}

bool aligned(const void* p, uint64_t n) { return ((uintptr_t)p % n) == 0; }

// ------------------------------------------------------------ scratch pool
// One grow-only device buffer per (device, stream).  A buffer that is outgrown
// is retired, not freed: launches already queued, or recorded into a HIP graph
// that may be replayed later, keep pointing at it.  Every buffer lives until
// process exit.  Layout: the mean's ticket counters first (kTicketBytes, zero
// between calls), then 256-byte-aligned regions carved by Carve.
struct Scratch {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, Scratch> g_scratch;
std::vector<void*> g_retired;
std::map<int, int> g_num_cus;

constexpr size_t kAlign = 256;
// Most bytes one kernel streams through a single buffer resource (32-bit
// offsets, with room for the batch loaded past the end).
constexpr int64_t kMaxStreamBytes = int64_t(1) << 30;
size_t round_up(size_t n, size_t a) { return (n + a - 1) / a * a; }

struct Carve {
  size_t off = round_up(lce::kTicketBytes, kAlign);  // the ticket counters come first
  size_t take(size_t n) {
    const size_t o = off;
    off = round_up(off + n, kAlign);
    return o;
  }
};

lce_status get_scratch(hipStream_t stream, size_t need, char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_mu);
  Scratch& s = g_scratch[{dev, stream}];
  if (s.bytes < need) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
    if (cap != hipStreamCaptureStatusNone)
      return fail(LCE_ERR_UNSUPPORTED,
                  "stream is being captured and its scratch must grow to %zu bytes: make one call "
                  "of the largest shape on this stream before capture", need);
    if (getenv("LCE_TEST_FAIL_ALLOC")) return fail(LCE_ERR_OOM, "scratch allocation refused (LCE_TEST_FAIL_ALLOC)");
    const size_t bytes = round_up(need + need / 4, size_t(1) << 20);
    void* p = nullptr;
    e = hipMalloc(&p, bytes);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(LCE_ERR_OOM, "hipMalloc of %zu bytes of scratch failed: %s", bytes, hipGetErrorName(e));
    }
    // Ticket counters, epoch and mean slots must start at zero (kernels leave
    // the counters at zero; a slot only ever holds tags of earlier launches).
    e = lce::launch_zero_u32((unsigned*)p, (int64_t)(bytes / sizeof(unsigned)), stream);
    if (e != hipSuccess) {
      (void)hipFree(p);
      return hip_fail(e, "scratch initialisation");
    }
    if (s.ptr) g_retired.push_back(s.ptr);
    s.ptr = p;
    s.bytes = bytes;
  }
  *out = (char*)s.ptr;
  return LCE_OK;
}

lce_status num_cus(int* n) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_mu);
  auto it = g_num_cus.find(dev);
  if (it == g_num_cus.end()) {
    int v = 0;
    e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    it = g_num_cus.emplace(dev, v > 0 ? v : 1).first;
  }
  *n = it->second;
  return LCE_OK;
}

int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return (v && *v) ? atoi(v) : dflt;
}

int64_t env_int64(const char* name, int64_t dflt) {
  const char* v = getenv(name);
  return (v && *v) ? (int64_t)strtoll(v, nullptr, 10) : dflt;
}

// ------------------------------------------------------------ validation (host only)
lce_status validate_common(int64_t tokens, const int64_t* target, int reduction, const float* out,
                           const char* out_name = "out", bool has_target = true) {
  if (reduction != LCE_REDUCTION_MEAN && reduction != LCE_REDUCTION_NONE)
    return fail(LCE_ERR_INVALID_ARG, "reduction must be LCE_REDUCTION_MEAN or LCE_REDUCTION_NONE (got %d)", reduction);
  if (tokens < 0) return fail(LCE_ERR_INVALID_ARG, "tokens must be >= 0 (got %lld)", (long long)tokens);
  if (tokens >= (int64_t(1) << 32) - 1)
    return fail(LCE_ERR_UNSUPPORTED, "tokens must be < 2^32 - 1 (got %lld)", (long long)tokens);
  // out_name == nullptr: the caller checks its own output.
  const bool writes = out_name && (reduction == LCE_REDUCTION_MEAN || tokens > 0);
  if (writes && !out) return fail(LCE_ERR_INVALID_ARG, "%s is NULL", out_name);
  if (has_target && tokens > 0 && !target) return fail(LCE_ERR_INVALID_ARG, "target is NULL");
  if (target && !aligned(target, 8)) return fail(LCE_ERR_INVALID_ARG, "target is not 8-byte aligned");
  if (out && !aligned(out, 4)) return fail(LCE_ERR_INVALID_ARG, "%s is not 4-byte aligned", out_name);
  return LCE_OK;
}

uint64_t out_bytes(int64_t tokens, int reduction) {
  return reduction == LCE_REDUCTION_MEAN ? 4u : (uint64_t)tokens * 4u;
}

// `out_elems` fp32 outputs per token (1, or 3 for shard statistics).
lce_status validate_xent(const void* logits, int dtype, int64_t tokens, int64_t vocab,
                         const int64_t* target, int reduction, const float* out,
                         const char* out_name = "out", int out_elems = 1) {
  if (dtype != LCE_F32 && dtype != LCE_BF16)
    return fail(LCE_ERR_INVALID_ARG, "dtype must be LCE_F32 or LCE_BF16 (got %d)", dtype);
  lce_status s = validate_common(tokens, target, reduction, out, out_name);
  if (s != LCE_OK) return s;
  if (vocab < 1) return fail(LCE_ERR_INVALID_ARG, "vocab must be >= 1 (got %lld)", (long long)vocab);
  if (vocab >= (int64_t(1) << 31))
    return fail(LCE_ERR_UNSUPPORTED, "vocab must be < 2^31 (got %lld)", (long long)vocab);
  const int64_t esize = dtype == LCE_F32 ? 4 : 2;
  if (tokens > 0 && !logits) return fail(LCE_ERR_INVALID_ARG, "logits is NULL");
  if (tokens > INT64_MAX / (vocab * esize))
    return fail(LCE_ERR_INVALID_ARG, "tokens * vocab overflows");
  if (logits && !aligned(logits, (uint64_t)esize))
    return fail(LCE_ERR_INVALID_ARG, "logits is not aligned to its element size");
  if (!out_name) return LCE_OK;
  const uint64_t ob = out_bytes(tokens, reduction) * (uint64_t)out_elems;
  if (overlaps(out, ob, logits, (uint64_t)(tokens * vocab * esize)))
    return fail(LCE_ERR_ALIAS, "%s overlaps logits", out_name);
  if (overlaps(out, ob, target, (uint64_t)tokens * 8u))
    return fail(LCE_ERR_ALIAS, "%s overlaps target", out_name);
  return LCE_OK;
}

// `out_floats` >= 0 overrides the output size implied by the reduction.
// One bf16 projection: activations x [tokens, hidden] and head w [vocab, hidden],
// against an output of `ob` bytes.
lce_status validate_head(const void* x, const void* w, int64_t tokens, int64_t hidden, int64_t vocab,
                         const float* out, uint64_t ob, const char* xn = "x",
                         const char* wn = "weight") {
  if (hidden < 1) return fail(LCE_ERR_INVALID_ARG, "hidden must be >= 1 (got %lld)", (long long)hidden);
  if (vocab < 1) return fail(LCE_ERR_INVALID_ARG, "vocab must be >= 1 (got %lld)", (long long)vocab);
  if (vocab >= (int64_t(1) << 31))
    return fail(LCE_ERR_UNSUPPORTED, "vocab must be < 2^31 (got %lld)", (long long)vocab);
  // The kernels address a tile of up to 256 rows through one buffer resource
  // with 32-bit offsets, and mark a slab past the end of a row with an offset
  // of 0x7ffffff0: 256 rows * 2 bytes * hidden must stay below it.
  if (hidden >= (int64_t(1) << 22))
    return fail(LCE_ERR_UNSUPPORTED, "hidden must be < 2^22 (got %lld)", (long long)hidden);
  if (!w) return fail(LCE_ERR_INVALID_ARG, "%s is NULL", wn);
  if (tokens > 0 && !x) return fail(LCE_ERR_INVALID_ARG, "%s is NULL", xn);
  if (hidden % 8 != 0)
    return fail(LCE_ERR_UNSUPPORTED, "hidden must be a multiple of 8 (got %lld)", (long long)hidden);
  if (!aligned(w, 16) || (x && !aligned(x, 16)))
    return fail(LCE_ERR_UNSUPPORTED, "%s and %s must be 16-byte aligned", xn, wn);
  if (vocab > INT64_MAX / (hidden * 2) || tokens > INT64_MAX / (hidden * 2))
    return fail(LCE_ERR_INVALID_ARG, "tensor size overflows");
  if (overlaps(out, ob, x, (uint64_t)(tokens * hidden * 2))) return fail(LCE_ERR_ALIAS, "out overlaps %s", xn);
  if (overlaps(out, ob, w, (uint64_t)(vocab * hidden * 2))) return fail(LCE_ERR_ALIAS, "out overlaps %s", wn);
  return LCE_OK;
}

lce_status validate_fused(const void* x, const void* w, int64_t tokens, int64_t hidden, int64_t vocab,
                          const int64_t* target, int reduction, const float* out,
                          int64_t out_floats = -1) {
  lce_status s = validate_common(tokens, target, reduction, out);
  if (s != LCE_OK) return s;
  uint64_t ob = out_bytes(tokens, reduction);
  if (out_floats >= 0) ob = (uint64_t)out_floats * 4u;
  if ((s = validate_head(x, w, tokens, hidden, vocab, out, ob)) != LCE_OK) return s;
  if (overlaps(out, ob, target, (uint64_t)tokens * 8u)) return fail(LCE_ERR_ALIAS, "out overlaps target");
  return LCE_OK;
}

// Row kernels for `tokens` rows of `vocab` columns: per-token losses or their
// mean into `out`, or (stats != nullptr) per-row vocab-shard statistics, with
// targets read relative to `vocab_start`.  Arguments are validated; tokens > 0.
// The first `reserved` bytes of scratch regions belong to the caller.
lce_status run_rows(const void* logits, int dtype, int64_t tokens, int64_t vocab,
                    const int64_t* target, bool mean, float* out, int64_t vocab_start,
                    float* stats, hipStream_t stream, size_t reserved = 0) {
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
  //  - rows up to 32 KiB: one wave per row; 4 waves per workgroup without a
  //    mean, 16 with a mean (a quarter of the ticket hand-offs);
  //  - longer rows: without a mean, one workgroup per row; with a mean, one
  //    wave per row in 16-wave workgroups; with few rows, several workgroups
  //    per row (split).
  const int64_t esize = a.bf16 ? 2 : 4;
  const int64_t row_bytes = vocab * esize;
  const int64_t nvec = row_bytes / 16;
  // Chunks per lane per batch (two batches are in flight at once).
  const int64_t per_lane = (nvec + 63) / 64;
  a.unroll = per_lane <= 4 ? 4 : 8;
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
  // Overrides for tuning and tests.
  const char* forced = getenv("LCE_PATH");
  if (forced && !strcmp(forced, "wave")) a.path = lce::XentPath::WaveRows;
  else if (forced && !strcmp(forced, "block")) a.path = lce::XentPath::BlockRows;
  else if (forced && !strcmp(forced, "split")) a.path = lce::XentPath::Split;
  const int forced_unroll = env_int("LCE_UNROLL", 0);
  if (forced_unroll == 4 || forced_unroll == 8 || forced_unroll == 16) a.unroll = forced_unroll;
  const int forced_waves = env_int("LCE_WAVES_PER_BLOCK", 0);
  if (forced_waves == 4 || forced_waves == 16) a.waves_per_block = forced_waves;
  if (a.waves_per_block == 16 && a.unroll > 8) a.unroll = 8;
  // The kernels address a row (or a split slice) with 32-bit buffer offsets.
  if (a.path != lce::XentPath::Split && row_bytes > kMaxStreamBytes) a.path = lce::XentPath::Split;

  size_t need_partials = 0, need_split = 0;
  if (a.path == lce::XentPath::Split) {
    if (tokens > 65535) return fail(LCE_ERR_UNSUPPORTED, "split path needs tokens <= 65535");
    // Enough workgroups for ~4 per CU, but at least one 256-thread batch of 8
    // chunks per workgroup.
    int64_t S = env_int("LCE_SPLITS", 0);
    if (S <= 0) S = (4 * (int64_t)cus + tokens - 1) / tokens;
    const int64_t max_s = (nvec + lce::kRowThreads * 8 - 1) / (lce::kRowThreads * 8);
    if (S > max_s) S = max_s;
    if (S < 1) S = 1;
    if (S > 65535) S = 65535;
    const int64_t min_s = (nvec * 16 + kMaxStreamBytes - 1) / kMaxStreamBytes;
    if (S < min_s) S = min_s;
    a.splits = (int)S;
    a.chunks_per_split = (int)((nvec + S - 1) / S);
    need_split = (size_t)tokens * (size_t)S * 8u;
  }
  const int64_t mean_blocks =
      (a.path == lce::XentPath::BlockRows) ? tokens
      : (a.path == lce::XentPath::WaveRows) ? (tokens + a.waves_per_block - 1) / a.waves_per_block
                                              : (tokens + lce::kRowThreads / 64 - 1) / (lce::kRowThreads / 64);
  need_partials = (size_t)mean_blocks * 8u;

  Carve cv;
  if (reserved) cv.take(reserved);
  const size_t off_mean = cv.take(need_partials);
  const size_t off_split = cv.take(need_split);
  char* base = nullptr;
  if ((s = get_scratch(stream, cv.off, &base)) != LCE_OK) return s;
  a.ticket = (unsigned*)base;
  a.mean_slots = (uint64_t*)(base + off_mean);
  a.split_partials = (float*)(base + off_split);

  hipError_t e = lce::launch_xent(a, stream);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return LCE_OK;
}

// Scratch plan of the fused projection + cross-entropy: vocab segments and the
// offsets of its regions after the caller's `reserved` bytes.
struct FusedPlan {
  int segments = 1;
  size_t off_seg = 0, off_zt = 0, off_mean = 0, end = 0;
};

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
  p.off_mean = cv.take((size_t)((tokens + lce::kRowThreads - 1) / lce::kRowThreads) * 8u);
  p.end = cv.off;
  return p;
}

// The fused projection + cross-entropy for validated arguments, tokens > 0.
// The first `reserved` bytes of scratch regions belong to the caller.  With
// lse_out set, writes ln sum_j e^(z_j) per token there instead of losses
// (target and out are then unused).  With z_out set, the logits are also
// stored there as [tokens, z_ld] fp32 rows.
lce_status run_fused(const void* x, const void* weight, int64_t tokens, int64_t hidden, int64_t vocab,
                     const int64_t* target, bool mean, float* out, hipStream_t stream,
                     size_t reserved = 0, float* lse_out = nullptr, float* z_out = nullptr,
                     int64_t z_ld = 0) {
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
  a.target = lse_out ? nullptr : target;
  a.out = lse_out ? nullptr : out;
  a.lse_out = lse_out;
  a.z_out = z_out;
  a.z_ld = z_ld;
  a.reduce_mean = (mean && !lse_out) ? 1 : 0;
  a.segments = p.segments;

  char* base = nullptr;
  if ((s = get_scratch(stream, p.end, &base)) != LCE_OK) return s;
  a.ticket = (unsigned*)base;
  a.seg_partials = (float*)(base + p.off_seg);
  a.target_logit = (float*)(base + p.off_zt);
  a.mean_slots = (uint64_t*)(base + p.off_mean);

  hipError_t e = lce::launch_fused(a, stream);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return LCE_OK;
}

// ------------------------------------------------------------ library GEMMs
// The two plain products of the fused-projection backward (dx = dZ W and
// dW = dZ^T x) go to hipBLASLt: bf16 operands, fp32 accumulation and output.
// One handle per device and one plan (descriptors, layouts and the heuristic's
// first algorithm) per GEMM shape, created on first use and kept for the
// process's lifetime.
struct GemmPlan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t a = nullptr, b = nullptr, d = nullptr;
  hipblasLtMatmulAlgo_t algo{};
  size_t ws = 0;
};
typedef std::tuple<int, int, int, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, size_t>
    GemmKey;
std::map<int, hipblasLtHandle_t> g_blaslt;
std::map<GemmKey, GemmPlan> g_gemm_plans;

lce_status blas_fail(hipblasStatus_t st, const char* what) {
  return fail(LCE_ERR_HIP, "hipBLASLt %s failed (status %d)", what, (int)st);
}

// D (fp32, column-major m x n, leading dimension ldd) = op(A) op(B) + beta D
// with bf16 A and B (column-major, op N or T).  `ws` is device workspace.
lce_status gemm_bf16_f32(hipblasOperation_t ta, hipblasOperation_t tb, int64_t m, int64_t n,
                         int64_t k, const void* A, int64_t lda, const void* B, int64_t ldb,
                         float beta, float* D, int64_t ldd, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  hipblasLtHandle_t h = nullptr;
  GemmPlan plan;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    const GemmKey key{dev, (int)ta, (int)tb, m, n, k, lda, ldb, ldd, ws_bytes};
    auto hit = g_gemm_plans.find(key);
    if (hit != g_gemm_plans.end()) {
      plan = hit->second;
      h = g_blaslt[dev];
    } else {
      // Creating a handle or a plan is not allowed inside a graph capture.
      hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
      e = hipStreamIsCapturing(stream, &cap);
      if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
      if (cap != hipStreamCaptureStatusNone)
        return fail(LCE_ERR_UNSUPPORTED,
                    "stream is being captured and this GEMM shape has not been planned yet: make "
                    "one call of the same shape on this device before capture");
      hipblasStatus_t st = HIPBLAS_STATUS_SUCCESS;
      auto it = g_blaslt.find(dev);
      if (it == g_blaslt.end()) {
        if ((st = hipblasLtCreate(&h)) != HIPBLAS_STATUS_SUCCESS) return blas_fail(st, "handle creation");
        g_blaslt[dev] = h;
      } else {
        h = it->second;
      }
      if ((st = hipblasLtMatmulDescCreate(&plan.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F)) != HIPBLAS_STATUS_SUCCESS)
        return blas_fail(st, "descriptor creation");
      const int32_t opa = (int32_t)ta, opb = (int32_t)tb;
      hipblasLtMatmulDescSetAttribute(plan.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opa, sizeof opa);
      hipblasLtMatmulDescSetAttribute(plan.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opb, sizeof opb);
      const bool an = ta == HIPBLAS_OP_N, bn = tb == HIPBLAS_OP_N;
      if ((st = hipblasLtMatrixLayoutCreate(&plan.a, HIP_R_16BF, an ? m : k, an ? k : m, lda)) != HIPBLAS_STATUS_SUCCESS ||
          (st = hipblasLtMatrixLayoutCreate(&plan.b, HIP_R_16BF, bn ? k : n, bn ? n : k, ldb)) != HIPBLAS_STATUS_SUCCESS ||
          (st = hipblasLtMatrixLayoutCreate(&plan.d, HIP_R_32F, m, n, ldd)) != HIPBLAS_STATUS_SUCCESS)
        return blas_fail(st, "layout creation");
      hipblasLtMatmulPreference_t pref = nullptr;
      if ((st = hipblasLtMatmulPreferenceCreate(&pref)) != HIPBLAS_STATUS_SUCCESS)
        return blas_fail(st, "preference creation");
      const uint64_t wsb = ws_bytes;
      hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb, sizeof wsb);
      hipblasLtMatmulHeuristicResult_t res[1];
      int found = 0;
      st = hipblasLtMatmulAlgoGetHeuristic(h, plan.desc, plan.a, plan.b, plan.d, plan.d, pref, 1, res, &found);
      hipblasLtMatmulPreferenceDestroy(pref);
      if (st != HIPBLAS_STATUS_SUCCESS || found < 1)
        return fail(LCE_ERR_UNSUPPORTED, "hipBLASLt has no algorithm for a %lld x %lld x %lld GEMM (status %d)",
                    (long long)m, (long long)n, (long long)k, (int)st);
      plan.algo = res[0].algo;
      plan.ws = res[0].workspaceSize;
      g_gemm_plans[key] = plan;
    }
  }
  const float alpha = 1.0f;
  hipblasStatus_t st = hipblasLtMatmul(h, plan.desc, &alpha, A, plan.a, B, plan.b, &beta, D, plan.d,
                                       D, plan.d, &plan.algo, ws, plan.ws, stream);
  if (st != HIPBLAS_STATUS_SUCCESS) return blas_fail(st, "matmul");
  return LCE_OK;
}

// Gradients of the fused projection + cross-entropy, for chunks of tokens.
// Stored path (default): the forward kernel's store mode gives each chunk's
// log-sum-exp and writes its fp32 logits [chunk, ld] into scratch, then
// fused_grad_rows_kernel turns them into the bf16 logit gradient dZ [chunk,
// ld].  Recompute path (when not even 256 tokens of fp32 logits and dZ fit):
// the forward kernel gives every token's log-sum-exp, then for each chunk
// the fused kernel's gradient mode recomputes the logits and writes dZ.
// Either way two library GEMMs consume dZ: dx[chunk] = dZ W and
// dW (+)= dZ^T x[chunk].  Chunks are the largest multiple of 256 tokens whose
// buffers (6 or 2 bytes per logit) fit in LCE_FUSED_BWD_STORE_BYTES (default
// 2 GiB), at least 256.
constexpr size_t kGemmWorkspace = size_t(128) << 20;

lce_status run_fused_bwd(const void* x, const void* weight, int64_t tokens, int64_t hidden,
                         int64_t vocab, const int64_t* target, bool mean, const float* grad,
                         float* dx, float* dw, hipStream_t stream) {
  lce_status s = LCE_OK;
  int cus = 0;
  if ((s = num_cus(&cus)) != LCE_OK) return s;
  const lce::FusedGeometry geo = lce::fused_geometry();
  const int64_t ld = (vocab + geo.block_vocab - 1) / geo.block_vocab * geo.block_vocab;
  const int64_t cap = env_int64("LCE_FUSED_BWD_STORE_BYTES", int64_t(2) << 30);
  const bool stored = cap / (ld * 6) >= geo.block_tokens;
  int64_t chunk = cap / (ld * (stored ? 6 : 2)) / geo.block_tokens * geo.block_tokens;
  if (chunk < geo.block_tokens) chunk = geo.block_tokens;
  if (chunk > tokens) chunk = tokens;

  Carve cv;
  const size_t off_lse = cv.take((size_t)tokens * 4u);
  const size_t off_ws = cv.take(kGemmWorkspace);
  const size_t off_dz = cv.take((size_t)chunk * (size_t)ld * 2u);
  const size_t off_z = cv.take(stored ? (size_t)chunk * (size_t)ld * 4u : 0u);
  const size_t reserved = cv.off - Carve().off;
  const int64_t last = tokens - (tokens - 1) / chunk * chunk;
  size_t need = cv.off;
  for (int64_t n : {stored ? chunk : tokens, last}) {
    const FusedPlan fp = plan_fused(n, vocab, cus, reserved);
    if (fp.end > need) need = fp.end;
  }
  char* base = nullptr;
  if ((s = get_scratch(stream, need, &base)) != LCE_OK) return s;
  float* lse = (float*)(base + off_lse);
  void* ws = base + off_ws;
  void* dz = base + off_dz;
  float* z = (float*)(base + off_z);

  if (!stored && (s = run_fused(x, weight, tokens, hidden, vocab, nullptr, false, nullptr, stream,
                                reserved, lse)) != LCE_OK)
    return s;
  const uint16_t* x16 = (const uint16_t*)x;
  for (int64_t c0 = 0; c0 < tokens; c0 += chunk) {
    const int64_t n = tokens - c0 < chunk ? tokens - c0 : chunk;
    hipError_t e = hipSuccess;
    if (stored) {
      if ((s = run_fused(x16 + c0 * hidden, weight, n, hidden, vocab, nullptr, false, nullptr,
                         stream, reserved, lse + c0, z, ld)) != LCE_OK)
        return s;
      lce::FusedGradRowsArgs g{};
      g.z = z;
      g.lse = lse + c0;
      g.target = target + c0;
      g.grad = mean ? grad : grad + c0;
      g.grad_mean = mean ? 1 : 0;
      g.grad_tokens = tokens;
      g.rows = n;
      g.vocab = vocab;
      g.ld = ld;
      g.dz = (uint16_t*)dz;
      e = lce::launch_fused_grad_rows(g, stream);
    } else {
      lce::FusedGradArgs g{};
      g.x = x16 + c0 * hidden;
      g.w = weight;
      g.tokens = n;
      g.hidden = hidden;
      g.vocab = vocab;
      g.target = target + c0;
      g.lse = lse + c0;
      g.grad = mean ? grad : grad + c0;
      g.grad_mean = mean ? 1 : 0;
      g.grad_tokens = tokens;
      g.dz = dz;
      g.dz_ld = ld;
      g.segments = lce::fused_segments(n, vocab, cus);
      e = lce::launch_fused_grad(g, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "kernel launch");
    // Row-major [r, c] is column-major [c, r]: dx^T[H, n] = W^T[H, V] dZ^T[V, n],
    // dW^T[H, V] (+)= x^T[H, n] dZ[n, V].
    if (dx && (s = gemm_bf16_f32(HIPBLAS_OP_N, HIPBLAS_OP_N, hidden, n, vocab, weight, hidden, dz,
                                 ld, 0.0f, dx + c0 * hidden, hidden, ws, kGemmWorkspace,
                                 stream)) != LCE_OK)
      return s;
    if (dw && (s = gemm_bf16_f32(HIPBLAS_OP_N, HIPBLAS_OP_T, hidden, vocab, n, x16 + c0 * hidden,
                                 hidden, dz, ld, c0 == 0 ? 0.0f : 1.0f, dw, hidden, ws,
                                 kGemmWorkspace, stream)) != LCE_OK)
      return s;
  }
  return LCE_OK;
}

// Fused linear + JSD.  Both paths first take each head's per-token
// log-sum-exp with the fused cross-entropy kernel.  The stored path has that
// kernel also write both heads' fp32 logits for a chunk of tokens into scratch
// and then streams them once (jsd_stored_rows_kernel); the recompute path
// multiplies both heads again, tile by tile (fused_jsd_partial_kernel), and
// needs no logit storage.  The stored path is taken when a chunk of at least
// one fused token tile fits in LCE_JSD_STORE_BYTES (default 2 GiB) of scratch.
struct JsdPlan {
  int64_t chunk = 0;  // tokens per chunk; 0: recompute path
  int64_t ld = 0;     // stored row length (vocab rounded up to the fused tile)
};

JsdPlan plan_jsd(int64_t tokens, int64_t vocab) {
  JsdPlan p;
  const lce::FusedGeometry g = lce::fused_geometry();
  const int64_t ld = (vocab + g.block_vocab - 1) / g.block_vocab * g.block_vocab;
  // Byte offsets within a token tile's rows are 32-bit.
  if (ld * g.block_tokens * 4 >= (int64_t(1) << 32)) return p;
  const int64_t cap = env_int64("LCE_JSD_STORE_BYTES", int64_t(2) << 30);
  const int64_t per_token = ld * 8;  // both heads' rows
  int64_t max_chunk = cap / per_token / g.block_tokens * g.block_tokens;
  if (max_chunk < g.block_tokens) return p;
  if (tokens <= max_chunk) {
    p.chunk = tokens;
  } else {
    const int64_t n = (tokens + max_chunk - 1) / max_chunk;
    const int64_t even = (tokens + n - 1) / n;
    p.chunk = (even + g.block_tokens - 1) / g.block_tokens * g.block_tokens;  // <= max_chunk
  }
  p.ld = ld;
  return p;
}

lce_status run_jsd_stored(const void* xs, const void* ws, const void* xt, const void* wt,
                          int64_t tokens, int64_t hidden, int64_t vocab, float beta, bool mean,
                          float* out, hipStream_t stream, int cus, const JsdPlan& plan) {
  lce_status s = LCE_OK;
  Carve cv;
  const size_t off_ls = cv.take((size_t)tokens * 4u);
  const size_t off_lt = cv.take((size_t)tokens * 4u);
  const size_t off_per = cv.take(mean ? (size_t)tokens * 4u : 0u);
  const size_t off_mean = cv.take((size_t)((tokens + lce::kRowThreads - 1) / lce::kRowThreads) * 8u);
  const size_t zbytes = (size_t)plan.chunk * (size_t)plan.ld * 4u;
  const size_t off_zs = cv.take(zbytes);
  const size_t off_zt = cv.take(zbytes);
  const size_t reserved = cv.off - Carve().off;
  // The fused kernel's own regions follow; size them for the largest chunk
  // and for the last (smaller) one, whose plan may differ.
  const int64_t last = tokens - (tokens - 1) / plan.chunk * plan.chunk;
  size_t need = cv.off;
  for (int64_t n : {plan.chunk, last}) {
    const FusedPlan fp = plan_fused(n, vocab, cus, reserved);
    if (fp.end > need) need = fp.end;
  }
  char* base = nullptr;
  if ((s = get_scratch(stream, need, &base)) != LCE_OK) return s;
  float* lse_s = (float*)(base + off_ls);
  float* lse_t = (float*)(base + off_lt);
  float* per = mean ? (float*)(base + off_per) : out;
  float* zs = (float*)(base + off_zs);
  float* zt = (float*)(base + off_zt);

  const uint16_t* xs16 = (const uint16_t*)xs;
  const uint16_t* xt16 = (const uint16_t*)xt;
  for (int64_t c0 = 0; c0 < tokens; c0 += plan.chunk) {
    const int64_t n = tokens - c0 < plan.chunk ? tokens - c0 : plan.chunk;
    if ((s = run_fused(xs16 + c0 * hidden, ws, n, hidden, vocab, nullptr, false, nullptr, stream,
                       reserved, lse_s + c0, zs, plan.ld)) != LCE_OK)
      return s;
    if ((s = run_fused(xt16 + c0 * hidden, wt, n, hidden, vocab, nullptr, false, nullptr, stream,
                       reserved, lse_t + c0, zt, plan.ld)) != LCE_OK)
      return s;
    lce::JsdRowsArgs r{};
    r.zs = zs;
    r.zt = zt;
    r.z_ld = plan.ld;
    r.rows = n;
    r.vocab = vocab;
    r.lse_s = lse_s + c0;
    r.lse_t = lse_t + c0;
    r.beta = beta;
    r.dst = per + c0;
    hipError_t e = lce::launch_jsd_rows(r, stream);
    if (e != hipSuccess) return hip_fail(e, "kernel launch");
  }
  if (mean) {
    hipError_t e = lce::launch_jsd_mean(tokens, per, out, (uint64_t*)(base + off_mean),
                                        (unsigned*)base, stream);
    if (e != hipSuccess) return hip_fail(e, "kernel launch");
  }
  return LCE_OK;
}

lce_status run_jsd_recompute(const void* xs, const void* ws, const void* xt, const void* wt,
                             int64_t tokens, int64_t hidden, int64_t vocab, float beta, bool mean,
                             float* out, hipStream_t stream, int cus) {
  lce_status s = LCE_OK;
  // Scratch: both heads' log-sum-exp, the divergence kernel's per-segment
  // sums and mean slots, then the cross-entropy kernel's own regions.
  lce::JsdArgs a{};
  a.xs = xs;
  a.ws = ws;
  a.xt = xt;
  a.wt = wt;
  a.tokens = tokens;
  a.hidden = hidden;
  a.vocab = vocab;
  a.beta = beta;
  a.out = out;
  a.reduce_mean = mean ? 1 : 0;
  a.segments = lce::jsd_segments(tokens, vocab, cus);
  Carve cv;
  const size_t off_ls = cv.take((size_t)tokens * 4u);
  const size_t off_lt = cv.take((size_t)tokens * 4u);
  const size_t off_part = cv.take((size_t)a.segments * (size_t)tokens * 4u);
  const size_t off_mean = cv.take((size_t)((tokens + lce::kRowThreads - 1) / lce::kRowThreads) * 8u);
  const size_t reserved = cv.off - Carve().off;
  const FusedPlan fp = plan_fused(tokens, vocab, cus, reserved);
  char* base = nullptr;
  if ((s = get_scratch(stream, fp.end > cv.off ? fp.end : cv.off, &base)) != LCE_OK) return s;
  float* lse_s = (float*)(base + off_ls);
  float* lse_t = (float*)(base + off_lt);
  a.lse_s = lse_s;
  a.lse_t = lse_t;
  a.partials = (float*)(base + off_part);
  a.mean_slots = (uint64_t*)(base + off_mean);
  a.ticket = (unsigned*)base;

  if ((s = run_fused(xs, ws, tokens, hidden, vocab, nullptr, false, nullptr, stream, reserved,
                     lse_s)) != LCE_OK)
    return s;
  if ((s = run_fused(xt, wt, tokens, hidden, vocab, nullptr, false, nullptr, stream, reserved,
                     lse_t)) != LCE_OK)
    return s;
  hipError_t e = lce::launch_jsd(a, stream);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return LCE_OK;
}

}  // namespace

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

const char* lce_last_error(void) { return g_last_error.c_str(); }

int lce_version(void) { return LCE_VERSION_MAJOR * 10000 + LCE_VERSION_MINOR * 100 + LCE_VERSION_PATCH; }

lce_status lce_xent_fwd(const void* logits, lce_dtype dtype, int64_t tokens, int64_t vocab,
                        const int64_t* target, lce_reduction reduction, float* out,
                        hipStream_t stream) {
  g_last_error.clear();
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
  g_last_error.clear();
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
  g_last_error.clear();
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
  Carve cv;
  const size_t off_mean = cv.take((size_t)((tokens + lce::kRowThreads - 1) / lce::kRowThreads) * 8u);
  char* base = nullptr;
  if ((s = get_scratch(stream, cv.off, &base)) != LCE_OK) return s;
  hipError_t e = lce::launch_stats_merge(partials, shards, tokens, target, vocab, out, mean ? 1 : 0,
                                         (uint64_t*)(base + off_mean), (unsigned*)base, stream);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return LCE_OK;
}

lce_status lce_xent_bwd(const void* logits, lce_dtype dtype, int64_t tokens, int64_t vocab,
                        const int64_t* target, lce_reduction reduction, const float* grad,
                        void* dlogits, hipStream_t stream) {
  g_last_error.clear();
  lce_status s = validate_xent(logits, (int)dtype, tokens, vocab, target, LCE_REDUCTION_NONE, nullptr,
                               nullptr);
  if (s != LCE_OK) return s;
  if (reduction != LCE_REDUCTION_MEAN && reduction != LCE_REDUCTION_NONE)
    return fail(LCE_ERR_INVALID_ARG, "reduction must be LCE_REDUCTION_MEAN or LCE_REDUCTION_NONE (got %d)",
                (int)reduction);
  if (tokens == 0) return LCE_OK;
  const int64_t esize = dtype == LCE_F32 ? 4 : 2;
  if (!grad) return fail(LCE_ERR_INVALID_ARG, "grad is NULL");
  if (!dlogits) return fail(LCE_ERR_INVALID_ARG, "dlogits is NULL");
  if (!aligned(grad, 4)) return fail(LCE_ERR_INVALID_ARG, "grad is not 4-byte aligned");
  if (!aligned(dlogits, (uint64_t)esize))
    return fail(LCE_ERR_INVALID_ARG, "dlogits is not aligned to its element size");
  const bool mean = reduction == LCE_REDUCTION_MEAN;
  const uint64_t zb = (uint64_t)(tokens * vocab * esize);
  const uint64_t gb = mean ? 4u : (uint64_t)tokens * 4u;
  // In place (dlogits == logits) is allowed; any other overlap is not.
  if (dlogits != logits && overlaps(dlogits, zb, logits, zb))
    return fail(LCE_ERR_ALIAS, "dlogits overlaps logits without being the same buffer");
  if (overlaps(dlogits, zb, target, (uint64_t)tokens * 8u))
    return fail(LCE_ERR_ALIAS, "dlogits overlaps target");
  if (overlaps(dlogits, zb, grad, gb)) return fail(LCE_ERR_ALIAS, "dlogits overlaps grad");

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
  const int64_t nvec = vocab * esize / 16;
  const int64_t per_lane = (nvec + 63) / 64;
  a.wave_chunks = per_lane <= 4 ? 4 : per_lane <= 8 ? 8 : per_lane <= 16 ? 16 : per_lane <= 32 ? 32 : 0;
  const char* forced = getenv("LCE_BWD_PATH");
  if (forced && !strcmp(forced, "apply")) a.wave_chunks = 0;
  if (a.wave_chunks == 0) {
    int cus = 0;
    if ((s = num_cus(&cus)) != LCE_OK) return s;
    int64_t S = (4 * (int64_t)cus + tokens - 1) / tokens;
    const int64_t max_s = (nvec + lce::kRowThreads * 4 - 1) / (lce::kRowThreads * 4);
    if (S > max_s) S = max_s;
    const int64_t min_s = (nvec * 16 + kMaxStreamBytes - 1) / kMaxStreamBytes;
    if (S < min_s) S = min_s;
    if (S < 1) S = 1;
    if (S * tokens >= (int64_t(1) << 31))
      return fail(LCE_ERR_UNSUPPORTED, "tokens * slices must be < 2^31 (got %lld)", (long long)(S * tokens));
    a.splits = (int)S;
    a.chunks_per_split = (int)((nvec + S - 1) / S);
    // Row states (m, sum e^(z - m), .) into scratch, then the gradient pass.
    Carve cv;
    const size_t off_stats = cv.take((size_t)tokens * 12u);
    char* base = nullptr;
    if ((s = get_scratch(stream, cv.off, &base)) != LCE_OK) return s;
    float* stats = (float*)(base + off_stats);
    if ((s = run_rows(logits, (int)dtype, tokens, vocab, target, false, nullptr, 0, stats, stream,
                      (size_t)tokens * 12u)) != LCE_OK)
      return s;
    a.stats = stats;
  }
  hipError_t e = lce::launch_bwd(a, stream);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return LCE_OK;
}

lce_status lce_fused_linear_xent_fwd(const void* x, const void* weight, int64_t tokens,
                                     int64_t hidden, int64_t vocab, const int64_t* target,
                                     lce_reduction reduction, float* out, hipStream_t stream) {
  g_last_error.clear();
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
  g_last_error.clear();
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
  return LCE_OK;
}

lce_status lce_fused_linear_jsd_fwd(const void* student_x, const void* student_weight,
                                    const void* teacher_x, const void* teacher_weight,
                                    int64_t tokens, int64_t hidden, int64_t vocab, float beta,
                                    lce_reduction reduction, float* out, hipStream_t stream) {
  g_last_error.clear();
  lce_status s = validate_common(tokens, nullptr, (int)reduction, out, "out", false);
  if (s != LCE_OK) return s;
  const uint64_t ob = out_bytes(tokens, (int)reduction);
  if ((s = validate_head(student_x, student_weight, tokens, hidden, vocab, out, ob, "student_x",
                         "student_weight")) != LCE_OK)
    return s;
  if ((s = validate_head(teacher_x, teacher_weight, tokens, hidden, vocab, out, ob, "teacher_x",
                         "teacher_weight")) != LCE_OK)
    return s;
  if (!(beta > 0.0f && beta < 1.0f))
    return fail(LCE_ERR_INVALID_ARG, "beta must be in (0, 1) (got %g)", (double)beta);
  const bool mean = reduction == LCE_REDUCTION_MEAN;
  if (tokens == 0) {
    if (!mean) return LCE_OK;
    hipError_t e = lce::launch_fill_f32(out, 1, __builtin_nanf(""), stream);
    return e == hipSuccess ? LCE_OK : hip_fail(e, "launch");
  }
  int cus = 0;
  if ((s = num_cus(&cus)) != LCE_OK) return s;
  const JsdPlan plan = plan_jsd(tokens, vocab);
  if (plan.chunk > 0)
    return run_jsd_stored(student_x, student_weight, teacher_x, teacher_weight, tokens, hidden,
                          vocab, beta, mean, out, stream, cus, plan);
  return run_jsd_recompute(student_x, student_weight, teacher_x, teacher_weight, tokens, hidden,
                           vocab, beta, mean, out, stream, cus);
}

lce_status lce_fused_linear_xent_bwd(const void* x, const void* weight, int64_t tokens,
                                     int64_t hidden, int64_t vocab, const int64_t* target,
                                     lce_reduction reduction, const float* grad, float* dx,
                                     float* dweight, hipStream_t stream) {
  g_last_error.clear();
  lce_status s = validate_common(tokens, target, (int)reduction, nullptr, nullptr);
  if (s != LCE_OK) return s;
  if ((s = validate_head(x, weight, tokens, hidden, vocab, nullptr, 0)) != LCE_OK) return s;
  const bool mean = reduction == LCE_REDUCTION_MEAN;
  if (!dx && !dweight) return fail(LCE_ERR_INVALID_ARG, "dx and dweight are both NULL");
  if (tokens > 0 && !grad) return fail(LCE_ERR_INVALID_ARG, "grad is NULL");
  if (grad && !aligned(grad, 4)) return fail(LCE_ERR_INVALID_ARG, "grad is not 4-byte aligned");
  if ((dx && !aligned(dx, 4)) || (dweight && !aligned(dweight, 4)))
    return fail(LCE_ERR_INVALID_ARG, "dx and dweight must be 4-byte aligned");
  const int64_t ld = (vocab + 255) / 256 * 256;
  if (ld * 256 * 2 >= (int64_t(1) << 32))
    return fail(LCE_ERR_UNSUPPORTED, "vocab must be < 2^23 - 256 for the fused backward (got %lld)",
                (long long)vocab);
  const uint64_t xb = (uint64_t)(tokens * hidden * 2), wb = (uint64_t)(vocab * hidden * 2);
  const uint64_t dxb = dx ? (uint64_t)(tokens * hidden * 4) : 0, dwb = dweight ? (uint64_t)(vocab * hidden * 4) : 0;
  const uint64_t gb = mean ? 4u : (uint64_t)tokens * 4u, tb = (uint64_t)tokens * 8u;
  const struct { const void* p; uint64_t n; const char* name; } outs[2] = {{dx, dxb, "dx"}, {dweight, dwb, "dweight"}};
  for (const auto& o : outs) {
    if (!o.p) continue;
    if (overlaps(o.p, o.n, x, xb)) return fail(LCE_ERR_ALIAS, "%s overlaps x", o.name);
    if (overlaps(o.p, o.n, weight, wb)) return fail(LCE_ERR_ALIAS, "%s overlaps weight", o.name);
    if (overlaps(o.p, o.n, target, tb)) return fail(LCE_ERR_ALIAS, "%s overlaps target", o.name);
    if (overlaps(o.p, o.n, grad, gb)) return fail(LCE_ERR_ALIAS, "%s overlaps grad", o.name);
  }
  if (overlaps(dx, dxb, dweight, dwb)) return fail(LCE_ERR_ALIAS, "dx overlaps dweight");
  if (tokens == 0) {  // no token contributes: dweight is zero, dx is empty
    if (!dweight) return LCE_OK;
    hipError_t e = lce::launch_fill_f32(dweight, vocab * hidden, 0.0f, stream);
    return e == hipSuccess ? LCE_OK : hip_fail(e, "launch");
  }
  return run_fused_bwd(x, weight, tokens, hidden, vocab, target, mean, grad, dx, dweight, stream);
}

}  // extern "C"
