// liblce host plumbing shared by the entry points: error reporting, the
// per-stream scratch pool, device queries, environment overrides and argument
// validation.  All of it runs on the host, before any kernel is launched.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "lce.h"
#include "lce_host.h"
#include "lce_internal.h"

namespace lce {
namespace host {

thread_local std::string g_last_error;

std::string& last_error() { return g_last_error; }

lce_status fail(lce_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

thread_local std::string g_last_launch;

std::string& last_launch() { return g_last_launch; }

void note_launch(const char* fmt, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (!g_last_launch.empty()) g_last_launch += " + ";
  g_last_launch += buf;
}

void begin_call() {
  g_last_error.clear();
  g_last_launch.clear();
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
// Grow-only device buffers per (device, stream): general scratch, carved into
// regions by Carve, and the deterministic mean's state (epoch word and
// slots), which nothing else writes.  A buffer that is outgrown is retired,
// not freed: launches already queued, or recorded into a HIP graph that may be
// replayed later, keep pointing at it.  Every buffer lives until process exit.
// A new buffer is zeroed whole.
struct Scratch {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, Scratch> g_scratch;
std::map<std::pair<int, hipStream_t>, Scratch> g_mean;
std::vector<void*> g_retired;
std::map<int, int> g_num_cus;

// Grows `s` (the buffer of `stream`) to at least `need` bytes; call with g_mu held.
static lce_status grow(Scratch& s, hipStream_t stream, size_t need) {
  if (s.bytes < need) {
    hipError_t e = hipSuccess;
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
    // The epoch word and the mean slots must start at zero (a slot then only
    // ever holds tags of earlier launches on this buffer).
    e = lce::launch_zero_u32((unsigned*)p, (int64_t)(bytes / sizeof(unsigned)), stream);
    if (e != hipSuccess) {
      (void)hipFree(p);
      return hip_fail(e, "scratch initialisation");
    }
    if (s.ptr) g_retired.push_back(s.ptr);
    s.ptr = p;
    s.bytes = bytes;
  }
  return LCE_OK;
}

lce_status get_scratch(hipStream_t stream, size_t need, char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_mu);
  Scratch& s = g_scratch[{dev, stream}];
  lce_status st = grow(s, stream, need);
  if (st != LCE_OK) return st;
  *out = (char*)s.ptr;
  return LCE_OK;
}

lce_status get_mean_state(hipStream_t stream, int64_t nslots, MeanState* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_mu);
  Scratch& s = g_mean[{dev, stream}];
  const size_t off_slots = round_up(lce::kMeanHeaderBytes, kAlign);
  lce_status st = grow(s, stream, off_slots + (size_t)(nslots > 0 ? nslots : 1) * 8u);
  if (st != LCE_OK) return st;
  out->epoch = (unsigned*)s.ptr;
  out->slots = (uint64_t*)((char*)s.ptr + off_slots);
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
                           const char* out_name, bool has_target) {
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
                         const char* out_name, int out_elems) {
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
  // The row kernels launch one wave (64 work-items) per row, or a 256-thread
  // workgroup per row for rows longer than 32 KiB; a dispatch counts its
  // work-items in 32 bits.
  const int64_t per_row = vocab * esize > 32 * 1024 ? lce::kRowThreads : 64;
  if (tokens > lce::kMaxGridItems / per_row)
    return fail(LCE_ERR_UNSUPPORTED,
                "tokens * %lld work-items per row must be < 2^32 (got %lld tokens)",
                (long long)per_row, (long long)tokens);
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
                         const float* out, uint64_t ob, const char* xn,
                         const char* wn) {
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
  // The projection kernels launch up to 4 work-items per token per vocab
  // segment (a dispatch counts its work-items in 32 bits).
  if (tokens >= (int64_t(1) << 30))
    return fail(LCE_ERR_UNSUPPORTED, "tokens must be < 2^30 for the fused projection (got %lld)",
                (long long)tokens);
  if (overlaps(out, ob, x, (uint64_t)(tokens * hidden * 2))) return fail(LCE_ERR_ALIAS, "out overlaps %s", xn);
  if (overlaps(out, ob, w, (uint64_t)(vocab * hidden * 2))) return fail(LCE_ERR_ALIAS, "out overlaps %s", wn);
  return LCE_OK;
}

lce_status validate_fused(const void* x, const void* w, int64_t tokens, int64_t hidden, int64_t vocab,
                          const int64_t* target, int reduction, const float* out,
                          int64_t out_floats) {
  lce_status s = validate_common(tokens, target, reduction, out);
  if (s != LCE_OK) return s;
  uint64_t ob = out_bytes(tokens, reduction);
  if (out_floats >= 0) ob = (uint64_t)out_floats * 4u;
  if ((s = validate_head(x, w, tokens, hidden, vocab, out, ob)) != LCE_OK) return s;
  if (overlaps(out, ob, target, (uint64_t)tokens * 8u)) return fail(LCE_ERR_ALIAS, "out overlaps target");
  return LCE_OK;
}

}  // namespace host
}  // namespace lce
