// Host-side plumbing shared by liblce's entry points (not part of the C ABI):
// errors, the scratch pool, validation, and the kernel paths other entry
// points build on.
#pragma once

#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "lce.h"
#include "lce_internal.h"

namespace lce {
namespace host {

// ---- errors: a status plus a thread-local message (lce_last_error)
std::string& last_error();
lce_status fail(lce_status s, const char* fmt, ...);
lce_status hip_fail(hipError_t e, const char* what);

// ---- what the call enqueued (lce_last_launch): a thread-local record of the
// kernels and their grids, appended to by every launch of the current call.
// begin_call() clears it and the error message; every entry point starts with it.
std::string& last_launch();
void note_launch(const char* fmt, ...);
void begin_call();

// [a, a + an) and [b, b + bn) overlap (byte ranges); p is n-byte aligned.
bool overlaps(const void* a, uint64_t an, const void* b, uint64_t bn);
bool aligned(const void* p, uint64_t n);

// ---- scratch: one grow-only device buffer per (device, stream), carved into
// 256-byte-aligned regions; the deterministic mean keeps its counters and
// slots in a second buffer of its own (MeanState).
constexpr size_t kAlign = 256;
// Most bytes one kernel streams through a single buffer resource (32-bit
// offsets, with room for the batch loaded past the end).
constexpr int64_t kMaxStreamBytes = int64_t(1) << 30;
inline size_t round_up(size_t n, size_t a) { return (n + a - 1) / a * a; }

struct Carve {
  size_t off = 0;
  size_t take(size_t n) {
    const size_t o = off;
    off = round_up(off + n, kAlign);
    return o;
  }
};

// This stream's scratch, grown (outside graph capture only) to `need` bytes.
lce_status get_scratch(hipStream_t stream, size_t need, char** out);

// The deterministic mean's state for one launch: the epoch word (on its own
// line of kMeanHeaderBytes), then one 64-bit (tag, partial) slot per
// workgroup.  It lives in a buffer that only the mean reductions write, so a
// slot can hold nothing but a tag of an earlier launch on the same buffer
// (or zero, for a new buffer); general scratch, which other calls fill with
// arbitrary data, never overlaps it.  One per (device, stream), grown
// (outside graph capture only) and zeroed whole when it grows.
struct MeanState {
  unsigned* epoch = nullptr;
  uint64_t* slots = nullptr;
};
lce_status get_mean_state(hipStream_t stream, int64_t nslots, MeanState* out);
lce_status num_cus(int* n);
int env_int(const char* name, int dflt);
int64_t env_int64(const char* name, int64_t dflt);

// ---- validation (host only)
lce_status validate_common(int64_t tokens, const int64_t* target, int reduction, const float* out,
                           const char* out_name = "out", bool has_target = true);
uint64_t out_bytes(int64_t tokens, int reduction);
// `out_elems` fp32 outputs per token (1, or 3 for shard statistics).
lce_status validate_xent(const void* logits, int dtype, int64_t tokens, int64_t vocab,
                         const int64_t* target, int reduction, const float* out,
                         const char* out_name = "out", int out_elems = 1);
// One bf16 projection: activations x [tokens, hidden] and head w [vocab, hidden],
// against an output of `ob` bytes.
lce_status validate_head(const void* x, const void* w, int64_t tokens, int64_t hidden, int64_t vocab,
                         const float* out, uint64_t ob, const char* xn = "x",
                         const char* wn = "weight");
// `out_floats` >= 0 overrides the output size implied by the reduction.
lce_status validate_fused(const void* x, const void* w, int64_t tokens, int64_t hidden, int64_t vocab,
                          const int64_t* target, int reduction, const float* out,
                          int64_t out_floats = -1);

// ---- kernel paths (arguments validated, tokens > 0).  The first `reserved`
// bytes of scratch regions belong to the caller.
//
// Device memory a caller brings for the row kernels instead of the pool: the
// mean's epoch word (kMeanHeaderBytes, zero before the first launch),
// `max_slots` mean slots, and `general_bytes` for the split path's partials.
struct RowWorkspace {
  unsigned* epoch = nullptr;
  uint64_t* slots = nullptr;
  int64_t max_slots = 0;
  char* general = nullptr;
  size_t general_bytes = 0;
};
lce_status run_rows(const void* logits, int dtype, int64_t tokens, int64_t vocab,
                    const int64_t* target, bool mean, float* out, int64_t vocab_start,
                    float* stats, hipStream_t stream, size_t reserved = 0,
                    const RowWorkspace* ws = nullptr);

// Scratch plan of the fused projection + cross-entropy: vocab segments and the
// offsets of its regions after the caller's `reserved` bytes.
struct FusedPlan {
  int segments = 1;
  size_t off_seg = 0, off_zt = 0, end = 0;
};
FusedPlan plan_fused(int64_t tokens, int64_t vocab, int cus, size_t reserved);
lce_status run_fused(const void* x, const void* weight, int64_t tokens, int64_t hidden, int64_t vocab,
                     const int64_t* target, bool mean, float* out, hipStream_t stream,
                     size_t reserved = 0, float* lse_out = nullptr, float* z_out = nullptr,
                     int64_t z_ld = 0);

// Chunking of the fused backward: `chunk` tokens per pass (a multiple of the
// fused tile's 256 tokens unless all tokens fit), logit rows of `ld` columns
// (vocab rounded up to the tile), and whether the chunk's fp32 logits are
// stored (6 bytes per logit with dZ) or recomputed (2 bytes per logit), for a
// scratch cap of `cap` bytes.
struct FusedBwdPlan {
  int64_t chunk = 0, ld = 0;
  bool stored = false;
};
FusedBwdPlan plan_fused_bwd(int64_t tokens, int64_t vocab, int64_t cap);

// D (fp32, column-major m x n, leading dimension ldd) = op(A) op(B) + beta D
// with bf16 A and B (column-major, op N or T), through hipBLASLt.
lce_status gemm_bf16_f32(hipblasOperation_t ta, hipblasOperation_t tb, int64_t m, int64_t n,
                         int64_t k, const void* A, int64_t lda, const void* B, int64_t ldb,
                         float beta, float* D, int64_t ldd, void* ws, size_t ws_bytes,
                         hipStream_t stream);

}  // namespace host
}  // namespace lce
