// Row cross-entropy for callers that cannot allocate (lce_xent_fwd_noalloc):
// the same kernels and path selection as lce_xent_fwd, with the scratch they
// need -- the mean's epoch word and per-workgroup slots, and
// the split path's per-slice partials -- in one file-scope device array
// instead of the library's grow-only pool.  The call makes no hipMalloc or
// hipFree and uses no allocating library routine.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <map>
#include <mutex>

#include "lce.h"
#include "lce_host.h"
#include "lce_internal.h"

namespace lce {

// Layout of the array: the mean's epoch word (kMeanHeaderBytes), then 2^19
// 64-bit mean slots (4 MiB: a mean over up to 2^23 rows of <= 32 KiB on the
// one-wave-per-row path, 16 rows per workgroup, and 2^22 to 2^24 rows of
// <= 2 KiB on the several-rows-per-wave path, 8 to 32 rows per workgroup),
// then the split path's (max, sum-exp) partials in the rest (8 bytes per row
// and slice).
constexpr size_t kStaticBytes = size_t(8) << 20;
constexpr size_t kSlotsOff = kMeanHeaderBytes;
constexpr int64_t kMaxSlots = int64_t(1) << 19;
constexpr size_t kGeneralOff = kSlotsOff + (size_t)kMaxSlots * 8u;
constexpr size_t kGeneralBytes = kStaticBytes - kGeneralOff;
static_assert(kSlotsOff % 256 == 0 && kGeneralOff % 256 == 0, "256-byte aligned regions");

// One copy per GPU, held until the process ends.  In host code the name is
// only a stand-in for the symbol: its device address on the current GPU
// comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[kStaticBytes];

namespace {

struct DeviceArray {
  unsigned char* ptr = nullptr;  // device address of `scratch` on this GPU
  bool cleared = false;          // epoch word and slots zeroed by an uncaptured call
};
std::mutex g_mu;
std::map<int, DeviceArray> g_arrays;

}  // namespace
}  // namespace lce

using namespace lce::host;

extern "C" {

lce_status lce_xent_fwd_noalloc(const void* logits, lce_dtype dtype, int64_t tokens, int64_t vocab,
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
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  unsigned char* base = nullptr;
  bool clear = false, mark = false;
  {
    std::lock_guard<std::mutex> lock(lce::g_mu);
    lce::DeviceArray& d = lce::g_arrays[dev];
    if (!d.ptr) {  // once per GPU, with that GPU current
      e = hipGetSymbolAddress((void**)&d.ptr, HIP_SYMBOL(lce::scratch));
      if (e != hipSuccess) {
        d.ptr = nullptr;
        return hip_fail(e, "hipGetSymbolAddress of the static scratch array");
      }
    }
    base = d.ptr;
    if (!d.cleared) {
      // The first call on a GPU zeroes the epoch word and slots with a
      // kernel on the caller's stream, ahead of its own kernels.  Under graph
      // capture the clear is recorded into the graph (each replay repeats it)
      // and the next uncaptured call clears again.
      hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
      e = hipStreamIsCapturing(stream, &cap);
      if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
      clear = true;
      mark = cap == hipStreamCaptureStatusNone;
    }
    if (clear) {
      e = lce::launch_zero_u32((unsigned*)base, (int64_t)(lce::kGeneralOff / sizeof(unsigned)), stream);
      if (e != hipSuccess) return hip_fail(e, "clearing the static scratch array");
      if (mark) d.cleared = true;
    }
  }
  RowWorkspace ws;
  ws.epoch = (unsigned*)base;
  ws.slots = (uint64_t*)(base + lce::kSlotsOff);
  ws.max_slots = lce::kMaxSlots;
  ws.general = (char*)(base + lce::kGeneralOff);
  ws.general_bytes = lce::kGeneralBytes;
  return run_rows(logits, (int)dtype, tokens, vocab, target, mean, out, 0, nullptr, stream, 0, &ws);
}

}  // extern "C"
