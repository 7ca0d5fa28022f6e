// Host-side driver for the sanitizer test: calls liblce's C ABI with the
// argument vectors read from stdin and checks each returned status and error
// detail.  Built with AddressSanitizer and UndefinedBehaviorSanitizer on the
// host code; every case fails validation (or is an empty no-op) before any
// HIP call, so no device is needed or touched.
//
// Input, one case per line:
//   <function> <expected status> <argument count> <arguments...> <needle...>
// Pointers and integers are decimal; a float argument (beta) is read by
// strtof.  The needle is the rest of the line and must occur in
// lce_last_error() (an empty needle requires an empty message).
//
// Then two threads make different failing calls at the same time and check
// that each one sees its own detail message (the message is per thread).
//
// The pseudo-call `plan_fused_bwd <tokens> <vocab> <cap>` runs the fused
// backward's chunk planner (host only) and returns 2 * chunk + stored as its
// "status", so the planner's choices are checked the same way.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>
#include <thread>
#include <vector>

#include "lce.h"
#include "lce_host.h"

namespace {

struct Args {
  std::vector<std::string> v;
  const void* p(size_t i) const { return (const void*)(uintptr_t)strtoull(v.at(i).c_str(), nullptr, 10); }
  int64_t n(size_t i) const { return (int64_t)strtoll(v.at(i).c_str(), nullptr, 10); }
  int e(size_t i) const { return (int)strtol(v.at(i).c_str(), nullptr, 10); }
  float f(size_t i) const { return strtof(v.at(i).c_str(), nullptr); }
};

// One call; returns -1 for an unknown function or a wrong argument count.
int call(const std::string& fn, const Args& a) {
  const size_t k = a.v.size();
  if (fn == "lce_xent_fwd" && k == 7)
    return lce_xent_fwd(a.p(0), (lce_dtype)a.e(1), a.n(2), a.n(3), (const int64_t*)a.p(4),
                        (lce_reduction)a.e(5), (float*)a.p(6), nullptr);
  if (fn == "lce_xent_fwd_noalloc" && k == 7)
    return lce_xent_fwd_noalloc(a.p(0), (lce_dtype)a.e(1), a.n(2), a.n(3), (const int64_t*)a.p(4),
                                (lce_reduction)a.e(5), (float*)a.p(6), nullptr);
  if (fn == "lce_fused_linear_xent_fwd" && k == 8)
    return lce_fused_linear_xent_fwd(a.p(0), a.p(1), a.n(2), a.n(3), a.n(4), (const int64_t*)a.p(5),
                                     (lce_reduction)a.e(6), (float*)a.p(7), nullptr);
  if (fn == "lce_xent_partial_fwd" && k == 7)
    return lce_xent_partial_fwd(a.p(0), (lce_dtype)a.e(1), a.n(2), a.n(3), a.n(4),
                                (const int64_t*)a.p(5), (float*)a.p(6), nullptr);
  if (fn == "lce_xent_merge" && k == 7)
    return lce_xent_merge((const float*)a.p(0), a.n(1), a.n(2), (const int64_t*)a.p(3), a.n(4),
                          (lce_reduction)a.e(5), (float*)a.p(6), nullptr);
  if (fn == "lce_xent_bwd" && k == 8)
    return lce_xent_bwd(a.p(0), (lce_dtype)a.e(1), a.n(2), a.n(3), (const int64_t*)a.p(4),
                        (lce_reduction)a.e(5), (const float*)a.p(6), (void*)a.p(7), nullptr);
  if (fn == "lce_xent_fwd_bwd" && k == 9)
    return lce_xent_fwd_bwd(a.p(0), (lce_dtype)a.e(1), a.n(2), a.n(3), (const int64_t*)a.p(4),
                            (lce_reduction)a.e(5), (const float*)a.p(6), (float*)a.p(7),
                            (void*)a.p(8), nullptr);
  if (fn == "lce_fused_linear_xent_fwd_bwd" && k == 11)
    return lce_fused_linear_xent_fwd_bwd(a.p(0), a.p(1), a.n(2), a.n(3), a.n(4),
                                         (const int64_t*)a.p(5), (lce_reduction)a.e(6),
                                         (const float*)a.p(7), (float*)a.p(8), (float*)a.p(9),
                                         (float*)a.p(10), nullptr);
  if (fn == "lce_fused_linear_logprob_sums" && k == 8)
    return lce_fused_linear_logprob_sums(a.p(0), a.p(1), a.n(2), a.n(3), a.n(4), a.n(5),
                                         (const int64_t*)a.p(6), (float*)a.p(7), nullptr);
  if (fn == "lce_fused_linear_jsd_fwd" && k == 10)
    return lce_fused_linear_jsd_fwd(a.p(0), a.p(1), a.p(2), a.p(3), a.n(4), a.n(5), a.n(6), a.f(7),
                                    (lce_reduction)a.e(8), (float*)a.p(9), nullptr);
  if (fn == "plan_fused_bwd" && k == 3) {
    lce::host::last_error().clear();
    const lce::host::FusedBwdPlan p = lce::host::plan_fused_bwd(a.n(0), a.n(1), a.n(2));
    return (int)(2 * p.chunk + (p.stored ? 1 : 0));
  }
  if (fn == "lce_fused_linear_xent_bwd" && k == 10)
    return lce_fused_linear_xent_bwd(a.p(0), a.p(1), a.n(2), a.n(3), a.n(4), (const int64_t*)a.p(5),
                                     (lce_reduction)a.e(6), (const float*)a.p(7), (float*)a.p(8),
                                     (float*)a.p(9), nullptr);
  return -1;
}

bool threads_keep_their_messages() {
  bool ok[2] = {false, false};
  auto worker = [&](int id) {
    bool good = true;
    for (int i = 0; i < 2000 && good; ++i) {
      int st;
      const char* want;
      if (id == 0) {
        st = lce_xent_fwd(nullptr, LCE_F32, 4, 8, (const int64_t*)(uintptr_t)0x1000, LCE_REDUCTION_NONE,
                          (float*)(uintptr_t)0x2000, nullptr);
        want = "logits is NULL";
      } else {
        st = lce_xent_merge((const float*)(uintptr_t)0x1000, 0, 4, (const int64_t*)(uintptr_t)0x2000,
                            8, LCE_REDUCTION_NONE, (float*)(uintptr_t)0x3000, nullptr);
        want = "shards";
      }
      good = st == LCE_ERR_INVALID_ARG && strstr(lce_last_error(), want) != nullptr;
    }
    ok[id] = good;
  };
  std::thread t0(worker, 0), t1(worker, 1);
  t0.join();
  t1.join();
  return ok[0] && ok[1];
}

}  // namespace

int main() {
  char line[4096];
  int cases = 0, bad = 0;
  while (fgets(line, sizeof line, stdin)) {
    std::string s(line);
    while (!s.empty() && (s.back() == '\n' || s.back() == '\r')) s.pop_back();
    if (s.empty()) continue;
    char fn[128];
    int want = 0, nargs = 0, used = 0;
    if (sscanf(s.c_str(), "%127s %d %d%n", fn, &want, &nargs, &used) != 3) {
      fprintf(stderr, "unparsable line: %s\n", s.c_str());
      return 2;
    }
    Args a;
    const char* p = s.c_str() + used;
    for (int i = 0; i < nargs; ++i) {
      char tok[64];
      int m = 0;
      if (sscanf(p, "%63s%n", tok, &m) != 1) {
        fprintf(stderr, "missing argument %d: %s\n", i, s.c_str());
        return 2;
      }
      a.v.emplace_back(tok);
      p += m;
    }
    while (*p == ' ') ++p;
    const std::string needle(p);
    const int got = call(fn, a);
    if (got < 0) {
      fprintf(stderr, "unknown call: %s\n", s.c_str());
      return 2;
    }
    const char* msg = lce_last_error();
    const bool msg_ok = needle.empty() ? msg[0] == '\0' : strstr(msg, needle.c_str()) != nullptr;
    if (got != want || !msg_ok) {
      fprintf(stderr, "FAIL %s: status %d (want %d), message \"%s\" (want \"%s\")\n", fn, got, want,
              msg, needle.c_str());
      ++bad;
    }
    ++cases;
  }
  for (int s = -1; s <= 6; ++s)
    if (!lce_status_string((lce_status)s) || !lce_status_string((lce_status)s)[0]) ++bad;
  if (lce_version() <= 0) ++bad;
  if (!threads_keep_their_messages()) {
    fprintf(stderr, "FAIL per-thread error messages\n");
    ++bad;
  }
  printf("cases %d failed %d\n", cases, bad);
  return bad ? 1 : 0;
}
