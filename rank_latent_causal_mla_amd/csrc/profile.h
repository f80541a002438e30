// Optional per-kernel timing: while enabled, each library kernel launch is
// bracketed by HIP events recorded on the launch stream.
#pragma once
#include <hip/hip_runtime.h>

namespace mla {

bool profiling_enabled();
void profile_record(const char* name, hipStream_t st, bool start);

struct ProfScope {
  const char* name;
  hipStream_t st;
  bool on;
  ProfScope(const char* n, hipStream_t s) : name(n), st(s), on(profiling_enabled()) {
    if (on) profile_record(name, st, true);
  }
  ~ProfScope() {
    if (on) profile_record(name, st, false);
  }
};

}  // namespace mla
