// Thread-safe one-time host set-up and per-device facts, shared by the launchers.
#pragma once
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

namespace mla {

// A set-up step (kernel attributes) that runs once per process even when
// several host threads make their first calls at the same time: the first
// caller runs it under the lock, later callers skip it.  A failed set-up is
// not recorded as done, so the next call tries again and reports its own
// result.
struct OnceFlag {
  std::mutex mu;
  std::atomic<bool> done{false};
};

template <typename F>
inline hipError_t run_once(OnceFlag& flag, F&& set_up) {
  if (flag.done.load(std::memory_order_acquire)) return hipSuccess;
  std::lock_guard<std::mutex> lock(flag.mu);
  if (flag.done.load(std::memory_order_relaxed)) return hipSuccess;
  const hipError_t e = set_up();
  if (e == hipSuccess) flag.done.store(true, std::memory_order_release);
  return e;
}

// Compute units of the calling thread's current device (queried once per
// device and cached; 256 if the query fails).
int device_cus();

// Chunks per head group of the decode split: 0 = one per compute unit (the
// default), else the count set by mla_decode_set_splits().
int decode_splits_override();

}  // namespace mla
