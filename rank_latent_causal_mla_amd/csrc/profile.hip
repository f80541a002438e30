// Per-kernel event timing behind mla_profile_enable / mla_profile_collect.
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/mla.h"
#include "profile.h"

namespace mla {
namespace {

struct Pending {
  hipEvent_t start = nullptr, stop = nullptr;
};
struct Stage {
  std::vector<Pending> launches;
  double total_ms = 0;
  int count = 0;
};

std::mutex g_mu;
bool g_on = false;
std::map<std::string, Stage> g_stages;
std::vector<hipEvent_t> g_free;

hipEvent_t take_event() {
  if (!g_free.empty()) {
    hipEvent_t e = g_free.back();
    g_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

bool profiling_enabled() { return g_on; }

void profile_record(const char* name, hipStream_t st, bool start) {
  std::lock_guard<std::mutex> lk(g_mu);
  Stage& s = g_stages[name];
  if (start) {
    Pending p;
    p.start = take_event();
    if (p.start) hipEventRecord(p.start, st);
    s.launches.push_back(p);
  } else if (!s.launches.empty() && !s.launches.back().stop) {
    Pending& p = s.launches.back();
    p.stop = take_event();
    if (p.stop) hipEventRecord(p.stop, st);
  }
}

}  // namespace mla

extern "C" {

mla_status mla_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(mla::g_mu);
  mla::g_on = on != 0;
  return MLA_OK;
}

mla_status mla_profile_collect(const char** names, double* total_ms, int* counts, int max, int* n) {
  if (!n || max < 0 || (max > 0 && (!names || !total_ms || !counts))) return MLA_ERR_INVALID_ARGUMENT;
  std::lock_guard<std::mutex> lk(mla::g_mu);
  int k = 0;
  for (auto& kv : mla::g_stages) {
    mla::Stage& s = kv.second;
    for (auto& p : s.launches) {
      if (p.start && p.stop) {
        float ms = 0.f;
        if (hipEventSynchronize(p.stop) == hipSuccess && hipEventElapsedTime(&ms, p.start, p.stop) == hipSuccess) {
          s.total_ms += ms;
          s.count += 1;
        }
      }
      if (p.start) mla::g_free.push_back(p.start);
      if (p.stop) mla::g_free.push_back(p.stop);
    }
    s.launches.clear();
    if (k < max) {
      names[k] = kv.first.c_str();
      total_ms[k] = s.total_ms;
      counts[k] = s.count;
    }
    ++k;
  }
  *n = k < max ? k : max;
  // statistics are handed out once
  for (auto& kv : mla::g_stages) {
    kv.second.total_ms = 0;
    kv.second.count = 0;
  }
  return MLA_OK;
}

}  // extern "C"
