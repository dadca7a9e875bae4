// Host-side runtime helpers: the kernel timing hook (HIP event pairs around
// every library launch while recording is on; msa_profile_begin /
// msa_profile_end in include/msa.h) and the device's compute-unit count.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "launch.h"
#include "msa.h"

namespace msa {
namespace {

struct Record {
  const char* name;
  hipEvent_t start, stop;
};

constexpr size_t kPoolEvents = 4096;      // created up front, so recording stays cheap

// g_pool, g_next, g_extra and g_records are only touched with g_mu held, so
// launches on other threads may overlap msa_profile_begin / msa_profile_end.
std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Record> g_records;
std::vector<hipEvent_t> g_pool;           // created by msa_profile_begin
size_t g_next = 0;
std::vector<hipEvent_t> g_extra;          // created on demand once the pool is used up

hipEvent_t take_event() {
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_next < g_pool.size()) return g_pool[g_next++];
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  g_extra.push_back(e);
  return e;
}

// Caller holds g_mu.
void release_events_locked() {
  for (hipEvent_t e : g_pool) (void)hipEventDestroy(e);
  for (hipEvent_t e : g_extra) (void)hipEventDestroy(e);
  g_pool.clear();
  g_extra.clear();
  g_next = 0;
}

}  // namespace

LaunchTimer::LaunchTimer(const char* name, hipStream_t stream) : name_(name), stream_(stream) {
  if (!g_on.load(std::memory_order_acquire)) return;
  start_ = take_event();
  if (start_ && hipEventRecord(start_, stream_) != hipSuccess) start_ = nullptr;
}

LaunchTimer::~LaunchTimer() {
  if (!start_) return;
  hipEvent_t stop = take_event();
  if (!stop || hipEventRecord(stop, stream_) != hipSuccess) return;
  std::lock_guard<std::mutex> lock(g_mu);
  g_records.push_back(Record{name_, start_, stop});
}

// Compute units of the current device (cached per device id).
int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace msa

extern "C" {

msa_status msa_profile_begin(void) {
  msa::g_on.store(false, std::memory_order_release);
  std::lock_guard<std::mutex> lock(msa::g_mu);
  msa::g_records.clear();
  msa::release_events_locked();
  msa::g_pool.reserve(msa::kPoolEvents);
  for (size_t i = 0; i < msa::kPoolEvents; ++i) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) {
      msa::release_events_locked();
      return MSA_ERR_HIP;
    }
    msa::g_pool.push_back(e);
  }
  msa::g_on.store(true, std::memory_order_release);
  return MSA_OK;
}

msa_status msa_profile_end(msa_kernel_time* out, int32_t capacity, int32_t* count) {
  msa::g_on.store(false, std::memory_order_release);
  std::vector<msa::Record> recs;
  {
    std::lock_guard<std::mutex> lock(msa::g_mu);
    recs.swap(msa::g_records);
  }
  bool ok = true;
  std::map<std::string, std::pair<int32_t, double>> agg;
  for (const msa::Record& r : recs) {
    float ms = 0.f;
    if (ok && (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess))
      ok = false;
    if (ok) {
      auto& a = agg[r.name];
      a.first += 1;
      a.second += ms;
    }
  }
  {
    std::lock_guard<std::mutex> lock(msa::g_mu);
    msa::release_events_locked();
  }
  if (!count) return MSA_ERR_NULL;
  if (!ok) return MSA_ERR_HIP;
  std::vector<std::pair<std::string, std::pair<int32_t, double>>> v(agg.begin(), agg.end());
  std::sort(v.begin(), v.end(), [](const auto& a, const auto& b) { return a.second.second > b.second.second; });
  *count = (int32_t)v.size();
  for (int32_t i = 0; out && i < capacity && i < (int32_t)v.size(); ++i) {
    std::memset(out[i].name, 0, sizeof out[i].name);
    std::strncpy(out[i].name, v[i].first.c_str(), sizeof out[i].name - 1);
    out[i].launches = v[i].second.first;
    out[i].total_ms = v[i].second.second;
  }
  return MSA_OK;
}

}  // extern "C"
