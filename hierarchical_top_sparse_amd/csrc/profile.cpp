// Optional per-kernel timing: when enabled, every kernel launch of the library is bracketed by
// two hipEvents recorded on the launch's stream.  llsa_profile_read() waits for the recorded
// events and reports, per kernel name, the launch count and the summed duration.  Disabled by
// default; when disabled a launch costs one predictable branch.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/llsa.h"
#include "kernels.hpp"

namespace llsa {

namespace {
struct Record {
  const char* name;
  hipEvent_t start, stop;
};
std::mutex g_mu;
bool g_on = false;
std::vector<Record> g_records;
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

void* prof_begin(const char* name, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_mu);
  Record r{name, take_event(), take_event()};
  if (!r.start || !r.stop) return nullptr;
  hipEventRecord(r.start, stream);
  g_records.push_back(r);
  return (void*)(g_records.size());   // 1-based handle
}

void prof_end(void* handle, hipStream_t stream) {
  if (!handle) return;
  std::lock_guard<std::mutex> lock(g_mu);
  const size_t i = (size_t)handle - 1;
  if (i < g_records.size()) hipEventRecord(g_records[i].stop, stream);
}

}  // namespace llsa

extern "C" {

int32_t llsa_profile_enable(int32_t on) {
  std::lock_guard<std::mutex> lock(llsa::g_mu);
  llsa::g_on = on != 0;
  return LLSA_OK;
}

int32_t llsa_profile_read(char* buf, size_t len) {
  std::vector<llsa::Record> recs;
  {
    std::lock_guard<std::mutex> lock(llsa::g_mu);
    recs.swap(llsa::g_records);
  }
  std::map<std::string, std::pair<long, double>> agg;
  int32_t status = LLSA_OK;
  for (auto& r : recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess ||
        hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
      status = LLSA_ERR_HIP;
    auto& a = agg[r.name];
    a.first += 1;
    a.second += ms;
  }
  {
    std::lock_guard<std::mutex> lock(llsa::g_mu);
    for (auto& r : recs) {
      llsa::g_free.push_back(r.start);
      llsa::g_free.push_back(r.stop);
    }
  }
  std::string out;
  for (auto& kv : agg) {
    char line[256];
    snprintf(line, sizeof(line), "%s %ld %.6f\n", kv.first.c_str(), kv.second.first,
             kv.second.second);
    out += line;
  }
  if (buf && len) {
    const size_t n = out.size() < len - 1 ? out.size() : len - 1;
    out.copy(buf, n);
    buf[n] = '\0';
  }
  return status;
}

}  // extern "C"
