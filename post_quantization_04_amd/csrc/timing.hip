// Optional per-launch kernel timing with HIP events (kq_timing_enable / kq_timing_query).
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kq_internal.h"

namespace kq {
namespace {

struct Record {
  std::string name;
  hipEvent_t begin;
  hipEvent_t end;
};

struct State {
  std::mutex mu;
  bool on = false;
  std::vector<std::string> filters;  // alternatives; a launch is timed if its name contains any
  std::vector<Record> records;
  std::vector<hipEvent_t> pool;
};

State& state() {
  static State s;
  return s;
}

hipEvent_t take_event(State& s) {
  if (!s.pool.empty()) {
    hipEvent_t e = s.pool.back();
    s.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void recycle(State& s) {
  for (Record& r : s.records) {
    if (r.begin) s.pool.push_back(r.begin);
    if (r.end) s.pool.push_back(r.end);
  }
  s.records.clear();
}

}  // namespace

LaunchTimer::LaunchTimer(const char* name, hipStream_t st) : name_(name), st_(st) {
  State& s = state();
  std::lock_guard<std::mutex> lock(s.mu);
  if (!s.on) return;
  bool hit = false;
  for (const std::string& f : s.filters) hit = hit || std::strstr(name, f.c_str()) != nullptr;
  if (!hit) return;
  begin_ = take_event(s);
  if (begin_ && hipEventRecord(begin_, st_) != hipSuccess) begin_ = nullptr;
}

LaunchTimer::~LaunchTimer() {
  if (!begin_) return;
  State& s = state();
  std::lock_guard<std::mutex> lock(s.mu);
  hipEvent_t end = take_event(s);
  if (!end || hipEventRecord(end, st_) != hipSuccess) {
    s.pool.push_back(begin_);
    if (end) s.pool.push_back(end);
    return;
  }
  s.records.push_back(Record{name_, begin_, end});
}

}  // namespace kq

extern "C" {

kq_status kq_timing_enable(const char* filter) {
  kq::State& s = kq::state();
  std::lock_guard<std::mutex> lock(s.mu);
  kq::recycle(s);
  s.on = filter != nullptr;
  s.filters.clear();
  if (filter) {
    std::string all(filter);
    size_t b = 0;
    for (size_t e; (e = all.find('|', b)) != std::string::npos; b = e + 1) s.filters.push_back(all.substr(b, e - b));
    s.filters.push_back(all.substr(b));
  }
  return KQ_OK;
}

kq_status kq_timing_query(const char* name, int64_t* launches, double* total_ms) {
  if (!name || !launches || !total_ms) return kq::fail(KQ_EINVAL, "kq_timing_query: NULL pointer");
  kq::State& s = kq::state();
  std::lock_guard<std::mutex> lock(s.mu);
  int64_t n = 0;
  double ms = 0.0;
  for (const kq::Record& r : s.records) {
    if (r.name.find(name) == std::string::npos) continue;
    if (hipEventSynchronize(r.end) != hipSuccess) return kq::fail(KQ_EDEVICE, "kq_timing_query: event wait failed");
    float t = 0.0f;
    if (hipEventElapsedTime(&t, r.begin, r.end) != hipSuccess)
      return kq::fail(KQ_EDEVICE, "kq_timing_query: elapsed time unavailable");
    ms += t;
    ++n;
  }
  *launches = n;
  *total_ms = ms;
  return KQ_OK;
}

}  // extern "C"
