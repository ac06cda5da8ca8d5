// Status strings, per-thread error messages and the optional per-kernel timing.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "moe_internal.h"

namespace moe {

static thread_local char g_last_error[512] = "";

void set_error(const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
}

void clear_error() { g_last_error[0] = '\0'; }

int check_launch(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: %s", what, hipGetErrorString(e));
    return MOE_ERR_HIP;
  }
  return MOE_OK;
}

// ------------------------------------------------------------------ timing

namespace {
struct Record {
  std::string name;
  hipEvent_t start, stop;
};
std::mutex g_mu;
bool g_timing = false;
std::vector<Record> g_records;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

TimedLaunch::TimedLaunch(const char *name, hipStream_t s) : name_(name), stream_(s), slot_(-1) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_timing) return;
  hipEvent_t a = take_event(), b = take_event();
  if (!a || !b) {   // no timing for this launch; keep what was taken
    if (a) g_pool.push_back(a);
    if (b) g_pool.push_back(b);
    return;
  }
  (void)hipEventRecord(a, s);
  g_records.push_back(Record{std::string(name), a, b});
  slot_ = (int)g_records.size() - 1;
}

TimedLaunch::~TimedLaunch() {
  if (slot_ < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (slot_ < (int)g_records.size()) (void)hipEventRecord(g_records[slot_].stop, stream_);
}

}  // namespace moe

extern "C" {

int moe_version(void) { return 100; }

const char *moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported dtype or shape";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char *moe_last_error(void) { return moe::g_last_error; }

int moe_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(moe::g_mu);
  moe::g_timing = on != 0;
  return MOE_OK;
}

int moe_timing_reset(void) {
  std::lock_guard<std::mutex> lk(moe::g_mu);
  for (auto &r : moe::g_records) {
    (void)hipEventSynchronize(r.stop);
    moe::g_pool.push_back(r.start);
    moe::g_pool.push_back(r.stop);
  }
  moe::g_records.clear();
  return MOE_OK;
}

int moe_timing_query(const char *name, double *total_ms, int64_t *launches) {
  if (!total_ms || !launches) {
    moe::set_error("moe_timing_query: null output pointer");
    return MOE_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lk(moe::g_mu);
  double tot = 0.0;
  int64_t n = 0;
  for (auto &r : moe::g_records) {
    if (name && strcmp(r.name.c_str(), name) != 0) continue;
    if (hipEventSynchronize(r.stop) != hipSuccess) {
      moe::set_error("moe_timing_query: event wait failed");
      return MOE_ERR_HIP;
    }
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) {
      moe::set_error("moe_timing_query: elapsed time failed");
      return MOE_ERR_HIP;
    }
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return MOE_OK;
}

}  // extern "C"
