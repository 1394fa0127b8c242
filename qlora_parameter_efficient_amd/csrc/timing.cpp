// Event timing of the product kernels (a measurement aid, off by default).
// While enabled, every launch of a bracketed kernel records a HIP event pair
// on its stream; lq_timing_read waits for the recorded pairs, sums their
// elapsed times per kernel name and recycles the events.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"

namespace lq {
namespace {

struct Record {
  const char* name;
  hipEvent_t start, stop;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Record> g_open;    // recorded, not yet read
std::vector<hipEvent_t> g_free;
const char* g_pending = nullptr;  // name of the launch being bracketed
hipEvent_t g_pending_start = nullptr;

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

void timing_begin(const char* name, hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return;
  hipEvent_t e = take_event();
  if (!e || hipEventRecord(e, st) != hipSuccess) return;
  g_pending = name;
  g_pending_start = e;
}

void timing_end(hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on || !g_pending) return;
  hipEvent_t e = take_event();
  if (e && hipEventRecord(e, st) == hipSuccess)
    g_open.push_back(Record{g_pending, g_pending_start, e});
  g_pending = nullptr;
}

bool timing_enabled() {
  std::lock_guard<std::mutex> lk(g_mu);
  return g_on;
}

}  // namespace lq

extern "C" {

int lq_timing_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(lq::g_mu);
  lq::g_on = on != 0;
  return LQ_OK;
}

int lq_timing_read(const char* name, double* total_ms, int64_t* launches) {
  if (!name || !total_ms || !launches) {
    lq::set_error("lq_timing_read: NULL argument");
    return LQ_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lk(lq::g_mu);
  double sum = 0.0;
  int64_t n = 0;
  std::vector<lq::Record> keep;
  for (const lq::Record& r : lq::g_open) {
    if (std::strcmp(r.name, name) != 0) {
      keep.push_back(r);
      continue;
    }
    float ms = 0.0f;
    if (hipEventSynchronize(r.stop) != hipSuccess ||
        hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
      return lq::hip_fail(hipGetLastError(), "lq_timing_read");
    sum += ms;
    ++n;
    lq::g_free.push_back(r.start);
    lq::g_free.push_back(r.stop);
  }
  lq::g_open.swap(keep);
  *total_ms = sum;
  *launches = n;
  return LQ_OK;
}

}  // extern "C"
