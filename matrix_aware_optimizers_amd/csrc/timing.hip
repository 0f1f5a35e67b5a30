// Optional HIP-event timing of the contraction launches (instrumentation for
// the benchmark's roofline figures). Disabled unless mao_timing_enable(1).
#include <atomic>
#include <mutex>
#include <vector>

#include "gemm.hpp"

namespace mao {

namespace {

struct Record {
  hipEvent_t start, stop;
  int tag;
  double flops;
};

std::mutex g_mu;
std::atomic<bool> g_on{false};
std::vector<Record> g_records;

}  // namespace

bool timing_on() { return g_on.load(std::memory_order_relaxed); }

void timing_record_begin(hipStream_t s, void** start) {
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) {
    *start = nullptr;
    return;
  }
  if (hipEventRecord(e, s) != hipSuccess) {  // nothing is timed for this launch
    (void)hipEventDestroy(e);
    *start = nullptr;
    return;
  }
  *start = (void*)e;
}

void timing_record_end(hipStream_t s, void* start, int tag, double flops) {
  if (!start) return;
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) {
    (void)hipEventDestroy((hipEvent_t)start);
    return;
  }
  if (hipEventRecord(e, s) != hipSuccess) {
    (void)hipEventDestroy(e);
    (void)hipEventDestroy((hipEvent_t)start);
    return;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  g_records.push_back(Record{(hipEvent_t)start, e, tag, flops});
}

}  // namespace mao

using namespace mao;

extern "C" {

MAO_API void mao_timing_enable(int on) { g_on.store(on != 0, std::memory_order_relaxed); }

MAO_API int mao_timing_collect(double* ms, int64_t* count, double* flops, int ntags) {
  std::vector<Record> recs;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    recs.swap(g_records);
  }
  for (int i = 0; i < ntags; ++i) {
    if (ms) ms[i] = 0.0;
    if (count) count[i] = 0;
    if (flops) flops[i] = 0.0;
  }
  int n = 0;
  for (Record& r : recs) {
    float t = 0.f;
    if (hipEventSynchronize(r.stop) == hipSuccess && hipEventElapsedTime(&t, r.start, r.stop) == hipSuccess &&
        r.tag >= 0 && r.tag < ntags) {
      if (ms) ms[r.tag] += t;
      if (count) count[r.tag] += 1;
      if (flops) flops[r.tag] += r.flops;
      ++n;
    }
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  return n;
}

}  // extern "C"
