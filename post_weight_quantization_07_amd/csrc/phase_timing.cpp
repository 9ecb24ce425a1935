// Per-phase launch timing, a measurement aid.  While it is switched on, every
// instrumented launch site records one HIP event before and one after its
// launch on the launch's own stream; the query sums, per phase, the time
// between each launch's pair of events.  Switched off (the default), a site
// costs one relaxed atomic load.  Not meant for calls running concurrently on
// several host threads while switched on.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "gptq_internal.h"

namespace gptq {
namespace {

struct Span {
  int phase;
  size_t begin, end;  // indices into the event pool
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<hipEvent_t> g_pool;  // created on demand, kept for reuse
size_t g_used = 0;
std::vector<Span> g_spans;
std::vector<size_t> g_open;      // per phase: index of the span being recorded, or npos
hipError_t g_err = hipSuccess;

constexpr size_t kNone = static_cast<size_t>(-1);

size_t take_event() {
  if (g_used == g_pool.size()) {
    hipEvent_t e = nullptr;
    const hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      g_err = r;
      return kNone;
    }
    g_pool.push_back(e);
  }
  return g_used++;
}

}  // namespace

bool phase_timing_on() { return g_on.load(std::memory_order_relaxed); }

void phase_mark(int phase, bool begin, hipStream_t st) {
  if (!phase_timing_on()) return;
  std::lock_guard<std::mutex> lock(g_mu);
  if (phase < 0 || phase >= kNumPhases) return;
  if (g_open.size() != static_cast<size_t>(kNumPhases)) g_open.assign(kNumPhases, kNone);
  const size_t ev = take_event();
  if (ev == kNone) return;
  const hipError_t r = hipEventRecord(g_pool[ev], st);
  if (r != hipSuccess) {
    g_err = r;
    return;
  }
  if (begin) {
    g_spans.push_back(Span{phase, ev, kNone});
    g_open[phase] = g_spans.size() - 1;
  } else if (g_open[phase] != kNone) {
    g_spans[g_open[phase]].end = ev;
    g_open[phase] = kNone;
  }
}

hipError_t phase_timing_set(bool on) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (on) {
    g_used = 0;
    g_spans.clear();
    g_open.assign(kNumPhases, kNone);
    g_err = hipSuccess;
  }
  g_on.store(on, std::memory_order_relaxed);
  return hipSuccess;
}

hipError_t phase_timing_read(float* ms, int32_t* launches, int n) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_err != hipSuccess) return g_err;
  for (int i = 0; i < n; ++i) {
    ms[i] = 0.f;
    launches[i] = 0;
  }
  for (const Span& s : g_spans) {
    if (s.end == kNone || s.phase >= n) continue;
    hipError_t r = hipEventSynchronize(g_pool[s.end]);
    if (r != hipSuccess) return r;
    float t = 0.f;
    r = hipEventElapsedTime(&t, g_pool[s.begin], g_pool[s.end]);
    if (r != hipSuccess) return r;
    ms[s.phase] += t;
    launches[s.phase] += 1;
  }
  return hipSuccess;
}

const char* phase_name(int phase) {
  switch (phase) {
    case kPhHessian: return "hessian_partial";
    case kPhHessReduce: return "hessian_reduce";
    case kPhPrepElem: return "prepare_elementwise";
    case kPhPanel: return "cholesky_panel";
    case kPhCholUpdate: return "cholesky_update";
    case kPhTrtri: return "triangular_inverse";
    case kPhQuantElem: return "quantize_elementwise";
    case kPhSweep: return "sweep";
    case kPhUpdate: return "trailing_update";
    case kPhPack: return "pack";
    default: return nullptr;
  }
}

}  // namespace gptq
