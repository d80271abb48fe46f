// Launch log and per-kernel event timing (see trace.h and the moe_trace_* calls in moe.h).
#include "trace.h"

#include <string>
#include <vector>

#include "../../include/moe.h"

namespace moe {
namespace trace {
namespace {

struct Rec {
  const char* name;
  hipStream_t stream;
  int ev0, ev1;  // indices into the event pool, -1 without timing
  bool launched; // the kernel dispatch recorded ev0/ev1
};

struct State {
  bool on = false;
  bool timing = false;
  std::string only;  // non-empty: timing events for launches of this name only
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;  // reused across logs; grows on demand
  size_t used = 0;
  int open = -1;
  hipError_t err = hipSuccess;
};

thread_local State g;

int take_event() {
  if (g.used == g.pool.size()) {
    hipEvent_t e;
    hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableSystemFence);  // timing only
    if (r != hipSuccess) { g.err = r; return -1; }
    g.pool.push_back(e);
  }
  return (int)g.used++;
}

}  // namespace

bool active() { return g.on; }

void begin(const char* name, hipStream_t s) {
  Rec r{name, s, -1, -1, false};
  if (g.timing && (g.only.empty() || g.only == name)) {
    r.ev0 = take_event();
    r.ev1 = take_event();
  }
  g.recs.push_back(r);
  g.open = (int)g.recs.size() - 1;
}

void launch_events(hipEvent_t* start, hipEvent_t* stop) {
  *start = *stop = nullptr;
  if (g.open < 0 || !g.timing) return;
  Rec& r = g.recs[g.open];
  if (r.ev0 < 0 || r.ev1 < 0 || r.launched) return;
  *start = g.pool[r.ev0];
  *stop = g.pool[r.ev1];
  r.launched = true;
}

void end(hipStream_t s) {
  if (g.open < 0) return;
  Rec& r = g.recs[g.open];
  if (g.timing && !r.launched) {  // no launch took the events: record them here so they are valid
    for (int ev : {r.ev0, r.ev1}) {
      if (ev < 0) continue;
      hipError_t e = hipEventRecord(g.pool[ev], s);
      if (e != hipSuccess) g.err = e;
    }
  }
  g.open = -1;
}

}  // namespace trace
}  // namespace moe

using moe::trace::g;

extern "C" {

moe_status moe_trace_enable(int32_t timing) {
  g.on = true;
  g.timing = timing != 0;
  g.only.clear();
  g.recs.clear();
  g.used = 0;
  g.open = -1;
  g.err = hipSuccess;
  return MOE_OK;
}

moe_status moe_trace_enable_only(const char* only) {
  if (!only) return MOE_ERR_ARG;
  moe_trace_enable(1);
  g.only = only;
  return MOE_OK;
}

moe_status moe_trace_disable(void) {
  g.on = false;
  return MOE_OK;
}

int64_t moe_trace_count(void) { return (int64_t)g.recs.size(); }

moe_status moe_trace_entry(int64_t i, const char** name, void** stream, float* ms) {
  if (i < 0 || i >= (int64_t)g.recs.size() || !name || !stream || !ms) return MOE_ERR_ARG;
  const auto& r = g.recs[(size_t)i];
  *name = r.name;
  *stream = (void*)r.stream;
  *ms = -1.f;
  if (r.ev0 >= 0 && r.ev1 >= 0) {
    hipError_t e = hipEventSynchronize(g.pool[r.ev1]);
    if (e == hipSuccess) e = hipEventElapsedTime(ms, g.pool[r.ev0], g.pool[r.ev1]);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  return g.err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_trace_span(int64_t i, float* start_ms, float* end_ms) {
  if (i < 0 || i >= (int64_t)g.recs.size() || !start_ms || !end_ms) return MOE_ERR_ARG;
  const auto& r0 = g.recs[0];
  const auto& r = g.recs[(size_t)i];
  if (r0.ev0 < 0 || r.ev0 < 0 || r.ev1 < 0) return MOE_ERR_HIP;
  hipError_t e = hipEventSynchronize(g.pool[r.ev1]);
  if (e == hipSuccess) e = hipEventSynchronize(g.pool[r0.ev0]);
  if (e == hipSuccess) e = hipEventElapsedTime(start_ms, g.pool[r0.ev0], g.pool[r.ev0]);
  if (e == hipSuccess) e = hipEventElapsedTime(end_ms, g.pool[r0.ev0], g.pool[r.ev1]);
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
