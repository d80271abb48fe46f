// Launch log and per-kernel HIP-event timing (host side). When tracing is on, every kernel launch
// the library makes on the calling thread is recorded with its name and stream; with timing on,
// the launch is bracketed by two HIP events on that stream.
#pragma once

#include <hip/hip_runtime.h>

namespace moe {
namespace trace {

bool active();
void begin(const char* name, hipStream_t s);  // before a kernel launch
void end(hipStream_t s);                      // after it

struct Scope {
  hipStream_t s;
  bool on;
  Scope(const char* name, hipStream_t st) : s(st), on(active()) { if (on) begin(name, st); }
  ~Scope() { if (on) end(s); }
};

}  // namespace trace
}  // namespace moe

#define MOE_TRACE(name, stream) ::moe::trace::Scope _moe_trace_scope_((name), (stream))
