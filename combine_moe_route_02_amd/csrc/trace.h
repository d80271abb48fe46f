// Launch log and per-kernel HIP-event timing (host side). When tracing is on, every kernel launch
// the library makes on the calling thread is recorded with its name and stream; with timing on,
// the kernel dispatch itself records a start and a stop event (hipExtLaunchKernel), which costs
// far less than event-record packets between kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace moe {
namespace trace {

bool active();
void begin(const char* name, hipStream_t s);  // before a kernel launch
void end(hipStream_t s);                      // after it
// The open record's two timing events, for the launch itself to record (as part of the kernel
// dispatch, with no separate marker packets); both null when timing is off.
void launch_events(hipEvent_t* start, hipEvent_t* stop);

struct Scope {
  hipStream_t s;
  bool on;
  Scope(const char* name, hipStream_t st) : s(st), on(active()) { if (on) begin(name, st); }
  ~Scope() { if (on) end(s); }
};

}  // namespace trace
}  // namespace moe

#define MOE_TRACE(name, stream) ::moe::trace::Scope _moe_trace_scope_((name), (stream))

// Kernel launch inside a MOE_TRACE scope: with timing, the dispatch records the scope's events.
#define MOE_LAUNCH(kernel, grid, block, shmem, stream, ...)                                         \
  do {                                                                                              \
    hipEvent_t _moe_e0 = nullptr, _moe_e1 = nullptr;                                                \
    ::moe::trace::launch_events(&_moe_e0, &_moe_e1);                                                \
    if (_moe_e0)                                                                                    \
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, _moe_e0, _moe_e1, 0, __VA_ARGS__);  \
    else                                                                                            \
      hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                          \
  } while (0)
