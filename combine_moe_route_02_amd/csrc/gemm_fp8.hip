// FP8 (OCP e4m3fn) grouped expert GEMMs. Not yet implemented: the entry point reports
// hipErrorNotSupported, which the C ABI returns as MOE_ERR_HIP with a message.
#include "common.h"
#include "launch.h"

namespace moe {

hipError_t launch_expert_fwd_fp8(const void*, const float*, const void*, const float*, const void*,
                                 const float*, const int32_t*, void*, float*, void*, int, int, int,
                                 int, int, int64_t, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace moe
