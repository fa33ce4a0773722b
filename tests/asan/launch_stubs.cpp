// Host-only stand-ins for the kernel launchers, so that the C-ABI layer
// (api.cpp) can be built with g++ and the address / undefined-behaviour
// sanitizers and driven through its validation paths on a machine without a
// GPU.  Every launcher refuses (a call that passes validation returns
// DIFFATTN_ERR_HIP), so nothing here touches device memory.
#include "internal.h"

namespace diffattn {

hipError_t launch_prefill_bf16(const PrefillProblem&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_decode_bf16(const DecodeProblem&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_backward_bf16(const BackwardProblem&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_decode_compare_bf16(const CompareProblem&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_lambda_proj(const void*, const void*, float*, int, int, int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_gemm_bf16(const void*, const void*, void*, int, int, int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_rows_f32(const PrefillProblem&, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_v1_lambda(const float*, const float*, const float*, const float*, float, float*, int, int, int,
                            hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t decode_scratch(void**) { return hipErrorNotSupported; }

}  // namespace diffattn
