// Kernel launchers for the host-only sanitizer build of the C ABI (api.cpp + plan.cpp built
// with g++ -fsanitize=address,undefined, no GPU code).  The ABI validation tests never reach a
// launch; if one did, the stub's error would surface as ATTN_ERR_HIP and fail the test.
#include "launch.h"

namespace fa {

hipError_t launch_prefill_bf16(const PrefillArgs&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_prefill_f32(const PrefillArgs&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_prefill_varlen_bf16(const PrefillArgs&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_mla_prefill(const PrefillArgs&, bool, bool, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_merge(const MergeArgs&, bool, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_quantize_rows(const QuantArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_gqa_decode(const DecodeArgs&, int, bool, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_gqa_decode_static(DecodeArgs, int, bool, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_mla_decode(const DecodeArgs&, bool, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace fa
