// Kernel launchers for the host-only sanitizer build: the validation and
// planning paths the driver exercises never reach them.
#include <hip/hip_runtime.h>

#include "../../long_context_mla_amd/csrc/device_common.h"
#include "../../long_context_mla_amd/csrc/launch.h"

namespace mla {
int decode_rows_fp8() { return 64; }
int decode_rows_per_group(int cache_kind) { return cache_kind == kFp8 ? 64 : 64; }
hipError_t launch_kv_append(const AppendArgs&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_decode(const DecodeArgs&, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_decode_fp8(const DecodeArgs&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_combine(const CombineArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_kv_check(const CheckArgs&, hipStream_t) { return hipErrorInvalidValue; }
}  // namespace mla
