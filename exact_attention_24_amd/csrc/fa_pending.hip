// Entry points whose kernels are not written yet: they report "not supported"
// instead of computing anything.
#include "fa_internal.h"

namespace fa {
hipError_t launch_fwd_fp8(const FwdArgs &, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_bf16(const BwdArgs &, int, hipStream_t) { return hipErrorNotSupported; }
size_t bwd_workspace_bytes(int, int, int, int, int) { return 0; }
}  // namespace fa
