// Entry points whose kernels are not written yet: they report "not supported"
// instead of computing anything.
#include "fa_internal.h"

namespace fa {
hipError_t launch_fwd_fp8(const FwdArgs &, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace fa
