// Internal declarations of the split-key forward (fa_fwd_split.hip): short
// causal bf16 calls without a window or dropout run 32-row work-groups whose
// 4 waves split the keys.  Used by the C-ABI layer (fa_api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {

constexpr int kFwdSplitRows = 32;        // query rows per work-group
constexpr int kFwdSplitMaxRows = 2048;   // longest Nq and Nk it takes
// whether a call takes the split-key launch (cus: the device's CUs)
bool fwd_split_keys(int causal, int window, uint32_t drop_k, int64_t nq, int64_t nk, int64_t batch_heads, int cus);
hipError_t launch_fwd_bf16_split(const FwdArgs &a, int head_dim, hipStream_t s);

}  // namespace fa
