// Level-by-level WTConv baseline (placeholder until the baseline kernels land).
#include <hip/hip_runtime.h>

#include "wtc_internal.h"

namespace wtc {
int unfused_plan(const wtc_desc*, int, UnfusedPlan*) { return WTC_EINVAL; }
int unfused_forward(const wtc_desc*, const UnfusedPlan&, const void*, const float*, const float*,
                    const float*, const float*, const float*, void*, char*, void*) {
    return WTC_EINVAL;
}
int unfused_backward(const wtc_desc*, const UnfusedPlan&, const void*, const void*, const float*,
                     const float*, const float*, const float*, void*, float*, float*, float*,
                     float*, float*, char*, void*) {
    return WTC_EINVAL;
}
}  // namespace wtc
