// Fixed-geometry instantiations of the fused WTConv kernels (k = 5): 112 x 112
// planes with two levels (the level-1 LL band of 224 x 224 planes, which the
// peeled path runs through the on-chip pipeline).  Each matches one launch
// plan exactly; any other plan takes the runtime-geometry kernel.
#include "wtconv_fused_kernel.h"

namespace wtc {

bool launch_fused_static_p112(const FusedArgs& a, int dtype, int bwd, int bpq, int nthr, size_t lds, int grid,
                              void* stream, int* err) {
    using namespace fused_detail;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    bool hit = false;
    if (!hit && dtype == WTC_FP32 && bwd == 0)
        hit = try_static<5, float, 0, 2, true, 112, 112, 2, 2, 1, 512, 0>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && dtype == WTC_FP32 && bwd == 1)
        hit = try_static<5, float, 1, 2, true, 112, 112, 2, 2, 1, 512, 0>(a, bpq, nthr, lds, grid, st, &e);
    *err = (int)e;
    return hit;
}

}  // namespace wtc
