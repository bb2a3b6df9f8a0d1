// Fixed-geometry instantiations of the fused WTConv kernels (k = 5): small.
// Each matches one launch plan exactly (plane size, levels, planes and threads
// per workgroup); any other plan takes the runtime-geometry kernel.
#include "wtconv_fused_kernel.h"

namespace wtc {

bool launch_fused_static_small(const FusedArgs& a, int dtype, int bwd, int bpq, int nthr, size_t lds,
                               int grid, void* stream, int* err) {
    using namespace fused_detail;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    bool hit = false;
    // 14 x 14 planes (the 14 x 14 network stage): the plane size fixed at compile time
    if (!hit && dtype == WTC_FP32 && bwd == 0)
        hit = try_static<5, float, 0, 1, false, 16, 16, 2, 2, 4, 64, 0, 0, false, false, 14, 14>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && dtype == WTC_FP32 && bwd == 1)
        hit = try_static<5, float, 1, 1, false, 16, 16, 2, 2, 4, 64, 2, 0, false, false, 14, 14>(a, bpq, nthr, lds, grid, st, &e);
    // other planes of this class
    if (!hit && dtype == WTC_FP32 && bwd == 0)
        hit = try_static<5, float, 0, 1, false, 16, 16, 2, 2, 4, 64, 0>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && dtype == WTC_FP32 && bwd == 1)
        hit = try_static<5, float, 1, 1, false, 16, 16, 2, 2, 4, 64, 2>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && dtype == WTC_BF16 && bwd == 0)
        hit = try_static<5, bf16_t, 0, 1, false, 16, 16, 2, 2, 4, 64, 0>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && dtype == WTC_BF16 && bwd == 1)
        hit = try_static<5, bf16_t, 1, 1, false, 16, 16, 2, 2, 4, 64, 2>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && dtype == WTC_FP32 && bwd == 0)
        hit = try_static<5, float, 0, 1, false, 8, 8, 1, 1, 31, 128, 0>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && dtype == WTC_FP32 && bwd == 1)
        hit = try_static<5, float, 1, 1, false, 8, 8, 1, 1, 16, 64, 1>(a, bpq, nthr, lds, grid, st, &e);
    *err = (int)e;
    return hit;
}

}  // namespace wtc
