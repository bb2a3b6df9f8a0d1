// Fixed-geometry instantiations of the fused WTConv kernels (k = 5): p128b.
// Each matches one launch plan exactly (plane size, levels, planes and threads
// per workgroup); any other plan takes the runtime-geometry kernel.
#include "wtconv_fused_kernel.h"

namespace wtc {

bool launch_fused_static_p128b(const FusedArgs& a, int dtype, int bwd, int bpq, int nthr, size_t lds,
                               int grid, void* stream, int* err) {
    using namespace fused_detail;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    bool hit = false;
    // planes of exactly 128 x 128 pixels: whole-plane instances
    if (!hit && dtype == WTC_FP32 && bwd == 0)
        hit = try_static<5, float, 0, 2, true, 128, 128, 3, 1, 1, 512, 0, 0, false, true>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && dtype == WTC_FP32 && bwd == 1)
        hit = try_static<5, float, 1, 2, true, 128, 128, 3, 1, 1, 512, 0, 0, false, true>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && dtype == WTC_FP32 && bwd == 0)
        hit = try_static<5, float, 0, 2, true, 128, 128, 4, 1, 1, 512, 0, 0, false, true>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && dtype == WTC_FP32 && bwd == 1)
        hit = try_static<5, float, 1, 2, true, 128, 128, 4, 1, 1, 512, 0, 0, false, true>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && dtype == WTC_FP32 && bwd == 0)
        hit = try_static<5, float, 0, 2, true, 128, 128, 5, 1, 1, 512, 0, 0, false, true>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && dtype == WTC_FP32 && bwd == 1)
        hit = try_static<5, float, 1, 2, true, 128, 128, 5, 1, 1, 512, 0, 0, false, true>(a, bpq, nthr, lds, grid, st, &e);
    // other planes zero-extended to 128 x 128
    if (!hit && dtype == WTC_FP32 && bwd == 0)
        hit = try_static<5, float, 0, 2, true, 128, 128, 3, 1, 1, 512, 0>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && dtype == WTC_FP32 && bwd == 1)
        hit = try_static<5, float, 1, 2, true, 128, 128, 3, 1, 1, 512, 0>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && dtype == WTC_FP32 && bwd == 0)
        hit = try_static<5, float, 0, 2, true, 128, 128, 4, 1, 1, 512, 0>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && dtype == WTC_FP32 && bwd == 1)
        hit = try_static<5, float, 1, 2, true, 128, 128, 4, 1, 1, 512, 0>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && dtype == WTC_FP32 && bwd == 0)
        hit = try_static<5, float, 0, 2, true, 128, 128, 5, 1, 1, 512, 0>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && dtype == WTC_FP32 && bwd == 1)
        hit = try_static<5, float, 1, 2, true, 128, 128, 5, 1, 1, 512, 0>(a, bpq, nthr, lds, grid, st, &e);
    *err = (int)e;
    return hit;
}

}  // namespace wtc
