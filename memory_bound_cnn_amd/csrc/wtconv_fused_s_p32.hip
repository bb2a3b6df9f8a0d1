// Fixed-geometry instantiations of the fused WTConv kernels (k = 5): p32.
// Each matches one launch plan exactly (plane size, levels, planes and threads
// per workgroup); any other plan takes the runtime-geometry kernel.
#include "wtconv_fused_kernel.h"

namespace wtc {

bool launch_fused_static_p32(const FusedArgs& a, int dtype, int bwd, int bpq, int nthr, size_t lds,
                               int grid, void* stream, int* err) {
    using namespace fused_detail;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    bool hit = false;
    // planes of exactly 32 x 32 pixels: whole-plane instances
    if (!hit && dtype == WTC_BF16 && bwd == 0)
        hit = try_static<5, bf16_t, 0, 1, true, 32, 32, 3, 3, 1, 64, 1, 0, false, true>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && dtype == WTC_BF16 && bwd == 1)
        hit = try_static<5, bf16_t, 1, 1, true, 32, 32, 3, 3, 1, 64, 0, 1, false, true>(a, bpq, nthr, lds, grid, st, &e);
    // other planes of this class
    if (!hit && dtype == WTC_FP32 && bwd == 0)
        hit = try_static<5, float, 0, 1, true, 32, 32, 2, 2, 1, 64, 0, 1>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && dtype == WTC_FP32 && bwd == 1)
        hit = try_static<5, float, 1, 1, true, 32, 32, 2, 2, 1, 64, 0, 1>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && dtype == WTC_FP32 && bwd == 0)
        hit = try_static<5, float, 0, 1, true, 32, 32, 3, 3, 1, 64, 0, 1>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && dtype == WTC_FP32 && bwd == 1)
        hit = try_static<5, float, 1, 1, true, 32, 32, 3, 3, 1, 64, 0, 1>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && dtype == WTC_BF16 && bwd == 0)
        hit = try_static<5, bf16_t, 0, 1, true, 32, 32, 3, 3, 1, 64, 1, 0>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && dtype == WTC_BF16 && bwd == 1)
        hit = try_static<5, bf16_t, 1, 1, true, 32, 32, 3, 3, 1, 64, 0, 1>(a, bpq, nthr, lds, grid, st, &e);
    *err = (int)e;
    return hit;
}

}  // namespace wtc
