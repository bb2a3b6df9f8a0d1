// Fixed-geometry instantiations of the fused kernels with no wavelet levels
// (L = 0: a plain depthwise k x k convolution with scale and bias) on fp32
// planes, k = 5 and k = 7: 64 x 64 in direct-load mode, 128 x 128 with two
// blocks per quad.  These are the depthwise convolutions that WTConv is
// measured against.
#include "wtconv_fused_kernel.h"

namespace wtc {

bool launch_fused_static_dw(const FusedArgs& a, int k, int dtype, int bwd, int bpq, int nthr, size_t lds,
                            int grid, void* stream, int* err) {
    using namespace fused_detail;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    bool hit = false;
    if (dtype != WTC_FP32 || a.L != 0) return false;
    if (!hit && k == 5 && bwd == 0)
        hit = try_static<5, float, 0, 1, true, 64, 64, 0, 0, 1, 256, 0, 1>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && k == 5 && bwd == 1)
        hit = try_static<5, float, 1, 1, true, 64, 64, 0, 0, 1, 256, 0, 1>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && k == 7 && bwd == 0)
        hit = try_static<7, float, 0, 1, true, 64, 64, 0, 0, 1, 256, 0, 1>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && k == 7 && bwd == 1)
        hit = try_static<7, float, 1, 1, true, 64, 64, 0, 0, 1, 256, 0, 1>(a, bpq, nthr, lds, grid, st, &e);
    // 128 x 128 planes: two blocks per quad, 512 threads
    if (!hit && k == 5 && bwd == 0)
        hit = try_static<5, float, 0, 2, true, 128, 128, 0, 0, 1, 512, 0>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && k == 5 && bwd == 1)
        hit = try_static<5, float, 1, 2, true, 128, 128, 0, 0, 1, 512, 0>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && k == 7 && bwd == 0)
        hit = try_static<7, float, 0, 2, true, 128, 128, 0, 0, 1, 512, 0>(a, bpq, nthr, lds, grid, st, &e);
    if (!hit && k == 7 && bwd == 1)
        hit = try_static<7, float, 1, 2, true, 128, 128, 0, 0, 1, 512, 0>(a, bpq, nthr, lds, grid, st, &e);
    *err = (int)e;
    return hit;
}

}  // namespace wtc
