// Runtime-geometry instantiations of the fused WTConv kernels for k = 3.
#include "wtconv_fused_kernel.h"

namespace wtc {

int launch_fused_rt_k3(const FusedArgs& a, int dtype, int bwd, int bpq, int nthr, size_t lds, int grid,
                       void* stream) {
    return (int)fused_detail::launch_rt<3>(a, dtype, bwd, bpq, nthr, lds, grid,
                                            reinterpret_cast<hipStream_t>(stream));
}

}  // namespace wtc
