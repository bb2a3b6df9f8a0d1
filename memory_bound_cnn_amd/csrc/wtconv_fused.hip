// Fused WTConv: dispatch over the kernel size, and the backward finalize
// kernel (deterministic cross-workgroup sum and chain rule through the folds).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "wtc_internal.h"

namespace wtc {

int launch_fused_rt_k1(const FusedArgs&, int, int, int, int, size_t, int, void*);
int launch_fused_rt_k3(const FusedArgs&, int, int, int, int, size_t, int, void*);
int launch_fused_rt_k5(const FusedArgs&, int, int, int, int, size_t, int, void*);
int launch_fused_rt_k7(const FusedArgs&, int, int, int, int, size_t, int, void*);
bool launch_fused_static_p64(const FusedArgs&, int, int, int, int, size_t, int, void*, int*);
bool launch_fused_static_p32(const FusedArgs&, int, int, int, int, size_t, int, void*, int*);
bool launch_fused_static_p128a(const FusedArgs&, int, int, int, int, size_t, int, void*, int*);
bool launch_fused_static_p128b(const FusedArgs&, int, int, int, int, size_t, int, void*, int*);
bool launch_fused_static_small(const FusedArgs&, int, int, int, int, size_t, int, void*, int*);
bool launch_fused_static_p112(const FusedArgs&, int, int, int, int, size_t, int, void*, int*);
bool launch_fused_static_dw(const FusedArgs&, int, int, int, int, int, size_t, int, void*, int*);

namespace {

// ---------------------------------------------------------------------------
// Finalize: deterministic sum over chunks, then the chain rule through the folds
// dW = 4^-i s C, ds = 4^-i sum_d W C (level 0: dW0 = s0 C_0, ds0 = sum W0 C_0).
// ---------------------------------------------------------------------------
// Parameters of chain-rule element e: its weight and the fold factor of its
// correlation (e < k^2: W0 and s0; else level i, band u, tap: W_i and 4^-i s_i).
__device__ __forceinline__ void fin_param(const FinalizeArgs& f, int c, int KK, int e, float& w, float& sc) {
    if (e < KK) {
        w = f.w0[(size_t)c * KK + e];
        sc = f.s0[c];
    } else {
        const int r = e - KK;
        const int i = r / (4 * KK), rem = r - i * 4 * KK, u = rem / KK, tap = rem - u * KK;
        const size_t pi = ((size_t)i * f.C + c) * 4 + u;
        w = f.wl[pi * KK + tap];
        sc = ldexpf(f.sl[pi], -2 * (i + 1));
    }
}

__global__ void __launch_bounds__(1024) wtc_finalize_kernel(const FinalizeArgs f) {
    extern __shared__ __align__(16) float tot[];
    const int c = blockIdx.x, tid = threadIdx.x, nthr = blockDim.x;
    const int KK = f.k * f.k;
    const int n0 = KK * (1 + 4 * f.L);   // chain-rule elements: [level 0 | levels 1..L x 4 bands][tap]
    // The launch gives one thread per element where it can (<= 1024): the
    // parameters of a thread's first element are loaded before the record sums,
    // and every record load of an element is in flight at once, so the kernel
    // waits for about one memory round trip.
    float w_first = 0.f, sc_first = 0.f;
    if (tid < n0) fin_param(f, c, KK, tid, w_first, sc_first);
    // records of channel c: workgroups whose plane range meets [c*B, (c+1)*B);
    // segment 0 if the range starts in channel c (w*ppw >= c*B), else segment 1.
    // Summed in a fixed order (deterministic).
    const int w_lo = (int)(((long)c * f.B) / f.ppw);
    const int w_hi = (int)(((long)(c + 1) * f.B - 1) / f.ppw);
    const long cB = (long)c * f.B;
    for (int e = tid; e < f.P; e += nthr) {
        float v = 0.f;
        if (f.chunks > 0) {
            // small-plane kernel: one record per (batch chunk, channel)
#pragma unroll 8
            for (int j = 0; j < f.chunks; ++j) v += f.partials[((size_t)j * f.C + c) * f.P + e];
        } else {
#pragma unroll 8
            for (int w = w_lo; w <= w_hi; ++w) {
                const int seg = (long)w * f.ppw >= cB ? 0 : 1;
                v += f.partials[((size_t)w * 2 + seg) * f.P + e];
            }
        }
        tot[e] = v;
    }
    __syncthreads();
    const float tail = tot[f.P - 1];
    // scale gradients are dot products of the weights with the correlations:
    // products staged in LDS, then one short sum per scale
    float* prod = tot + ((f.P + 3) & ~3);
    for (int e = tid; e < n0; e += nthr) {
        float w = w_first, sc = sc_first;
        if (e != tid) fin_param(f, c, KK, e, w, sc);
        float cv;
        if (e < KK) {
            cv = tot[e];
            f.dw0[(size_t)c * KK + e] = sc * cv;
        } else {
            const int r = e - KK;
            const int i = r / (4 * KK), rem = r - i * 4 * KK, u = rem / KK, tap = rem - u * KK;
            cv = (i < f.Lm) ? tot[e] : ((tap == KK / 2) ? tail : 0.f);
            f.dwl[(((size_t)i * f.C + c) * 4 + u) * KK + tap] = sc * cv;
        }
        prod[e] = w * cv;
    }
    __syncthreads();
    for (int e = tid; e < 1 + 4 * f.L; e += nthr) {
        float s = 0.f;
        for (int tap = 0; tap < KK; ++tap) s += prod[e * KK + tap];
        if (e == 0) {
            f.ds0[c] = s;
            f.db0[c] = tot[f.P - 2];
        } else {
            const int i = (e - 1) >> 2, u = (e - 1) & 3;
            f.dsl[((size_t)i * f.C + c) * 4 + u] = ldexpf(s, -2 * (i + 1));
        }
    }
}

}  // namespace

int launch_fused(const FusedArgs& a, int k, int dtype, int bwd, int bpq, int nthr, size_t lds_bytes,
                 int grid, void* stream) {
    if (k == 5 || k == 7) {
        int err = 0;
        if (launch_fused_static_dw(a, k, dtype, bwd, bpq, nthr, lds_bytes, grid, stream, &err)) return err;
    }
    if (k == 5) {
        // fixed-geometry kernels for the plane classes compiled in; else runtime geometry
        int err = 0;
        if (launch_fused_static_p64(a, dtype, bwd, bpq, nthr, lds_bytes, grid, stream, &err) ||
            launch_fused_static_p32(a, dtype, bwd, bpq, nthr, lds_bytes, grid, stream, &err) ||
            launch_fused_static_p128a(a, dtype, bwd, bpq, nthr, lds_bytes, grid, stream, &err) ||
            launch_fused_static_p128b(a, dtype, bwd, bpq, nthr, lds_bytes, grid, stream, &err) ||
            launch_fused_static_p112(a, dtype, bwd, bpq, nthr, lds_bytes, grid, stream, &err) ||
            launch_fused_static_small(a, dtype, bwd, bpq, nthr, lds_bytes, grid, stream, &err))
            return err;
    }
    switch (k) {
        case 1: return launch_fused_rt_k1(a, dtype, bwd, bpq, nthr, lds_bytes, grid, stream);
        case 3: return launch_fused_rt_k3(a, dtype, bwd, bpq, nthr, lds_bytes, grid, stream);
        case 5: return launch_fused_rt_k5(a, dtype, bwd, bpq, nthr, lds_bytes, grid, stream);
        case 7: return launch_fused_rt_k7(a, dtype, bwd, bpq, nthr, lds_bytes, grid, stream);
        default: return (int)hipErrorInvalidValue;
    }
}

int launch_finalize(const FinalizeArgs& f, void* stream) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int n0 = f.k * f.k * (1 + 4 * f.L);
    const size_t lds = ((size_t)((f.P + 3) & ~3) + (size_t)n0) * sizeof(float);
    const int nthr = std::min(1024, (std::max(f.P, n0) + 63) / 64 * 64);
    hipLaunchKernelGGL(wtc_finalize_kernel, dim3(f.C), dim3(nthr), lds, st, f);
    return (int)hipGetLastError();
}

}  // namespace wtc
