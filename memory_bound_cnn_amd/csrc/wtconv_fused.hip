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
// Lanes per scale group in the chain-rule phase: the smallest power of two
// that holds the k^2 taps (one wave at most), so each scale's sum W.C is a
// butterfly within its lanes.
template <int K>
constexpr int fin_group() {
    return K * K <= 1 ? 1 : K * K <= 4 ? 4 : K * K <= 16 ? 16 : K * K <= 32 ? 32 : 64;
}

// One workgroup per channel. Chain-rule group g in [0, 1 + 4L): g = 0 is level
// 0 (W0, s0), g = 1 + 4i + u is level i + 1, band u (W_i, 4^-(i+1) s_i).
template <int K>
__global__ void __launch_bounds__(1024) wtc_finalize_kernel(const FinalizeArgs f) {
    constexpr int KK = K * K, GS = fin_group<K>();
    extern __shared__ __align__(16) float tot[];
    const int c = blockIdx.x, tid = threadIdx.x, nthr = blockDim.x;
    const int ng = 1 + 4 * f.L, tap = tid % GS;
    auto param = [&](int g, float& w, float& sc) {
        w = 0.f;
        sc = 0.f;
        if (tap >= KK || g >= ng) return;
        if (g == 0) {
            w = f.w0[(size_t)c * KK + tap];
            sc = f.s0[c];
        } else {
            const int i = (g - 1) >> 2, u = (g - 1) & 3;
            const size_t pi = ((size_t)i * f.C + c) * 4 + u;
            w = f.wl[pi * KK + tap];
            sc = ldexpf(f.sl[pi], -2 * (i + 1));
        }
    };
    // the parameters of a thread's first group are loaded before the record
    // sums, and every record load of an element is in flight at once, so the
    // kernel waits for about one memory round trip
    float w, sc;
    param(tid / GS, w, sc);
    // records of channel c: workgroups whose plane range meets [c*B, (c+1)*B);
    // segment 0 if the range starts in channel c (w*ppw >= c*B), else segment 1.
    // Summed in a fixed order (deterministic).
    const int w_lo = (int)(((long)c * f.B) / f.ppw);
    const int w_hi = (int)(((long)(c + 1) * f.B - 1) / f.ppw);
    const long cB = (long)c * f.B;
    for (int e = tid; e < f.P; e += nthr) {
        float v = 0.f;
        if (f.chunks > 0) {
            // small-plane kernels: one record per (batch chunk, channel)
#pragma unroll 8
            for (int j = 0; j < f.chunks; ++j) v += f.partials[((size_t)j * f.C + c) * f.P + e];
        } else {
#pragma unroll 8
            for (int wg = w_lo; wg <= w_hi; ++wg) {
                const int seg = (long)wg * f.ppw >= cB ? 0 : 1;
                v += f.partials[((size_t)wg * 2 + seg) * f.P + e];
            }
        }
        tot[e] = v;
    }
    __syncthreads();
    const float tail = tot[f.P - 1];
    // groups whose level has no record (a 1x1 grid: the tail) keep the centre tap only
    for (int g = tid / GS; g < ng; g += nthr / GS) {
        if (g != tid / GS) param(g, w, sc);
        float cv = 0.f;
        if (tap < KK) {
            if (g == 0) {
                cv = tot[tap];
                f.dw0[(size_t)c * KK + tap] = sc * cv;
            } else {
                const int i = (g - 1) >> 2, u = (g - 1) & 3;
                cv = (i < f.Lm) ? tot[g * KK + tap] : ((tap == KK / 2) ? tail : 0.f);
                f.dwl[(((size_t)i * f.C + c) * 4 + u) * KK + tap] = sc * cv;
            }
        }
        // scale gradient: sum over the group's taps of W * C
        float p = w * cv;
#pragma unroll
        for (int m = GS / 2; m >= 1; m >>= 1) p += __shfl_xor(p, m, GS);
        if (tap == 0) {
            if (g == 0) {
                f.ds0[c] = p;
                f.db0[c] = tot[f.P - 2];
            } else {
                const int i = (g - 1) >> 2, u = (g - 1) & 3;
                f.dsl[((size_t)i * f.C + c) * 4 + u] = ldexpf(p, -2 * (i + 1));
            }
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
    const size_t lds = (size_t)f.P * sizeof(float);
    const int ng = 1 + 4 * f.L;
    auto go = [&](auto kern, int gs) {
        // whole groups per workgroup, at least one pass over the record elements
        const int nthr = std::min(1024, (std::max(f.P, ng * gs) + 63) / 64 * 64);
        hipLaunchKernelGGL(kern, dim3(f.C), dim3(nthr), lds, st, f);
        return (int)hipGetLastError();
    };
    switch (f.k) {
        case 1: return go(wtc_finalize_kernel<1>, fin_group<1>());
        case 3: return go(wtc_finalize_kernel<3>, fin_group<3>());
        case 5: return go(wtc_finalize_kernel<5>, fin_group<5>());
        case 7: return go(wtc_finalize_kernel<7>, fin_group<7>());
        default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace wtc
