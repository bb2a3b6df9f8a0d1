// WTConv for 7 x 7 planes with one wavelet level (k = 5), one plane per lane
// (gfx950).  (The kernel template takes any plane up to 8 x 8; only 7 x 7 is
// instantiated: at 8 x 8 the backward no longer fits the register file.)
//
// A workgroup is two waves over the same 64 batch entries of one channel, so
// every weight is uniform (scalar registers) and every index into a plane is a
// compile-time constant.  Lane l of both waves holds plane l.  Forward: wave 0
// computes the base conv, wave 1 the four level-1 subbands (conv and
// synthesis) and hands its sum to wave 0 through LDS.  Backward: wave 0 all of
// dx, wave 1 all the correlations (x is needed there only).  The multiply-add
// counts of the two waves are about equal either way (841 and 784 per plane).
// (One wave per 64 planes gave 1.5 waves per SIMD on the 7 x 7 stage shapes,
// one or two per SIMD; split, the waves are half as long and three per SIMD.)
// All of it is straight-line multiply-adds over registers, with the zero
// extension and the zero padding resolved at compile time (no work on
// padding).  Planes move between device memory and registers through LDS: a
// plane is 49 contiguous values, loaded and stored one plane per wave
// instruction (coalesced), and read by its lane at an odd stride (no bank
// conflicts); each wave moves half of the planes.
//
// Same operator and conventions as the other fused kernels: raw +-1 Haar
// butterflies, level weights folded as 4^-1 s_u W_u (applied to each conv
// output), backward = the same pipeline on g with 180-degree-rotated weights,
// plus the correlations C_0[d] = sum g[p] x[p + d] and
// C_1^u[d] = sum G_u[j] X_u[j + d] (raw bands), reduced over the wave into one
// record per (batch chunk, channel): [C_0][C_1 bands 0..3][sum g][tail = 0].
#include <hip/hip_runtime.h>

#include "wtc_internal.h"
#include "wtc_numeric.h"

namespace wtc {
namespace {

constexpr int K = 5, R = 2, KK = 25;

struct bf16v {
    uint16_t bits;
};
__device__ __forceinline__ float lval(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float lval(const bf16v* p, size_t i) { return __uint_as_float(((uint32_t)p[i].bits) << 16); }
__device__ __forceinline__ void lput(float* p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void lput(bf16v* p, size_t i, float v) { p[i].bits = bf16_rne(v); }

// Value of v in lane l - N of the same 16-lane row (0 for the row's first N lanes).
template <int N>
__device__ __forceinline__ float lshr(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x110 | N, 0xF, 0xF, true));
}
// Lane 15 of every 16-lane row: the sum of v over the row.
__device__ __forceinline__ float lrow_sum(float v) {
    v += lshr<1>(v);
    v += lshr<2>(v);
    v += lshr<4>(v);
    return v + lshr<8>(v);
}

// Plane staging: planes j = j0 .. j0 + 31 of the workgroup (batch entries b0 + j
// of channel c, n valid) into lds[j * SP + e] (e < N values per plane), all 32
// loads in flight before the LDS writes.
template <int N, int SP, typename ST>
__device__ __forceinline__ void stage_in(float* lds, const ST* src, int C, int c, int b0, int n, int lane, int j0) {
    constexpr int G = 32;
    float v[G];
#pragma unroll
    for (int j = 0; j < G; ++j)
        v[j] = (lane < N && j0 + j < n) ? lval(src, ((size_t)(b0 + j0 + j) * C + c) * N + lane) : 0.f;
#pragma unroll
    for (int j = 0; j < G; ++j)
        if (lane < N) lds[(j0 + j) * SP + lane] = v[j];
}
template <int N, int SP, typename ST>
__device__ __forceinline__ void stage_out(const float* lds, ST* dst, int C, int c, int b0, int n, int lane, int j0) {
#pragma unroll 16
    for (int j = j0; j < j0 + 32; ++j)
        if (lane < N && j < n) lput(dst, ((size_t)(b0 + j) * C + c) * N + lane, lds[j * SP + lane]);
}

// Raw Haar band u of the 2 x 2 block at level-1 position (jy, jx) of an
// HP x WP plane held in registers (zero beyond the plane).
template <int HP, int WP>
__device__ __forceinline__ float band_at(const float (&P)[HP][WP], int u, int jy, int jx) {
    const int y = 2 * jy, x = 2 * jx;
    const float a = P[y][x];
    const float b = (x + 1 < WP) ? P[y][x + 1] : 0.f;
    const float c = (y + 1 < HP) ? P[y + 1][x] : 0.f;
    const float d = (y + 1 < HP && x + 1 < WP) ? P[y + 1][x + 1] : 0.f;
    switch (u) {
        case 0: return (a + b) + (c + d);
        case 1: return (a - b) + (c - d);
        case 2: return (a + b) - (c + d);
        default: return (a - b) - (c - d);
    }
}

template <typename ST, bool BWD, int HP, int WP>
__global__ void __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(3)))
k_lane(const FusedArgs a) {
    constexpr int N = HP * WP, SP = (N % 2 == 0) ? N + 1 : N;
    constexpr int H1 = (HP + 1) / 2, W1 = (WP + 1) / 2;   // level-1 grid
    constexpr int RL = 5 * KK + 1;                         // record elements with a row partial
    __shared__ float lds[64 * SP];
    __shared__ float red[4 * RL];   // backward: partials per 16-lane row
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    // Units (batch chunk, channel), chunk-major, dealt to the XCDs in
    // contiguous ranges: workgroup i runs on XCD i % 8 (workgroups are dealt to
    // the XCDs in turn), so the planes of neighbouring channels -- 196-byte
    // planes that share cache lines -- pass through one L2 at about the same
    // time instead of being fetched once per XCD.
    const int nchunk = (a.B + 63) / 64;
    const int U = a.C * nchunk, per = (U + 7) / 8;
    const int k8 = blockIdx.x >> 3, u = (blockIdx.x & 7) * per + k8;
    if (k8 >= per || u >= U) return;   // whole workgroup, before any barrier
    const int c = u % a.C, chunk = u / a.C;
    const int b0 = chunk * 64, n = min(64, a.B - b0);
    const ST* srcp = reinterpret_cast<const ST*>(a.src);
    const ST* auxp = reinterpret_cast<const ST*>(a.aux);
    ST* dstp = reinterpret_cast<ST*>(a.dst);

    // ---- this lane's plane (g in the backward); each wave stages half of the
    // planes.  Backward: x is staged next and stays in LDS until wave 1 reads it.
    float P[HP][WP];
    stage_in<N, SP, ST>(lds, srcp, a.C, c, b0, n, lane, 32 * wave);
    __syncthreads();
#pragma unroll
    for (int y = 0; y < HP; ++y)
#pragma unroll
        for (int x = 0; x < WP; ++x) P[y][x] = lds[lane * SP + y * WP + x];
    __syncthreads();   // every plane of g / x is in registers
    if constexpr (BWD) {
        stage_in<N, SP, ST>(lds, auxp, a.C, c, b0, n, lane, 32 * wave);
        __syncthreads();
    }

    // level 1, one subband at a time: raw band, conv with W_u (rotated
    // backward), scaled by 4^-1 s_u, synthesised into O (raw +-1 signs)
    auto level1 = [&](float (&O)[HP][WP]) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float Bv[H1][W1];
#pragma unroll
            for (int jy = 0; jy < H1; ++jy)
#pragma unroll
                for (int jx = 0; jx < W1; ++jx) Bv[jy][jx] = band_at<HP, WP>(P, u, jy, jx);
            const size_t pu = (size_t)c * 4 + u;
            float w[KK];
#pragma unroll
            for (int t = 0; t < KK; ++t) w[t] = a.wl[pu * KK + (BWD ? KK - 1 - t : t)];
            const float su = ldexpf(a.sl[pu], -2);
#pragma unroll
            for (int jy = 0; jy < H1; ++jy)
#pragma unroll
                for (int jx = 0; jx < W1; ++jx) {
                    float s = 0.f;
#pragma unroll
                    for (int ky = 0; ky < K; ++ky)
#pragma unroll
                        for (int kx = 0; kx < K; ++kx) {
                            const int yy = jy + ky - R, xx = jx + kx - R;
                            if (yy >= 0 && yy < H1 && xx >= 0 && xx < W1) s = fmaf(w[ky * K + kx], Bv[yy][xx], s);
                        }
                    const float yv = su * s;
                    // synthesis: pixel (2 jy + dy, 2 jx + dx) gets sign_u(dy, dx) * yv
#pragma unroll
                    for (int dy = 0; dy < 2; ++dy)
#pragma unroll
                        for (int dx = 0; dx < 2; ++dx) {
                            const int y = 2 * jy + dy, x = 2 * jx + dx;
                            if (y >= HP || x >= WP) continue;
                            const bool neg = ((u & 1) && dx) != ((u & 2) && dy);
                            O[y][x] = neg ? O[y][x] - yv : O[y][x] + yv;
                        }
                }
        }
    };

    // Forward: wave 0 the base conv, wave 1 level 1 (its synthesis sum is added
    // through LDS).  Backward: wave 0 all of dx (base and level 1), wave 1 all
    // the correlations (base, sum of g, level 1), so that no wave holds both an
    // output plane and x.
    float O[HP][WP];
    if (wave == 0) {
        // ---- base conv (rotated weights backward), zero padding resolved at compile time
        float w[KK];
#pragma unroll
        for (int t = 0; t < KK; ++t) w[t] = a.w0[(size_t)c * KK + (BWD ? KK - 1 - t : t)];
#pragma unroll
        for (int y = 0; y < HP; ++y)
#pragma unroll
            for (int x = 0; x < WP; ++x) {
                float s = 0.f;
#pragma unroll
                for (int ky = 0; ky < K; ++ky)
#pragma unroll
                    for (int kx = 0; kx < K; ++kx) {
                        const int yy = y + ky - R, xx = x + kx - R;
                        if (yy >= 0 && yy < HP && xx >= 0 && xx < WP) s = fmaf(w[ky * K + kx], P[yy][xx], s);
                    }
                O[y][x] = s;
            }
        const float s0 = a.s0[c], bias = BWD ? 0.f : a.b0[c];
#pragma unroll
        for (int y = 0; y < HP; ++y)
#pragma unroll
            for (int x = 0; x < WP; ++x) O[y][x] = fmaf(s0, O[y][x], bias);
        if constexpr (BWD) level1(O);
    } else if constexpr (!BWD) {
#pragma unroll
        for (int y = 0; y < HP; ++y)
#pragma unroll
            for (int x = 0; x < WP; ++x) O[y][x] = 0.f;
        level1(O);
        // the level-1 synthesis sum to wave 0 (every plane was read before the
        // barrier above)
#pragma unroll
        for (int y = 0; y < HP; ++y)
#pragma unroll
            for (int x = 0; x < WP; ++x) lds[lane * SP + y * WP + x] = O[y][x];
    } else {
        // ---- correlations: C_0 and sum of g, then C_1 per subband, each reduced
        // per 16-lane row into the row partials
        float X[HP][WP];
#pragma unroll
        for (int y = 0; y < HP; ++y)
#pragma unroll
            for (int x = 0; x < WP; ++x) X[y][x] = lds[lane * SP + y * WP + x];
        {
            float C0[KK], sg = 0.f;
#pragma unroll
            for (int t = 0; t < KK; ++t) C0[t] = 0.f;
#pragma unroll
            for (int y = 0; y < HP; ++y)
#pragma unroll
                for (int x = 0; x < WP; ++x) {
                    sg += P[y][x];
#pragma unroll
                    for (int ky = 0; ky < K; ++ky)
#pragma unroll
                        for (int kx = 0; kx < K; ++kx) {
                            const int yy = y + ky - R, xx = x + kx - R;
                            if (yy >= 0 && yy < HP && xx >= 0 && xx < WP)
                                C0[ky * K + kx] = fmaf(P[y][x], X[yy][xx], C0[ky * K + kx]);
                        }
                }
#pragma unroll
            for (int t = 0; t < KK; ++t) C0[t] = lrow_sum(C0[t]);
            sg = lrow_sum(sg);
            if ((lane & 15) == 15) {
                const int row = lane >> 4;
#pragma unroll
                for (int t = 0; t < KK; ++t) red[row * RL + t] = C0[t];
                red[row * RL + 5 * KK] = sg;
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float Bv[H1][W1], Xv[H1][W1], C1[KK];
#pragma unroll
            for (int jy = 0; jy < H1; ++jy)
#pragma unroll
                for (int jx = 0; jx < W1; ++jx) {
                    Bv[jy][jx] = band_at<HP, WP>(P, u, jy, jx);
                    Xv[jy][jx] = band_at<HP, WP>(X, u, jy, jx);
                }
#pragma unroll
            for (int t = 0; t < KK; ++t) C1[t] = 0.f;
#pragma unroll
            for (int jy = 0; jy < H1; ++jy)
#pragma unroll
                for (int jx = 0; jx < W1; ++jx)
#pragma unroll
                    for (int ky = 0; ky < K; ++ky)
#pragma unroll
                        for (int kx = 0; kx < K; ++kx) {
                            const int yy = jy + ky - R, xx = jx + kx - R;
                            if (yy >= 0 && yy < H1 && xx >= 0 && xx < W1)
                                C1[ky * K + kx] = fmaf(Bv[jy][jx], Xv[yy][xx], C1[ky * K + kx]);
                        }
#pragma unroll
            for (int t = 0; t < KK; ++t) C1[t] = lrow_sum(C1[t]);
            if ((lane & 15) == 15) {
                const int row = lane >> 4;
#pragma unroll
                for (int t = 0; t < KK; ++t) red[row * RL + KK + u * KK + t] = C1[t];
            }
        }
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int y = 0; y < HP; ++y)
#pragma unroll
            for (int x = 0; x < WP; ++x) {
                float* q = lds + lane * SP + y * WP + x;
                *q = BWD ? O[y][x] : O[y][x] + *q;
            }
    }
    // ---- records (backward): the row partials of both waves, summed in row order
    if constexpr (BWD) {
        float* rec = a.partials + ((size_t)chunk * a.C + c) * a.P;
        for (int e = threadIdx.x; e < a.P; e += 128) {
            float v = 0.f;
            if (e < RL)
#pragma unroll
                for (int row = 0; row < 4; ++row) v += red[row * RL + e];
            rec[e] = v;   // e = P - 1: tail term, 0 (every level is on a grid larger than 1 x 1)
        }
    }
    __syncthreads();
    stage_out<N, SP, ST>(lds, dstp, a.C, c, b0, n, lane, 32 * wave);
}

template <typename ST, bool BWD>
hipError_t lane_launch(const FusedArgs& a, int grid, hipStream_t st) {
    hipLaunchKernelGGL((k_lane<ST, BWD, 7, 7>), dim3(grid), dim3(128), 0, st, a);
    return hipGetLastError();
}

}  // namespace

int launch_lane(const FusedArgs& a, int dtype, int bwd, int grid, void* stream) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (dtype == WTC_BF16)
        return (int)(bwd ? lane_launch<bf16v, true>(a, grid, st) : lane_launch<bf16v, false>(a, grid, st));
    return (int)(bwd ? lane_launch<float, true>(a, grid, st) : lane_launch<float, false>(a, grid, st));
}

}  // namespace wtc
