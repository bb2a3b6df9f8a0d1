// Level-by-level WTConv baseline for gfx950: one kernel per step of the
// cascade, with every intermediate (subbands, convolution outputs, partial
// syntheses) stored in device memory in float32.  This is the execution
// structure that "Fast and Memory-Efficient Wavelet Convolutions via
// I/O-Aware Reformulation" (abstract) describes for the original WTConv: the
// same operator, its intermediates travelling through HBM between steps.
//
// Forward:  analysis L times -> scaled subband conv per level -> synthesis L
//           times (deepest first) -> base conv + bias + Z_1.
// Backward: analysis cascade of g (adjoint of the synthesis), analysis cascade
//           of x, per level the rotated subband conv and the weight-gradient
//           correlation, synthesis of the subband gradients (adjoint of the
//           analysis), base rotated conv + correlation; a small kernel per
//           level applies the chain rule through the scales.
//
// The stencil kernels stage tiles in LDS and unroll for the kernel size, and
// the elementwise ones stream, so the baseline is limited by the HBM round
// trips of its intermediates rather than by its own arithmetic.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "wtc_internal.h"
#include "wtc_numeric.h"

namespace wtc {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float ldv(const float* p, uint32_t i) { return p[i]; }
__device__ __forceinline__ float ldv(const uint16_t* p, uint32_t i) {
    return __uint_as_float(((uint32_t)p[i]) << 16);
}
__device__ __forceinline__ void stv(float* p, uint32_t i, float v) { p[i] = v; }
// four consecutive values at a 4-element aligned index
__device__ __forceinline__ void st4(float* p, uint32_t i, const float (&v)[4]) {
    *reinterpret_cast<float4*>(p + i) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint32_t bf16_bits(float v) { return bf16_rne(v); }
__device__ __forceinline__ void st4(uint16_t* p, uint32_t i, const float (&v)[4]) {
    *reinterpret_cast<uint2*>(p + i) = make_uint2(bf16_bits(v[0]) | (bf16_bits(v[1]) << 16),
                                                  bf16_bits(v[2]) | (bf16_bits(v[3]) << 16));
}
__device__ __forceinline__ void stv(uint16_t* p, uint32_t i, float v) { p[i] = (uint16_t)bf16_rne(v); }

uint32_t blocks_for(uint64_t n) {
    const uint64_t b = (n + kThreads - 1) / kThreads;
    return (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>(b, 1u << 20));
}

// One level of the orthonormal 2x2 Haar analysis.  Input plane p is
// in[p * in_ps + y * w_in + x] (h_in x w_in, zero beyond: the pad to even);
// output out[(p * 4 + u) * h_o * w_o + j], u = 2 u_y + u_x.
template <typename T>
__global__ void __launch_bounds__(kThreads) k_analysis(const T* __restrict__ in, uint32_t in_ps, uint32_t n,
                                                       int h_in, int w_in, float* __restrict__ out, int h_o,
                                                       int w_o) {
    for (uint32_t e = blockIdx.x * kThreads + threadIdx.x; e < n; e += gridDim.x * kThreads) {
        const uint32_t jx = e % (uint32_t)w_o;
        const uint32_t t = e / (uint32_t)w_o;
        const uint32_t jy = t % (uint32_t)h_o;
        const uint32_t p = t / (uint32_t)h_o;
        const uint32_t base = p * in_ps;
        const int y = 2 * (int)jy, x = 2 * (int)jx;
        const bool rx = x + 1 < w_in, ry = y + 1 < h_in;
        const float a = ldv(in, base + y * w_in + x);
        const float b = rx ? ldv(in, base + y * w_in + x + 1) : 0.f;
        const float c = ry ? ldv(in, base + (y + 1) * w_in + x) : 0.f;
        const float d = (rx && ry) ? ldv(in, base + (y + 1) * w_in + x + 1) : 0.f;
        const uint32_t bs = (uint32_t)h_o * w_o;
        const uint32_t o = p * 4 * bs + jy * w_o + jx;
        out[o] = 0.5f * ((a + b) + (c + d));
        out[o + bs] = 0.5f * ((a - b) + (c - d));
        out[o + 2 * bs] = 0.5f * ((a + b) - (c + d));
        out[o + 3 * bs] = 0.5f * ((a - b) - (c - d));
    }
}

// Tiling of one level's planes for the LDS-staged stencil kernels.  A
// workgroup stages NPB planes (consecutive planes for the convolutions, the
// same channel across the batch for the correlation) and one TH x TW tile of
// each, with a halo of R = k/2, in LDS; each thread then produces 4 vertically
// adjacent outputs of one column per work item.
struct Tile {
    int h, w;       // plane
    int TH, TW;     // output tile
    int ntx, nty;   // tiles per plane along x and y
    int NPB;        // planes per workgroup
    int NRG;        // 4-row groups per tile (rows staged: 4 NRG + 2 halo)
};

constexpr int kTileOut = 2048;                  // outputs per workgroup (target)
constexpr size_t kTileLdsBytes = 48 * 1024;     // LDS per workgroup (cap)

size_t tile_lds_floats(const Tile& t, int k, bool corr) {
    const int R = k / 2;
    const size_t halo_tile = (size_t)(4 * t.NRG + 2 * R) * (t.TW + 2 * R);
    if (corr) return (size_t)t.NPB * (4 * t.NRG * t.TW + halo_tile);
    return (size_t)t.NPB * (k * k + 2 + halo_tile);
}

Tile make_tile(int h, int w, int k, bool corr) {
    Tile t;
    t.h = h;
    t.w = w;
    t.TW = std::min(w, 64);
    t.TH = std::min(h, 32);
    t.ntx = (w + t.TW - 1) / t.TW;
    t.nty = (h + t.TH - 1) / t.TH;
    t.NRG = (t.TH + 3) / 4;
    t.NPB = std::max(1, std::min(256, kTileOut / (t.TH * t.TW)));
    while (t.NPB > 1 && tile_lds_floats(t, k, corr) * sizeof(float) > kTileLdsBytes) --t.NPB;
    return t;
}

// Incremental walk over a [n2][n1][n0] index space in flat steps of `step`
// (avoids a division per element).
struct Walk3 {
    int i0, i1, i2, d0, d1, d2, n0, n1;
    __device__ Walk3(int start, int step, int n0_, int n1_) : n0(n0_), n1(n1_) {
        i0 = start % n0;
        const int r = start / n0;
        i1 = r % n1;
        i2 = r / n1;
        d0 = step % n0;
        const int q = step / n0;
        d1 = q % n1;
        d2 = q / n1;
    }
    __device__ void next() {
        i0 += d0;
        i1 += d1;
        i2 += d2;
        if (i0 >= n0) { i0 -= n0; ++i1; }
        if (i1 >= n1) { i1 -= n1; ++i2; }
    }
};

// Stage planes p0 + j * pstride (j < np_valid; zero for j >= np_valid) of the
// h x w tensor `src`, rows ty0 - halo .. ty0 + 4 NRG + halo - 1 and columns
// tx0 - halo .. tx0 + TW + halo - 1, zero outside the plane, into
// lds[j][row][col] (row stride TW + 2 halo).
template <typename T>
__device__ void stage(float* lds, const T* __restrict__ src, int p0, int pstride, int np_valid, const Tile& t,
                      int ty0, int tx0, int halo) {
    const int RH = 4 * t.NRG + 2 * halo, SW = t.TW + 2 * halo;
    const int total = t.NPB * RH * SW;
    const uint32_t hw = (uint32_t)t.h * t.w;
    Walk3 it(threadIdx.x, kThreads, SW, RH);
    // four elements per thread in flight: their loads are issued before any of
    // their LDS writes, so one wait covers four loads
    constexpr int U = 4;
    for (int f0 = threadIdx.x; f0 < total; f0 += U * kThreads) {
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int y = ty0 + it.i1 - halo, x = tx0 + it.i0 - halo;
            v[u] = 0.f;
            if (f0 + u * kThreads < total && it.i2 < np_valid && y >= 0 && y < t.h && x >= 0 && x < t.w)
                v[u] = ldv(src, (uint32_t)(p0 + it.i2 * pstride) * hw + (uint32_t)(y * t.w + x));
            it.next();
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (f0 + u * kThreads < total) lds[f0 + u * kThreads] = v[u];
    }
}

// Depthwise K x K cross-correlation (weights rotated by 180 degrees if ROT) of
// P planes, channel ch = p % nch, zero padding K/2:
//   out[p] = scale[ch] * (W[ch] * in[p]) + bias[ch] + Z[p]   (bias, Z optional)
// 1-D grid: workgroup = (plane group, tile).
template <int K, bool ROT, typename TI, typename TO>
__global__ void __launch_bounds__(kThreads) k_tconv(const TI* __restrict__ in, int P, int nch, Tile t,
                                                    const float* __restrict__ wt, const float* __restrict__ scale,
                                                    const float* __restrict__ bias, const float* __restrict__ Z,
                                                    TO* __restrict__ out) {
    extern __shared__ float lds[];
    constexpr int R = K / 2, KK = K * K, NR = 4 + 2 * R;
    const int ntile = t.ntx * t.nty;
    const int g = blockIdx.x / ntile, tile = blockIdx.x - g * ntile;
    const int ty0 = (tile / t.ntx) * t.TH, tx0 = (tile % t.ntx) * t.TW;
    const int p0 = g * t.NPB;
    const int npv = min(t.NPB, P - p0);
    float* wl = lds;                        // [NPB][KK + 2]: weights, scale, bias
    float* xs = lds + t.NPB * (KK + 2);     // [NPB][4 NRG + 2R][TW + 2R]
    for (int f = threadIdx.x; f < npv * (KK + 2); f += kThreads) {
        const int j = f / (KK + 2), d = f - j * (KK + 2);
        const int ch = (p0 + j) % nch;
        float v;
        if (d < KK) v = wt[ch * KK + (ROT ? KK - 1 - d : d)];
        else if (d == KK) v = scale[ch];
        else v = bias ? bias[ch] : 0.f;
        wl[f] = v;
    }
    stage(xs, in, p0, 1, npv, t, ty0, tx0, R);
    __syncthreads();
    const int SW = t.TW + 2 * R, RH = 4 * t.NRG + 2 * R;
    const int total = t.NPB * t.NRG * t.TW;
    const uint32_t hw = (uint32_t)t.h * t.w;
    Walk3 it(threadIdx.x, kThreads, t.TW, t.NRG);
    for (int f = threadIdx.x; f < total; f += kThreads, it.next()) {
        const int j = it.i2, rg = it.i1, c = it.i0;
        if (j >= npv) continue;
        const float* wp = wl + j * (KK + 2);
        const float* xb = xs + (j * RH + rg * 4) * SW + c;
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int xr = 0; xr < NR; ++xr) {
            float xv[K];
#pragma unroll
            for (int kx = 0; kx < K; ++kx) xv[kx] = xb[xr * SW + kx];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int ky = xr - q;
                if (ky < 0 || ky >= K) continue;
#pragma unroll
                for (int kx = 0; kx < K; ++kx) acc[q] = fmaf(wp[ky * K + kx], xv[kx], acc[q]);
            }
        }
        const float sc = wp[KK], bi = wp[KK + 1];
        const uint32_t pbase = (uint32_t)(p0 + j) * hw;
        const int x = tx0 + c;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = rg * 4 + q, y = ty0 + r;
            if (r < t.TH && y < t.h && x < t.w) {
                const uint32_t o = pbase + (uint32_t)(y * t.w + x);
                float v = fmaf(sc, acc[q], bi);
                if (Z) v += Z[o];
                stv(out, o, v);
            }
        }
    }
}

// Inverse Haar of one level cropped to h_up x w_up: T^0 = Y^0 + Zd (Zd, on the
// h x w grid, is optional).  The 2x2 orthonormal matrix is its own inverse;
// one thread writes the 2x2 output block of one coarse position.
__global__ void __launch_bounds__(kThreads) k_synthesis(const float* __restrict__ Y, const float* __restrict__ Zd,
                                                        uint32_t n, int h, int w, float* __restrict__ Z, int h_up,
                                                        int w_up) {
    for (uint32_t e = blockIdx.x * kThreads + threadIdx.x; e < n; e += gridDim.x * kThreads) {
        const uint32_t jx = e % (uint32_t)w;
        const uint32_t t = e / (uint32_t)w;
        const uint32_t jy = t % (uint32_t)h;
        const uint32_t p = t / (uint32_t)h;
        const uint32_t bs = (uint32_t)h * w;
        const uint32_t j = jy * w + jx;
        const float* yp = Y + p * 4 * bs + j;
        float t0 = yp[0];
        if (Zd) t0 += Zd[p * bs + j];
        const float t1 = yp[bs], t2 = yp[2 * bs], t3 = yp[3 * bs];
        const float a = t0 + t1, b = t0 - t1, c = t2 + t3, d = t2 - t3;
        const int X0 = 2 * (int)jx, Y0 = 2 * (int)jy;
        float* zp = Z + p * (uint32_t)(h_up * w_up) + (uint32_t)(Y0 * w_up + X0);
        const bool rx = X0 + 1 < w_up, ry = Y0 + 1 < h_up;
        zp[0] = 0.5f * (a + c);
        if (rx) zp[1] = 0.5f * (b + d);
        if (ry) {
            zp[w_up] = 0.5f * (a - c);
            if (rx) zp[w_up + 1] = 0.5f * (b - d);
        }
    }
}

// Weight-gradient correlation of channel ch = blockIdx.x over the batch slice
// of workgroup blockIdx.y (planes (b * nch + ch), b in the slice):
//   part[(blk * nch + ch) * (K*K + 1) + d] = sum_j A[j] X[j + d]   (X zero outside)
//   part[(blk * nch + ch) * (K*K + 1) + K*K] = sum_j A[j]
template <int K, typename TA, typename TX>
__global__ void __launch_bounds__(kThreads) k_tcorr(const TA* __restrict__ A, const TX* __restrict__ X, int nb,
                                                    int nch, Tile t, int nblk, float* __restrict__ part) {
    extern __shared__ float lds[];
    constexpr int R = K / 2, KK = K * K, NR = 4 + 2 * R, NW = kThreads / 64;
    __shared__ float red[NW][KK + 1];
    const int ch = blockIdx.x, blk = blockIdx.y;
    const int b0 = (int)((long)nb * blk / nblk), b1 = (int)((long)nb * (blk + 1) / nblk);
    const int ARH = 4 * t.NRG, SW = t.TW + 2 * R, RH = 4 * t.NRG + 2 * R;
    float* as = lds;                            // [NPB][4 NRG][TW]
    float* xs = lds + t.NPB * ARH * t.TW;       // [NPB][4 NRG + 2R][TW + 2R]
    float acc[KK + 1];
#pragma unroll
    for (int d = 0; d <= KK; ++d) acc[d] = 0.f;
    const int total = t.NPB * t.NRG * t.TW;
    for (int bg = b0; bg < b1; bg += t.NPB) {
        const int npv = min(t.NPB, b1 - bg);
        for (int tile = 0; tile < t.ntx * t.nty; ++tile) {
            const int ty0 = (tile / t.ntx) * t.TH, tx0 = (tile % t.ntx) * t.TW;
            __syncthreads();   // the previous tile's reads are done
            stage(as, A, bg * nch + ch, nch, npv, t, ty0, tx0, 0);
            stage(xs, X, bg * nch + ch, nch, npv, t, ty0, tx0, R);
            __syncthreads();
            Walk3 it(threadIdx.x, kThreads, t.TW, t.NRG);
            for (int f = threadIdx.x; f < total; f += kThreads, it.next()) {
                const int j = it.i2, rg = it.i1, c = it.i0;
                if (j >= npv) continue;
                const float* ab = as + (j * ARH + rg * 4) * t.TW + c;
                const float* xb = xs + (j * RH + rg * 4) * SW + c;
                float av[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) av[q] = ab[q * t.TW];   // zero outside the plane and tile rows
                acc[KK] += (av[0] + av[1]) + (av[2] + av[3]);
#pragma unroll
                for (int xr = 0; xr < NR; ++xr) {
                    float xv[K];
#pragma unroll
                    for (int kx = 0; kx < K; ++kx) xv[kx] = xb[xr * SW + kx];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int ky = xr - q;
                        if (ky < 0 || ky >= K) continue;
#pragma unroll
                        for (int kx = 0; kx < K; ++kx) acc[ky * K + kx] = fmaf(av[q], xv[kx], acc[ky * K + kx]);
                    }
                }
            }
        }
    }
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
    for (int d = 0; d <= KK; ++d) {
        float v = acc[d];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
        if (lane == 0) red[wv][d] = v;
    }
    __syncthreads();
    for (int d = threadIdx.x; d <= KK; d += kThreads) {
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < NW; ++q) s += red[q][d];
        part[((uint32_t)blk * nch + ch) * (KK + 1) + d] = s;
    }
}

// Runtime kernel size (odd k beyond the unrolled instances, k <= kMaxKAny):
// the same tiles and contract as k_tconv, the taps looped at run time.
template <bool ROT, typename TI, typename TO>
__global__ void __launch_bounds__(kThreads) k_tconv_rk(const TI* __restrict__ in, int P, int nch, Tile t, int k,
                                                       const float* __restrict__ wt, const float* __restrict__ scale,
                                                       const float* __restrict__ bias, const float* __restrict__ Z,
                                                       TO* __restrict__ out) {
    extern __shared__ float lds[];
    const int R = k / 2, KK = k * k;
    const int ntile = t.ntx * t.nty;
    const int g = blockIdx.x / ntile, tile = blockIdx.x - g * ntile;
    const int ty0 = (tile / t.ntx) * t.TH, tx0 = (tile % t.ntx) * t.TW;
    const int p0 = g * t.NPB;
    const int npv = min(t.NPB, P - p0);
    float* wl = lds;                        // [NPB][KK + 2]: weights, scale, bias
    float* xs = lds + t.NPB * (KK + 2);     // [NPB][4 NRG + 2R][TW + 2R]
    for (int f = threadIdx.x; f < npv * (KK + 2); f += kThreads) {
        const int j = f / (KK + 2), d = f - j * (KK + 2);
        const int ch = (p0 + j) % nch;
        float v;
        if (d < KK) v = wt[ch * KK + (ROT ? KK - 1 - d : d)];
        else if (d == KK) v = scale[ch];
        else v = bias ? bias[ch] : 0.f;
        wl[f] = v;
    }
    stage(xs, in, p0, 1, npv, t, ty0, tx0, R);
    __syncthreads();
    const int SW = t.TW + 2 * R, RH = 4 * t.NRG + 2 * R;
    const int total = t.NPB * t.NRG * t.TW;
    const uint32_t hw = (uint32_t)t.h * t.w;
    Walk3 it(threadIdx.x, kThreads, t.TW, t.NRG);
    for (int f = threadIdx.x; f < total; f += kThreads, it.next()) {
        const int j = it.i2, rg = it.i1, c = it.i0;
        if (j >= npv) continue;
        const float* wp = wl + j * (KK + 2);
        const float* xb = xs + (j * RH + rg * 4) * SW + c;
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int ky = 0; ky < k; ++ky)
            for (int kx = 0; kx < k; ++kx) {
                const float wv = wp[ky * k + kx];
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[q] = fmaf(wv, xb[(q + ky) * SW + kx], acc[q]);
            }
        const float sc = wp[KK], bi = wp[KK + 1];
        const uint32_t pbase = (uint32_t)(p0 + j) * hw;
        const int x = tx0 + c;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = rg * 4 + q, y = ty0 + r;
            if (r < t.TH && y < t.h && x < t.w) {
                const uint32_t o = pbase + (uint32_t)(y * t.w + x);
                float v = fmaf(sc, acc[q], bi);
                if (Z) v += Z[o];
                stv(out, o, v);
            }
        }
    }
}

// Runtime kernel size, weight-gradient correlation: the same contract and
// tiles as k_tcorr, output-stationary (thread d owns taps d, d + kThreads, ...
// and the sum slot KK), so no per-thread array of k^2 accumulators.
template <typename TA, typename TX>
__global__ void __launch_bounds__(kThreads) k_tcorr_rk(const TA* __restrict__ A, const TX* __restrict__ X, int nb,
                                                       int nch, Tile t, int k, int nblk, float* __restrict__ part) {
    extern __shared__ float lds[];
    const int R = k / 2, KK = k * k;
    const int ch = blockIdx.x, blk = blockIdx.y;
    const int b0 = (int)((long)nb * blk / nblk), b1 = (int)((long)nb * (blk + 1) / nblk);
    const int ARH = 4 * t.NRG, SW = t.TW + 2 * R, RH = 4 * t.NRG + 2 * R;
    float* as = lds;                            // [NPB][4 NRG][TW]
    float* xs = lds + t.NPB * ARH * t.TW;       // [NPB][4 NRG + 2R][TW + 2R]
    constexpr int kMaxPer = (kMaxKAny * kMaxKAny + 1 + kThreads - 1) / kThreads;
    float acc[kMaxPer];
#pragma unroll
    for (int q = 0; q < kMaxPer; ++q) acc[q] = 0.f;
    for (int bg = b0; bg < b1; bg += t.NPB) {
        const int npv = min(t.NPB, b1 - bg);
        for (int tile = 0; tile < t.ntx * t.nty; ++tile) {
            const int ty0 = (tile / t.ntx) * t.TH, tx0 = (tile % t.ntx) * t.TW;
            __syncthreads();   // the previous tile's reads are done
            stage(as, A, bg * nch + ch, nch, npv, t, ty0, tx0, 0);
            stage(xs, X, bg * nch + ch, nch, npv, t, ty0, tx0, R);
            __syncthreads();
#pragma unroll
            for (int q = 0; q < kMaxPer; ++q) {
                const int d = threadIdx.x + q * kThreads;
                if (d > KK) continue;
                const int ky = d < KK ? d / k : 0, kx = d < KK ? d - ky * k : 0;
                float s = 0.f;
                for (int j = 0; j < npv; ++j)
                    for (int r = 0; r < ARH; ++r) {
                        const float* ar = as + (j * ARH + r) * t.TW;
                        const float* xr = xs + (j * RH + r + ky) * SW + kx;
                        if (d == KK)
                            for (int c = 0; c < t.TW; ++c) s += ar[c];
                        else
                            for (int c = 0; c < t.TW; ++c) s = fmaf(ar[c], xr[c], s);
                    }
                acc[q] += s;
            }
        }
    }
#pragma unroll
    for (int q = 0; q < kMaxPer; ++q) {
        const int d = threadIdx.x + q * kThreads;
        if (d <= KK) part[((uint32_t)blk * nch + ch) * (KK + 1) + d] = acc[q];
    }
}

// ---------------------------------------------------------------------------
// Large planes (both sides >= kBigSide): 64 x 64 tiles, each thread a 4 x 4
// block with a register-blocked window (two window rows live, read as 16-byte
// LDS rows), so a window row of X serves 4 x K multiply-adds per value.
// ---------------------------------------------------------------------------
constexpr int kBigTile = kUnfusedBigTile;

__host__ __device__ constexpr int big_xs_stride(int R) { return (kBigTile + 2 * R + 3) & ~3; }

bool big_planes(int h, int w) { return unfused_big_planes(h, w); }

// Stage rows [y0, y0 + rows) x columns [x0, x0 + cols) of plane `src` (h x w,
// zero outside) into lds[r * stride + c]; cols <= 64 + 2 * kMaxK.  Wave v takes
// rows v, v + 4, ...; lane l column l (and l + 64 where cols > 64).  All loads
// of a thread are issued before its LDS writes.
template <int ROWS, int COLS, typename T>
__device__ __forceinline__ void stage_rows(float* lds, int stride, const T* __restrict__ src, int h, int w, int y0,
                                           int x0) {
    constexpr int NW = kThreads / 64, RPW = (ROWS + NW - 1) / NW, CPL = (COLS + 63) / 64;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    float v[RPW][CPL];
#pragma unroll
    for (int k = 0; k < RPW; ++k)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            const int r = wave + k * NW, c = lane + cc * 64;
            const int y = y0 + r, x = x0 + c;
            v[k][cc] = (r < ROWS && c < COLS && y >= 0 && y < h && x >= 0 && x < w) ? ldv(src, (uint32_t)(y * w + x)) : 0.f;
        }
#pragma unroll
    for (int k = 0; k < RPW; ++k)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            const int r = wave + k * NW, c = lane + cc * 64;
            if (r < ROWS && c < COLS) lds[r * stride + c] = v[k][cc];
        }
}

// Read WW consecutive floats of a 16-byte aligned LDS row.
template <int WW>
__device__ __forceinline__ void lds_row4(const float* p, float (&row)[WW]) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    typedef float f2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int q = 0; q + 4 <= WW; q += 4) {
        const f4 v = *reinterpret_cast<const f4*>(p + q);
        row[q] = v.x; row[q + 1] = v.y; row[q + 2] = v.z; row[q + 3] = v.w;
    }
    constexpr int done = (WW / 4) * 4;
    if constexpr (WW - done >= 2) {
        const f2 v = *reinterpret_cast<const f2*>(p + done);
        row[done] = v.x; row[done + 1] = v.y;
    }
    if constexpr ((WW - done) % 2 == 1) row[WW - 1] = p[WW - 1];
}

// Same contract as k_tcorr, for large planes: the units of channel ch are
// (batch entry, 64 x 64 tile) pairs, nb * ntile of them, split evenly over the
// nblk workgroups of the channel (grid nch x nblk).
template <int K, typename TA, typename TX>
__global__ void __launch_bounds__(kThreads) k_tcorr_big(const TA* __restrict__ A, const TX* __restrict__ X, int nb,
                                                        int nch, int h, int w, int ntx, int nty, int nblk,
                                                        float* __restrict__ part) {
    constexpr int R = K / 2, KK = K * K, WW = 4 + 2 * R, NW = kThreads / 64;
    constexpr int SA = kBigTile + 4, SX = big_xs_stride(R);
    __shared__ __align__(16) float as[kBigTile * SA];
    __shared__ __align__(16) float xs[(kBigTile + 2 * R) * SX];
    __shared__ float red[NW][KK + 1];
    const int ch = blockIdx.x, blk = blockIdx.y;
    const int ntile = ntx * nty, units = nb * ntile;
    const int u0 = (int)((long)units * blk / nblk), u1 = (int)((long)units * (blk + 1) / nblk);
    const uint32_t hw = (uint32_t)h * w;
    const int qy = threadIdx.x >> 4, qx = threadIdx.x & 15;
    float acc[KK + 1];
#pragma unroll
    for (int d = 0; d <= KK; ++d) acc[d] = 0.f;
    for (int u = u0; u < u1; ++u) {
        const int b = u / ntile, tile = u - b * ntile;
        const int ty0 = (tile / ntx) * kBigTile, tx0 = (tile % ntx) * kBigTile;
        const uint32_t pbase = (uint32_t)(b * nch + ch) * hw;
        __syncthreads();   // the previous unit's reads are done
        stage_rows<kBigTile, kBigTile>(as, SA, A + pbase, h, w, ty0, tx0);
        stage_rows<kBigTile + 2 * R, kBigTile + 2 * R>(xs, SX, X + pbase, h, w, ty0 - R, tx0 - R);
        __syncthreads();
        float a[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) lds_row4<4>(as + (4 * qy + i) * SA + 4 * qx, a[i]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[KK] += (a[i][0] + a[i][1]) + (a[i][2] + a[i][3]);
        const float* xb = xs + (4 * qy) * SX + 4 * qx;
        float rows[2][WW];
        lds_row4<WW>(xb, rows[0]);
#pragma unroll
        for (int wy = 0; wy < 4 + 2 * R; ++wy) {
            float (&row)[WW] = rows[wy & 1];
            if (wy + 1 < 4 + 2 * R) lds_row4<WW>(xb + (wy + 1) * SX, rows[(wy + 1) & 1]);
#pragma unroll
            for (int oy = 0; oy < 4; ++oy) {
                const int ky = wy - oy;
                if (ky < 0 || ky >= K) continue;
#pragma unroll
                for (int kx = 0; kx < K; ++kx)
#pragma unroll
                    for (int ox = 0; ox < 4; ++ox) acc[ky * K + kx] = fmaf(a[oy][ox], row[ox + kx], acc[ky * K + kx]);
            }
        }
    }
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
    for (int d = 0; d <= KK; ++d) {
        float v = acc[d];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
        if (lane == 0) red[wv][d] = v;
    }
    __syncthreads();
    for (int d = threadIdx.x; d <= KK; d += kThreads) {
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < NW; ++q) s += red[q][d];
        part[((uint32_t)blk * nch + ch) * (KK + 1) + d] = s;
    }
}

// Same contract as k_tconv, for large planes: one workgroup per (plane,
// 64 x 64 tile), grid P * ntile.
template <int K, bool ROT, typename TI, typename TO>
__global__ void __launch_bounds__(kThreads) k_tconv_big(const TI* __restrict__ in, int nch, int h, int w, int ntx,
                                                        int nty, const float* __restrict__ wt,
                                                        const float* __restrict__ scale,
                                                        const float* __restrict__ bias, const float* __restrict__ Z,
                                                        TO* __restrict__ out) {
    constexpr int R = K / 2, KK = K * K, WW = 4 + 2 * R, SX = big_xs_stride(R);
    __shared__ __align__(16) float xs[(kBigTile + 2 * R) * SX];
    const int ntile = ntx * nty;
    const int p = blockIdx.x / ntile, tile = blockIdx.x - p * ntile;
    const int ty0 = (tile / ntx) * kBigTile, tx0 = (tile % ntx) * kBigTile;
    const int ch = p % nch;
    const uint32_t hw = (uint32_t)h * w, pbase = (uint32_t)p * hw;
    stage_rows<kBigTile + 2 * R, kBigTile + 2 * R>(xs, SX, in + pbase, h, w, ty0 - R, tx0 - R);
    float wk[KK];
#pragma unroll
    for (int q = 0; q < KK; ++q) wk[q] = wt[ch * KK + (ROT ? KK - 1 - q : q)];
    const float sc = scale[ch], bi = bias ? bias[ch] : 0.f;
    __syncthreads();
    const int qy = threadIdx.x >> 4, qx = threadIdx.x & 15;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
    const float* xb = xs + (4 * qy) * SX + 4 * qx;
    float rows[2][WW];
    lds_row4<WW>(xb, rows[0]);
#pragma unroll
    for (int wy = 0; wy < 4 + 2 * R; ++wy) {
        float (&row)[WW] = rows[wy & 1];
        if (wy + 1 < 4 + 2 * R) lds_row4<WW>(xb + (wy + 1) * SX, rows[(wy + 1) & 1]);
#pragma unroll
        for (int oy = 0; oy < 4; ++oy) {
            const int ky = wy - oy;
            if (ky < 0 || ky >= K) continue;
#pragma unroll
            for (int kx = 0; kx < K; ++kx)
#pragma unroll
                for (int ox = 0; ox < 4; ++ox) acc[oy][ox] = fmaf(wk[ky * K + kx], row[ox + kx], acc[oy][ox]);
        }
    }
    const int x0 = tx0 + 4 * qx;
    // whole 4-pixel rows as one 16-byte (8-byte for bf16) access where aligned
    const bool vec = (w & 3) == 0 && x0 + 4 <= w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int y = ty0 + 4 * qy + i;
        if (y >= h) continue;
        const uint32_t o = pbase + (uint32_t)(y * w + x0);
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = fmaf(sc, acc[i][j], bi);
        if (vec) {
            if (Z) {
                const float4 z = *reinterpret_cast<const float4*>(Z + o);
                v[0] += z.x; v[1] += z.y; v[2] += z.z; v[3] += z.w;
            }
            st4(out, o, v);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (x0 + j >= w) continue;
                float u = v[j];
                if (Z) u += Z[o + j];
                stv(out, o + j, u);
            }
        }
    }
}

// dW = s * C, ds = sum_d W * C, and (base level) db = sum g, from the partials.
// One workgroup of 64 lanes per channel; lane l sums slots l, l + 64, ... over
// the partial blocks in a fixed order.
__global__ void __launch_bounds__(64) k_corr_finalize(const float* __restrict__ part, int nch, int nblk, int k,
                                                      const float* __restrict__ wt, const float* __restrict__ scale,
                                                      float* __restrict__ dw, float* __restrict__ ds,
                                                      float* __restrict__ db) {
    const int ch = blockIdx.x;
    const int kk = k * k;
    const size_t stride = (size_t)nch * (kk + 1);
    float wv = 0.f;
    for (int d = threadIdx.x; d <= kk; d += 64) {
        const float* pp = part + (size_t)ch * (kk + 1) + d;
        float cv = 0.f;
#pragma unroll 8
        for (int b = 0; b < nblk; ++b) cv += pp[b * stride];
        if (d < kk) {
            dw[(size_t)ch * kk + d] = scale[ch] * cv;
            wv = fmaf(wt[(size_t)ch * kk + d], cv, wv);
        } else if (db) {
            db[ch] = cv;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) wv += __shfl_xor(wv, o, 64);
    if (threadIdx.x == 0) ds[ch] = wv;
}

template <typename T>
void launch_analysis(const T* in, uint32_t in_ps, int P, int h_in, int w_in, float* out, int h_o, int w_o,
                     hipStream_t st) {
    const uint32_t n = (uint32_t)P * h_o * w_o;
    hipLaunchKernelGGL(k_analysis<T>, dim3(blocks_for(n)), dim3(kThreads), 0, st, in, in_ps, n, h_in, w_in, out,
                       h_o, w_o);
}

void launch_synthesis(const float* Y, const float* Zd, int P, int h, int w, float* Z, int h_up, int w_up,
                      hipStream_t st) {
    const uint32_t n = (uint32_t)P * h * w;
    hipLaunchKernelGGL(k_synthesis, dim3(blocks_for(n)), dim3(kThreads), 0, st, Y, Zd, n, h, w, Z, h_up, w_up);
}

// out = scale * conv(in) + bias + Z over P planes of h x w, channel p % nch
template <int K, typename TI, typename TO>
void launch_conv(bool rot, const TI* in, int P, int nch, int h, int w, const float* wt, const float* scale,
                 const float* bias, const float* Z, TO* out, hipStream_t st, int k_rt = K) {
    if constexpr (K == 0) {
        // runtime kernel size: the small-tile kernel with the taps looped
        const Tile t = make_tile(h, w, k_rt, false);
        const uint32_t grid = (uint32_t)((P + t.NPB - 1) / t.NPB) * (uint32_t)(t.ntx * t.nty);
        const size_t lds = tile_lds_floats(t, k_rt, false) * sizeof(float);
        if (rot)
            hipLaunchKernelGGL((k_tconv_rk<true, TI, TO>), dim3(grid), dim3(kThreads), lds, st, in, P, nch, t, k_rt,
                               wt, scale, bias, Z, out);
        else
            hipLaunchKernelGGL((k_tconv_rk<false, TI, TO>), dim3(grid), dim3(kThreads), lds, st, in, P, nch, t, k_rt,
                               wt, scale, bias, Z, out);
    } else {
    if (big_planes(h, w)) {
        const int ntx = (w + kBigTile - 1) / kBigTile, nty = (h + kBigTile - 1) / kBigTile;
        const uint32_t grid = (uint32_t)P * ntx * nty;
        if (rot)
            hipLaunchKernelGGL((k_tconv_big<K, true, TI, TO>), dim3(grid), dim3(kThreads), 0, st, in, nch, h, w, ntx,
                               nty, wt, scale, bias, Z, out);
        else
            hipLaunchKernelGGL((k_tconv_big<K, false, TI, TO>), dim3(grid), dim3(kThreads), 0, st, in, nch, h, w, ntx,
                               nty, wt, scale, bias, Z, out);
        return;
    }
    const Tile t = make_tile(h, w, K, false);
    const uint32_t grid = (uint32_t)((P + t.NPB - 1) / t.NPB) * (uint32_t)(t.ntx * t.nty);
    const size_t lds = tile_lds_floats(t, K, false) * sizeof(float);
    if (rot)
        hipLaunchKernelGGL((k_tconv<K, true, TI, TO>), dim3(grid), dim3(kThreads), lds, st, in, P, nch, t, wt, scale,
                           bias, Z, out);
    else
        hipLaunchKernelGGL((k_tconv<K, false, TI, TO>), dim3(grid), dim3(kThreads), lds, st, in, P, nch, t, wt,
                           scale, bias, Z, out);
    }
}

}  // namespace

int launch_corr_finalize(const float* part, int nch, int nblk, int k, const float* wt, const float* scale, float* dw,
                         float* ds, float* db, void* stream) {
    hipLaunchKernelGGL(k_corr_finalize, dim3(nch), dim3(64), 0, reinterpret_cast<hipStream_t>(stream), part, nch,
                       nblk, k, wt, scale, dw, ds, db);
    return hipGetLastError() == hipSuccess ? WTC_OK : WTC_EHIP;
}


namespace {

// correlation partials of one level (nch channels, nb planes per channel):
// part[blk][ch][K*K + 1]; returns the number of blocks
template <int K, typename TA, typename TX>
int launch_corr_parts(const TA* A, const TX* X, int nb, int nch, int h, int w, float* part, hipStream_t st,
                      int k_rt = K) {
    const int nblk = unfused_corr_blocks(nb, nch, h, w);
    if constexpr (K == 0) {
        // runtime kernel size: small tiles for every plane size (blocks beyond
        // the batch, where the split counts tiles, add zero partials)
        const Tile t = make_tile(h, w, k_rt, true);
        const size_t lds = tile_lds_floats(t, k_rt, true) * sizeof(float);
        hipLaunchKernelGGL((k_tcorr_rk<TA, TX>), dim3(nch, nblk), dim3(kThreads), lds, st, A, X, nb, nch, t, k_rt,
                           nblk, part);
    } else if (big_planes(h, w)) {
        const int ntx = (w + kBigTile - 1) / kBigTile, nty = (h + kBigTile - 1) / kBigTile;
        hipLaunchKernelGGL((k_tcorr_big<K, TA, TX>), dim3(nch, nblk), dim3(kThreads), 0, st, A, X, nb, nch, h, w,
                           ntx, nty, nblk, part);
    } else {
        const Tile t = make_tile(h, w, K, true);
        const size_t lds = tile_lds_floats(t, K, true) * sizeof(float);
        hipLaunchKernelGGL((k_tcorr<K, TA, TX>), dim3(nch, nblk), dim3(kThreads), lds, st, A, X, nb, nch, t, nblk,
                           part);
    }
    return nblk;
}

// correlation + finalize of one level (nch channels, nb planes per channel)
template <int K, typename TA, typename TX>
void launch_corr(const TA* A, const TX* X, int nb, int nch, int h, int w, const float* wt, const float* scale,
                 float* dw, float* ds, float* db, float* part, hipStream_t st, int k_rt = K) {
    const int nblk = launch_corr_parts<K, TA, TX>(A, X, nb, nch, h, w, part, st, k_rt);
    hipLaunchKernelGGL(k_corr_finalize, dim3(nch), dim3(64), 0, st, part, nch, nblk, k_rt, wt, scale, dw, ds, db);
}

template <int K, typename T>
int fwd_t(const wtc_desc* d, const UnfusedPlan& p, const T* x, const float* w0, const float* s0,
          const float* b0, const float* wl, const float* sl, T* out, char* ws, hipStream_t st, int stage,
          const float* zext) {
    const int B = d->B, C = d->C, L = d->L;
    const int P = B * C;
    const size_t KK = (size_t)d->k * d->k;
    auto F = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
    for (int i = 1; i <= L && stage != 2; ++i) {
        if (i == 1)
            launch_analysis<T>(x, (uint32_t)(p.h[0] * p.w[0]), P, p.h[0], p.w[0], F(p.s_off[1]), p.h[1], p.w[1], st);
        else
            launch_analysis<float>(F(p.s_off[i - 1]), (uint32_t)(4 * p.h[i - 1] * p.w[i - 1]), P, p.h[i - 1],
                                   p.w[i - 1], F(p.s_off[i]), p.h[i], p.w[i], st);
    }
    if (stage == 1) return hipGetLastError() == hipSuccess ? WTC_OK : WTC_EHIP;
    for (int i = 1; i <= L; ++i)
        launch_conv<K, float, float>(false, F(p.s_off[i]), 4 * P, 4 * C, p.h[i], p.w[i],
                                     wl + (size_t)(i - 1) * 4 * C * KK, sl + (size_t)(i - 1) * 4 * C, nullptr,
                                     nullptr, F(p.y_off[i]), st, d->k);
    for (int i = L; i >= 1; --i)
        launch_synthesis(F(p.y_off[i]), i < L ? F(p.z_off[i + 1]) : zext, P, p.h[i], p.w[i], F(p.z_off[i]),
                         p.h[i - 1], p.w[i - 1], st);
    launch_conv<K, T, T>(false, x, P, C, d->H, d->W, w0, s0, b0, L > 0 ? F(p.z_off[1]) : nullptr, out, st, d->k);
    return hipGetLastError() == hipSuccess ? WTC_OK : WTC_EHIP;
}

template <int K, typename T>
int bwd_t(const wtc_desc* d, const UnfusedPlan& p, const T* x, const T* g, const float* w0, const float* s0,
          const float* wl, const float* sl, T* dx, float* dw0, float* ds0, float* db0, float* dwl, float* dsl,
          char* ws, hipStream_t st, int stage, const float* zext) {
    const int B = d->B, C = d->C, L = d->L;
    const int P = B * C;
    const size_t KK = (size_t)d->k * d->k;
    auto F = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
    float* part = F(p.part_off);
    // analysis cascades of g (the adjoint of the synthesis) and of x
    for (int i = 1; i <= L && stage != 2; ++i) {
        if (i == 1) {
            const uint32_t ps = (uint32_t)(p.h[0] * p.w[0]);
            launch_analysis<T>(g, ps, P, p.h[0], p.w[0], F(p.dt_off[1]), p.h[1], p.w[1], st);
            launch_analysis<T>(x, ps, P, p.h[0], p.w[0], F(p.s_off[1]), p.h[1], p.w[1], st);
        } else {
            const uint32_t ps = (uint32_t)(4 * p.h[i - 1] * p.w[i - 1]);
            launch_analysis<float>(F(p.dt_off[i - 1]), ps, P, p.h[i - 1], p.w[i - 1], F(p.dt_off[i]), p.h[i],
                                   p.w[i], st);
            launch_analysis<float>(F(p.s_off[i - 1]), ps, P, p.h[i - 1], p.w[i - 1], F(p.s_off[i]), p.h[i], p.w[i],
                                   st);
        }
    }
    if (stage == 1) return hipGetLastError() == hipSuccess ? WTC_OK : WTC_EHIP;
    // per level: dS = s * (rot W * dY);  dW, ds from corr(dY, S)
    for (int i = 1; i <= L; ++i) {
        const float* wli = wl + (size_t)(i - 1) * 4 * C * KK;
        const float* sli = sl + (size_t)(i - 1) * 4 * C;
        launch_conv<K, float, float>(true, F(p.dt_off[i]), 4 * P, 4 * C, p.h[i], p.w[i], wli, sli, nullptr, nullptr,
                                     F(p.y_off[i]), st, d->k);
        launch_corr<K, float, float>(F(p.dt_off[i]), F(p.s_off[i]), B, 4 * C, p.h[i], p.w[i], wli, sli,
                                     dwl + (size_t)(i - 1) * 4 * C * KK, dsl + (size_t)(i - 1) * 4 * C, nullptr,
                                     part, st, d->k);
    }
    // adjoint of the analysis: synthesis of dS, deepest first
    for (int i = L; i >= 1; --i)
        launch_synthesis(F(p.y_off[i]), i < L ? F(p.z_off[i + 1]) : zext, P, p.h[i], p.w[i], F(p.z_off[i]),
                         p.h[i - 1], p.w[i - 1], st);
    // base: dx = s0 * (rot W0 * g) + dLL_0;  dW0, ds0, db0 from corr(g, x)
    launch_conv<K, T, T>(true, g, P, C, d->H, d->W, w0, s0, nullptr, L > 0 ? F(p.z_off[1]) : nullptr, dx, st, d->k);
    launch_corr<K, T, T>(g, x, B, C, d->H, d->W, w0, s0, dw0, ds0, db0, part, st, d->k);
    return hipGetLastError() == hipSuccess ? WTC_OK : WTC_EHIP;
}


}  // namespace

namespace {

template <int K>
int fwd_k(const wtc_desc* d, const UnfusedPlan& p, const void* x, const float* w0, const float* s0,
          const float* b0, const float* wl, const float* sl, void* out, char* ws, hipStream_t st, int stage,
          const float* zext) {
    if (d->dtype == WTC_BF16)
        return fwd_t<K, uint16_t>(d, p, static_cast<const uint16_t*>(x), w0, s0, b0, wl, sl,
                                  static_cast<uint16_t*>(out), ws, st, stage, zext);
    return fwd_t<K, float>(d, p, static_cast<const float*>(x), w0, s0, b0, wl, sl, static_cast<float*>(out), ws, st,
                           stage, zext);
}

template <int K>
int bwd_k(const wtc_desc* d, const UnfusedPlan& p, const void* x, const void* g, const float* w0,
          const float* s0, const float* wl, const float* sl, void* dx, float* dw0, float* ds0, float* db0,
          float* dwl, float* dsl, char* ws, hipStream_t st, int stage, const float* zext) {
    if (d->dtype == WTC_BF16)
        return bwd_t<K, uint16_t>(d, p, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(g), w0, s0, wl,
                                  sl, static_cast<uint16_t*>(dx), dw0, ds0, db0, dwl, dsl, ws, st, stage, zext);
    return bwd_t<K, float>(d, p, static_cast<const float*>(x), static_cast<const float*>(g), w0, s0, wl, sl,
                           static_cast<float*>(dx), dw0, ds0, db0, dwl, dsl, ws, st, stage, zext);
}

__global__ void __launch_bounds__(256) k_fill_zero(float* p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

}  // namespace

int unfused_forward(const wtc_desc* d, const UnfusedPlan& p, const void* x, const float* w0, const float* s0,
                    const float* b0, const float* wl, const float* sl, void* out, char* ws, void* stream,
                    int stage, const float* zext) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    switch (d->k) {
        case 1: return fwd_k<1>(d, p, x, w0, s0, b0, wl, sl, out, ws, st, stage, zext);
        case 3: return fwd_k<3>(d, p, x, w0, s0, b0, wl, sl, out, ws, st, stage, zext);
        case 5: return fwd_k<5>(d, p, x, w0, s0, b0, wl, sl, out, ws, st, stage, zext);
        case 7: return fwd_k<7>(d, p, x, w0, s0, b0, wl, sl, out, ws, st, stage, zext);
        default: return fwd_k<0>(d, p, x, w0, s0, b0, wl, sl, out, ws, st, stage, zext);
    }
}

int unfused_backward(const wtc_desc* d, const UnfusedPlan& p, const void* x, const void* g, const float* w0,
                     const float* s0, const float* wl, const float* sl, void* dx, float* dw0, float* ds0,
                     float* db0, float* dwl, float* dsl, char* ws, void* stream, int stage, const float* zext) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    switch (d->k) {
        case 1: return bwd_k<1>(d, p, x, g, w0, s0, wl, sl, dx, dw0, ds0, db0, dwl, dsl, ws, st, stage, zext);
        case 3: return bwd_k<3>(d, p, x, g, w0, s0, wl, sl, dx, dw0, ds0, db0, dwl, dsl, ws, st, stage, zext);
        case 5: return bwd_k<5>(d, p, x, g, w0, s0, wl, sl, dx, dw0, ds0, db0, dwl, dsl, ws, st, stage, zext);
        case 7: return bwd_k<7>(d, p, x, g, w0, s0, wl, sl, dx, dw0, ds0, db0, dwl, dsl, ws, st, stage, zext);
        default: return bwd_k<0>(d, p, x, g, w0, s0, wl, sl, dx, dw0, ds0, db0, dwl, dsl, ws, st, stage, zext);
    }
}

int base_corr_partials(const wtc_desc* d, const void* x, const void* g, float* part, int* nblk, void* stream) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    auto go = [&](auto kc, auto tag) {
        using T = decltype(tag);
        constexpr int K = decltype(kc)::value;
        *nblk = launch_corr_parts<K, T, T>(static_cast<const T*>(g), static_cast<const T*>(x), d->B, d->C, d->H,
                                           d->W, part, st, d->k);
    };
    const bool bf = d->dtype == WTC_BF16;
    switch (d->k) {
        case 1: bf ? go(std::integral_constant<int, 1>{}, uint16_t{}) : go(std::integral_constant<int, 1>{}, float{}); break;
        case 3: bf ? go(std::integral_constant<int, 3>{}, uint16_t{}) : go(std::integral_constant<int, 3>{}, float{}); break;
        case 5: bf ? go(std::integral_constant<int, 5>{}, uint16_t{}) : go(std::integral_constant<int, 5>{}, float{}); break;
        case 7: bf ? go(std::integral_constant<int, 7>{}, uint16_t{}) : go(std::integral_constant<int, 7>{}, float{}); break;
        default: bf ? go(std::integral_constant<int, 0>{}, uint16_t{}) : go(std::integral_constant<int, 0>{}, float{}); break;
    }
    return hipGetLastError() == hipSuccess ? WTC_OK : WTC_EHIP;
}

int launch_fill_zero(float* p, int n, void* stream) {
    if (n <= 0) return 0;
    hipLaunchKernelGGL(k_fill_zero, dim3((n + 255) / 256), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), p, n);
    return (int)hipGetLastError();
}

}  // namespace wtc
