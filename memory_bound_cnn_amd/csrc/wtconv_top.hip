// Top level of a peeled plane (planes beyond the on-chip pipeline).
//
// The levels >= 2 of WTConv are WTConv itself applied to the level-1 LL band,
// so a large plane runs its deeper levels as a sub-problem on that band and
// only level 1 and the base conv at full resolution.  Those two are fused
// here over 64 x 64 output tiles: each workgroup stages its x tile with the
// halo both convolutions need (k/2 at level 0, k/2 level-1 positions = 2 (k/2)
// pixels for the level-1 conv), recomputes the four level-1 subbands of the
// tile on chip, convolves them (one subband per wave), synthesizes level 1
// (adding the sub-problem's result to the LL band) and writes
//   out = s0 (W0 * x) + b0 + synthesis(Y1)
// with one HBM read of x and one write of out.  Orthonormal Haar factors as
// in the level-by-level kernels (0.5 per 2x2 butterfly), so the LL band and
// the sub-problem's input and output are the same tensors.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "wtc_internal.h"
#include "wtc_numeric.h"

namespace wtc {
namespace {

constexpr int kTop = kTopTile;  // output tile side
constexpr int kTopThreads = 256;

__device__ __forceinline__ float tld(const float* p, uint32_t i) { return p[i]; }
__device__ __forceinline__ float tld(const uint16_t* p, uint32_t i) { return __uint_as_float(((uint32_t)p[i]) << 16); }
// four consecutive values at a 4-element aligned index
__device__ __forceinline__ void tld4(const float* p, uint32_t i, float (&v)[4]) {
    const float4 q = *reinterpret_cast<const float4*>(p + i);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}
__device__ __forceinline__ void tld4(const uint16_t* p, uint32_t i, float (&v)[4]) {
    const uint2 q = *reinterpret_cast<const uint2*>(p + i);
    v[0] = __uint_as_float(q.x << 16); v[1] = __uint_as_float(q.x & 0xFFFF0000u);
    v[2] = __uint_as_float(q.y << 16); v[3] = __uint_as_float(q.y & 0xFFFF0000u);
}
__device__ __forceinline__ uint32_t tbf16(float v) { return bf16_rne(v); }
__device__ __forceinline__ void tst(float* p, uint32_t i, float v) { p[i] = v; }
__device__ __forceinline__ void tst(uint16_t* p, uint32_t i, float v) { p[i] = (uint16_t)tbf16(v); }
__device__ __forceinline__ void tst4(float* p, uint32_t i, const float (&v)[4]) {
    *reinterpret_cast<float4*>(p + i) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void tst4(uint16_t* p, uint32_t i, const float (&v)[4]) {
    *reinterpret_cast<uint2*>(p + i) = make_uint2(tbf16(v[0]) | (tbf16(v[1]) << 16), tbf16(v[2]) | (tbf16(v[3]) << 16));
}

typedef float tf4 __attribute__((ext_vector_type(4)));
typedef float tf2 __attribute__((ext_vector_type(2)));

// WW consecutive floats of a 16-byte aligned LDS row
template <int WW>
__device__ __forceinline__ void trow(const float* p, float (&row)[WW]) {
#pragma unroll
    for (int q = 0; q + 4 <= WW; q += 4) {
        const tf4 v = *reinterpret_cast<const tf4*>(p + q);
        row[q] = v.x; row[q + 1] = v.y; row[q + 2] = v.z; row[q + 3] = v.w;
    }
    constexpr int done = (WW / 4) * 4;
    if constexpr (WW - done >= 2) {
        const tf2 v = *reinterpret_cast<const tf2*>(p + done);
        row[done] = v.x; row[done + 1] = v.y;
    }
    if constexpr ((WW - done) % 2 == 1) row[WW - 1] = p[WW - 1];
}

// 4 x 4 outputs of a K x K cross-correlation from an LDS window whose row 0
// is output row -R (two window rows live).
template <int K>
__device__ __forceinline__ void tstencil(const float* win, int S, const float (&w)[K * K], float (&acc)[4][4]) {
    constexpr int R = K / 2, WW = 4 + 2 * R, WH = 4 + 2 * R;
    float rows[2][WW];
    trow<WW>(win, rows[0]);
#pragma unroll
    for (int wy = 0; wy < WH; ++wy) {
        float (&row)[WW] = rows[wy & 1];
        if (wy + 1 < WH) trow<WW>(win + (wy + 1) * S, rows[(wy + 1) & 1]);
#pragma unroll
        for (int oy = 0; oy < 4; ++oy) {
            const int ky = wy - oy;
            if (ky < 0 || ky >= K) continue;
#pragma unroll
            for (int kx = 0; kx < K; ++kx)
#pragma unroll
                for (int ox = 0; ox < 4; ++ox) acc[oy][ox] = fmaf(w[ky * K + kx], row[ox + kx], acc[oy][ox]);
        }
    }
}

// tstencil plus the correlation of the window with a 4 x 4 block xv:
//   corr[ky K + kx] += xv[oy][ox] win[oy + ky][ox + kx]
template <int K>
__device__ __forceinline__ void tstencil_corr(const float* win, int S, const float (&w)[K * K], float (&acc)[4][4],
                                              const float (&xv)[4][4], float (&corr)[K * K]) {
    constexpr int R = K / 2, WW = 4 + 2 * R, WH = 4 + 2 * R;
    float rows[2][WW];
    trow<WW>(win, rows[0]);
#pragma unroll
    for (int wy = 0; wy < WH; ++wy) {
        float (&row)[WW] = rows[wy & 1];
        if (wy + 1 < WH) trow<WW>(win + (wy + 1) * S, rows[(wy + 1) & 1]);
#pragma unroll
        for (int oy = 0; oy < 4; ++oy) {
            const int ky = wy - oy;
            if (ky < 0 || ky >= K) continue;
#pragma unroll
            for (int kx = 0; kx < K; ++kx)
#pragma unroll
                for (int ox = 0; ox < 4; ++ox) {
                    acc[oy][ox] = fmaf(w[ky * K + kx], row[ox + kx], acc[oy][ox]);
                    corr[ky * K + kx] = fmaf(xv[oy][ox], row[ox + kx], corr[ky * K + kx]);
                }
        }
    }
}

// Value of v in lane l - N of the same 16-lane row (0 for the row's first N
// lanes): DPP row shift.
template <int N>
__device__ __forceinline__ float trow_shr(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x110 | N, 0xF, 0xF, true));
}
// Lane 15 of every 16-lane row: the sum of v over the row.
__device__ __forceinline__ float trow_sum(float v) {
    v += trow_shr<1>(v);
    v += trow_shr<2>(v);
    v += trow_shr<4>(v);
    return v + trow_shr<8>(v);
}

// Geometry of the staged x tile and of the level-1 band tile (compile time).
template <int K>
struct TopGeom {
    static constexpr int R = K / 2;
    // x tile: global rows ty0 - 2R .., columns tx0 - CO ..; CO >= 2R with
    // CO = R (mod 4), so that a base-conv window starts on a 16-byte boundary
    static constexpr int CO = 2 * R + ((R - 2 * R) % 4 + 4) % 4;
    static constexpr int XR = kTop + 4 * R;
    static constexpr int XS = (CO + kTop + 2 * R + 3) & ~3;
    // band tile: level-1 positions -R .. 32 + R of the tile's 32 x 32
    static constexpr int BR = kTop / 2 + 2 * R;
    static constexpr int BS = (BR + 3) & ~3;
    static constexpr int BSZ = BR * BS;
    // level-1 results, 32 x 32 per band (stride 36: 16-byte rows)
    static constexpr int YS = kTop / 2 + 4;
    static constexpr int YSZ = (kTop / 2) * YS;
    // the level-1 results reuse the x tile's storage
    static constexpr int XN = XR * XS > 4 * YSZ ? XR * XS : 4 * YSZ;
};

// Tile units (plane-major, tiles in row order) dealt to the XCDs in
// contiguous ranges: workgroup i runs on XCD i % 8 (workgroups are dealt to
// the XCDs in turn) and takes unit (i % 8) ceil(n / 8) + i / 8, so the tiles
// of one plane -- whose halos share rows and cache lines -- pass through one
// L2 one after another.  The grid is 8 ceil(n / 8) workgroups.
__device__ __forceinline__ uint32_t top_unit(uint32_t n) {
    const uint32_t per = (n + 7) >> 3;
    return (blockIdx.x & 7) * per + (blockIdx.x >> 3);
}

template <int K, typename T>
__global__ void __launch_bounds__(kTopThreads) k_top_fwd(const T* __restrict__ x, int C, int H, int W, int ntx,
                                                         int nty, const float* __restrict__ w0,
                                                         const float* __restrict__ s0, const float* __restrict__ b0,
                                                         const float* __restrict__ wl, const float* __restrict__ sl,
                                                         const float* __restrict__ zext, T* __restrict__ out,
                                                         uint32_t nunit) {
    using G = TopGeom<K>;
    constexpr int R = G::R, KK = K * K;
    __shared__ __align__(16) float xs[G::XN];   // x tile; later the level-1 results
    __shared__ __align__(16) float bs[4 * G::BSZ];      // the four level-1 bands of the tile
    const int ntile = ntx * nty;
    const uint32_t unit = top_unit(nunit);
    if (unit >= nunit) return;   // whole workgroup, before any barrier
    const int p = (int)(unit / ntile), tile = (int)(unit - (uint32_t)p * ntile);
    const int ty0 = (tile / ntx) * kTop, tx0 = (tile % ntx) * kTop;
    const int c = p % C;
    const int h1 = (H + 1) >> 1, w1 = (W + 1) >> 1;
    const uint32_t hw = (uint32_t)H * W;
    const T* xp = x + (size_t)p * hw;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;

    // ---- stage the x tile (zero outside the plane): wave v takes rows v, v + 4, ...;
    // every load of a thread is issued before its LDS writes
    {
        constexpr int NW = kTopThreads / 64, RPW = (G::XR + NW - 1) / NW, CPL = (G::XS + 63) / 64;
        float v[RPW][CPL];
#pragma unroll
        for (int k = 0; k < RPW; ++k)
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                const int r = wave + k * NW, col = lane + cc * 64;
                const int y = ty0 - 2 * R + r, xg = tx0 - G::CO + col;
                v[k][cc] = (r < G::XR && col < G::XS && y >= 0 && y < H && xg >= 0 && xg < W)
                               ? tld(xp, (uint32_t)(y * W + xg)) : 0.f;
            }
#pragma unroll
        for (int k = 0; k < RPW; ++k)
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                const int r = wave + k * NW, col = lane + cc * 64;
                if (r < G::XR && col < G::XS) xs[r * G::XS + col] = v[k][cc];
            }
    }
    __syncthreads();

    // ---- level-1 bands of the tile, positions -R .. 32 + R (zero outside the
    // level-1 plane follows from x being zero outside the plane)
    for (int e = tid; e < G::BR * G::BR; e += kTopThreads) {
        const int jy = e / G::BR, jx = e - jy * G::BR;
        const float* q = xs + (2 * jy) * G::XS + (G::CO - 2 * R + 2 * jx);
        const float a = q[0], b = q[1], cc = q[G::XS], d = q[G::XS + 1];
        const float s01 = a + b, d01 = a - b, s23 = cc + d, d23 = cc - d;
        float* o = bs + jy * G::BS + jx;
        o[0] = 0.5f * (s01 + s23);
        o[G::BSZ] = 0.5f * (d01 + d23);
        o[2 * G::BSZ] = 0.5f * (s01 - s23);
        o[3 * G::BSZ] = 0.5f * (d01 - d23);
    }

    // ---- base conv: this thread's 4 x 4 output block
    const int qy = tid >> 4, qx = tid & 15;
    // the deeper levels' result at this block's 2 x 2 level-1 positions, loaded
    // now so that its latency passes during the convolutions
    float zq[2][2];
    {
        const float* zp = zext ? zext + (size_t)p * h1 * w1 : nullptr;
#pragma unroll
        for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
            for (int b2 = 0; b2 < 2; ++b2) {
                const int gy = (ty0 >> 1) + 2 * qy + a2, gx = (tx0 >> 1) + 2 * qx + b2;
                zq[a2][b2] = (zp && gy < h1 && gx < w1) ? zp[gy * w1 + gx] : 0.f;
            }
    }
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
    // (a block that starts below the plane stores nothing: in the bottom tiles
    // of a plane whose height is not a multiple of the tile, whole waves skip)
    if (ty0 + 4 * qy < H) {
        float w[KK];
#pragma unroll
        for (int t = 0; t < KK; ++t) w[t] = w0[c * KK + t];
        tstencil<K>(xs + (4 * qy + R) * G::XS + (4 * qx + G::CO - R), G::XS, w, acc);
    }
    __syncthreads();   // bands written; every x read done

    // ---- level-1 conv: wave u convolves band u, lane l the 4 x 4 block (l / 8, l % 8)
    {
        const int u = wave, by = lane >> 3, bx = lane & 7;
        const size_t pu = (size_t)c * 4 + u;
        float w[KK];
#pragma unroll
        for (int t = 0; t < KK; ++t) w[t] = wl[pu * KK + t];
        const float su = sl[pu];
        float y1[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) y1[i][j] = 0.f;
        tstencil<K>(bs + u * G::BSZ + (4 * by) * G::BS + 4 * bx, G::BS, w, y1);
        // results over the dead x tile: ys[u][32][YS]
        float* yo = xs + u * G::YSZ + (4 * by) * G::YS + 4 * bx;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<tf4*>(yo + i * G::YS) = tf4{su * y1[i][0], su * y1[i][1], su * y1[i][2], su * y1[i][3]};
    }
    __syncthreads();

    // ---- level-1 synthesis (LL + the deeper levels' result) fused with the output
    const float sc = s0[c], bi = b0[c];
    float o[4][4];
#pragma unroll
    for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2) {
            const int jy = 2 * qy + a2, jx = 2 * qx + b2;   // level-1 position in the tile
            const float* yp = xs + jy * G::YS + jx;
            const float t0 = yp[0] + zq[a2][b2];
            const float t1 = yp[G::YSZ], t2 = yp[2 * G::YSZ], t3 = yp[3 * G::YSZ];
            const float pa = t0 + t1, pb = t0 - t1, pc = t2 + t3, pd = t2 - t3;
            o[2 * a2][2 * b2] = fmaf(sc, acc[2 * a2][2 * b2], bi) + 0.5f * (pa + pc);
            o[2 * a2][2 * b2 + 1] = fmaf(sc, acc[2 * a2][2 * b2 + 1], bi) + 0.5f * (pb + pd);
            o[2 * a2 + 1][2 * b2] = fmaf(sc, acc[2 * a2 + 1][2 * b2], bi) + 0.5f * (pa - pc);
            o[2 * a2 + 1][2 * b2 + 1] = fmaf(sc, acc[2 * a2 + 1][2 * b2 + 1], bi) + 0.5f * (pb - pd);
        }
    const int x0 = tx0 + 4 * qx;
    const bool vec = (W & 3) == 0 && x0 + 4 <= W;
    T* op = out + (size_t)p * hw;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int y = ty0 + 4 * qy + i;
        if (y >= H) continue;
        if (vec) {
            tst4(op, (uint32_t)(y * W + x0), o[i]);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (x0 + j < W) tst(op, (uint32_t)(y * W + x0 + j), o[i][j]);
        }
    }
}

// Backward of the top level over one 64 x 64 tile of plane p = b C + c:
//   dx = s0 (rot W0 * g) + synthesis(dS1),  dS1_u = s1_u (rot W1_u * G1_u) (+ dLL, band 0)
// with G1 = level-1 analysis of g (recomputed from the staged g tile), and the
// tile's correlations C0[d] = sum g[p] x[p + d], sum g, C1_u[d] = sum G1_u[j] X1_u[j + d]
// (X1 from this thread's own 4 x 4 block of x, which is exactly its 2 x 2
// level-1 positions).  Each window of g (G1) serves the rotated conv and the
// correlation with the x (X1) block, which yields C[-d]: stored un-rotated.
// Records: part0[(b ntile + tile) C + c][k^2 + 1] (slot k^2: sum g), part1[(b
// ntile + tile) 4C + 4c + u][k^2 + 1] (slot k^2: 0), for the per-level finalize.
template <int K, typename T>
__global__ void __launch_bounds__(kTopThreads) __attribute__((amdgpu_waves_per_eu(K <= 5 ? 3 : 2))) k_top_bwd(const T* __restrict__ x, const T* __restrict__ g, int C,
                                                         int H, int W, int ntx, int nty, const float* __restrict__ w0,
                                                         const float* __restrict__ s0, const float* __restrict__ wl,
                                                         const float* __restrict__ sl, const float* __restrict__ dll,
                                                         T* __restrict__ dx, float* __restrict__ part0,
                                                         float* __restrict__ part1, uint32_t nunit) {
    using G = TopGeom<K>;
    constexpr int R = G::R, KK = K * K;
    __shared__ __align__(16) float gs[G::XN];       // g tile; then X1; then the level-1 results
    __shared__ __align__(16) float bs[4 * G::BSZ];  // the four level-1 bands of g; then level-1 partials
    __shared__ float r0[16][KK + 1];                 // base correlation partials, one per 16-lane row
    const int ntile = ntx * nty;
    const uint32_t unit = top_unit(nunit);
    if (unit >= nunit) return;   // whole workgroup, before any barrier
    const int p = (int)(unit / ntile), tile = (int)(unit - (uint32_t)p * ntile);
    const int ty0 = (tile / ntx) * kTop, tx0 = (tile % ntx) * kTop;
    const int c = p % C, bb = p / C;
    const int h1 = (H + 1) >> 1, w1 = (W + 1) >> 1;
    const uint32_t hw = (uint32_t)H * W;
    const T* gp = g + (size_t)p * hw;
    const T* xp = x + (size_t)p * hw;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int qy = tid >> 4, qx = tid & 15;
    const int x0 = tx0 + 4 * qx;

    // ---- stage the g tile (as the forward's x tile); this thread's 4 x 4 block
    // of x and the sub-problem's gradient at its 2 x 2 level-1 positions into
    // registers; every load issued before any use
    float xb[4][4], zq[2][2];
    {
        constexpr int NW = kTopThreads / 64, RPW = (G::XR + NW - 1) / NW, CPL = (G::XS + 63) / 64;
        float v[RPW][CPL];
#pragma unroll
        for (int k = 0; k < RPW; ++k)
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                const int r = wave + k * NW, col = lane + cc * 64;
                const int y = ty0 - 2 * R + r, xg = tx0 - G::CO + col;
                v[k][cc] = (r < G::XR && col < G::XS && y >= 0 && y < H && xg >= 0 && xg < W)
                               ? tld(gp, (uint32_t)(y * W + xg)) : 0.f;
            }
        const bool xvec = (W & 3) == 0 && x0 + 4 <= W;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int y = ty0 + 4 * qy + i;
            if (xvec) {
                tld4(xp, (uint32_t)(min(y, H - 1) * W + x0), xb[i]);
                if (y >= H) xb[i][0] = xb[i][1] = xb[i][2] = xb[i][3] = 0.f;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    xb[i][j] = (y < H && x0 + j < W) ? tld(xp, (uint32_t)(y * W + x0 + j)) : 0.f;
            }
        }
        const float* zp = dll ? dll + (size_t)p * h1 * w1 : nullptr;
#pragma unroll
        for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
            for (int b2 = 0; b2 < 2; ++b2) {
                const int gy = (ty0 >> 1) + 2 * qy + a2, gx = (tx0 >> 1) + 2 * qx + b2;
                zq[a2][b2] = (zp && gy < h1 && gx < w1) ? zp[gy * w1 + gx] : 0.f;
            }
#pragma unroll
        for (int k = 0; k < RPW; ++k)
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                const int r = wave + k * NW, col = lane + cc * 64;
                if (r < G::XR && col < G::XS) gs[r * G::XS + col] = v[k][cc];
            }
    }
    __syncthreads();

    // ---- base: rotated conv of g, correlation of g with the x block, sum of g
    float acc[4][4], corr0[KK], sumg = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
#pragma unroll
    for (int q = 0; q < KK; ++q) corr0[q] = 0.f;
    {
        float w[KK];
#pragma unroll
        for (int t = 0; t < KK; ++t) w[t] = w0[c * KK + (KK - 1 - t)];
        tstencil_corr<K>(gs + (4 * qy + R) * G::XS + (4 * qx + G::CO - R), G::XS, w, acc, xb, corr0);
        const float* gc = gs + (4 * qy + 2 * R) * G::XS + (4 * qx + G::CO);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float r4[4];
            trow<4>(gc + i * G::XS, r4);
            sumg += (r4[0] + r4[1]) + (r4[2] + r4[3]);
        }
    }
    // base correlation: DPP row sums now (its accumulators are then free)
    const int row = tid >> 4;   // 16 rows of 16 lanes
#pragma unroll
    for (int q = 0; q < KK; ++q) corr0[q] = trow_sum(corr0[q]);
    sumg = trow_sum(sumg);
    if ((lane & 15) == 15) {
#pragma unroll
        for (int q = 0; q < KK; ++q) r0[row][q] = corr0[q];
        r0[row][KK] = sumg;
    }
    // ---- level-1 bands of g (positions -R .. 32 + R) into LDS
    for (int e = tid; e < G::BR * G::BR; e += kTopThreads) {
        const int jy = e / G::BR, jx = e - jy * G::BR;
        const float* q = gs + (2 * jy) * G::XS + (G::CO - 2 * R + 2 * jx);
        const float a = q[0], b = q[1], cc = q[G::XS], d = q[G::XS + 1];
        const float s01 = a + b, d01 = a - b, s23 = cc + d, d23 = cc - d;
        float* o = bs + jy * G::BS + jx;
        o[0] = 0.5f * (s01 + s23);
        o[G::BSZ] = 0.5f * (d01 + d23);
        o[2 * G::BSZ] = 0.5f * (s01 - s23);
        o[3 * G::BSZ] = 0.5f * (d01 - d23);
    }
    __syncthreads();   // g tile no longer read

    // ---- X1 of this thread's block (its 2 x 2 level-1 positions) over the g tile
#pragma unroll
    for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2) {
            const float a = xb[2 * a2][2 * b2], b = xb[2 * a2][2 * b2 + 1];
            const float cc = xb[2 * a2 + 1][2 * b2], d = xb[2 * a2 + 1][2 * b2 + 1];
            const float s01 = a + b, d01 = a - b, s23 = cc + d, d23 = cc - d;
            float* o = gs + (2 * qy + a2) * G::YS + 2 * qx + b2;
            o[0] = 0.5f * (s01 + s23);
            o[G::YSZ] = 0.5f * (d01 + d23);
            o[2 * G::YSZ] = 0.5f * (s01 - s23);
            o[3 * G::YSZ] = 0.5f * (d01 - d23);
        }
    __syncthreads();

    // ---- level 1: wave u takes band u, lane l the 4 x 4 block (l / 8, l % 8)
    float y1[4][4], corr1[KK];
    const int u = wave, by = lane >> 3, bx = lane & 7;
    const size_t pu = (size_t)c * 4 + u;
    const float su = sl[pu];
    {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) y1[i][j] = 0.f;
#pragma unroll
        for (int q = 0; q < KK; ++q) corr1[q] = 0.f;
        float w[KK];
#pragma unroll
        for (int t = 0; t < KK; ++t) w[t] = wl[pu * KK + (KK - 1 - t)];
        float xv[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) trow<4>(gs + u * G::YSZ + (4 * by + i) * G::YS + 4 * bx, xv[i]);
        tstencil_corr<K>(bs + u * G::BSZ + (4 * by) * G::BS + 4 * bx, G::BS, w, y1, xv, corr1);
    }
    __syncthreads();   // X1 and G1 no longer read
    {
        float* yo = gs + u * G::YSZ + (4 * by) * G::YS + 4 * bx;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<tf4*>(yo + i * G::YS) = tf4{su * y1[i][0], su * y1[i][1], su * y1[i][2], su * y1[i][3]};
    }
    // ---- level-1 correlation: DPP row sums, one partial per 16-lane row (over the bands)
    float* r1 = bs;   // [16][KK]: rows 4u .. 4u + 3 belong to band u
#pragma unroll
    for (int q = 0; q < KK; ++q) corr1[q] = trow_sum(corr1[q]);
    if ((lane & 15) == 15) {
#pragma unroll
        for (int q = 0; q < KK; ++q) r1[row * KK + q] = corr1[q];
    }
    __syncthreads();

    // ---- level-1 synthesis (+ the sub-problem's gradient on the LL band) and dx
    const float sc = s0[c];
    float o[4][4];
#pragma unroll
    for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2) {
            const float* yp = gs + (2 * qy + a2) * G::YS + 2 * qx + b2;
            const float t0 = yp[0] + zq[a2][b2];
            const float t1 = yp[G::YSZ], t2 = yp[2 * G::YSZ], t3 = yp[3 * G::YSZ];
            const float pa = t0 + t1, pb = t0 - t1, pc = t2 + t3, pd = t2 - t3;
            o[2 * a2][2 * b2] = fmaf(sc, acc[2 * a2][2 * b2], 0.5f * (pa + pc));
            o[2 * a2][2 * b2 + 1] = fmaf(sc, acc[2 * a2][2 * b2 + 1], 0.5f * (pb + pd));
            o[2 * a2 + 1][2 * b2] = fmaf(sc, acc[2 * a2 + 1][2 * b2], 0.5f * (pa - pc));
            o[2 * a2 + 1][2 * b2 + 1] = fmaf(sc, acc[2 * a2 + 1][2 * b2 + 1], 0.5f * (pb - pd));
        }
    const bool vec = (W & 3) == 0 && x0 + 4 <= W;
    T* op = dx + (size_t)p * hw;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int y = ty0 + 4 * qy + i;
        if (y >= H) continue;
        if (vec) {
            tst4(op, (uint32_t)(y * W + x0), o[i]);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (x0 + j < W) tst(op, (uint32_t)(y * W + x0 + j), o[i][j]);
        }
    }
    // ---- the tile's records (fixed summation order)
    const size_t blk = (size_t)bb * ntile + tile;
    for (int e = tid; e < (KK + 1) + 4 * (KK + 1); e += kTopThreads) {
        if (e < KK + 1) {
            float v = 0.f;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) v += r0[rr][e < KK ? KK - 1 - e : KK];
            part0[(blk * C + c) * (KK + 1) + e] = v;
        } else {
            const int f = e - (KK + 1), ub = f / (KK + 1), d = f - ub * (KK + 1);
            float v = 0.f;
            if (d < KK) {
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) v += r1[(4 * ub + rr) * KK + (KK - 1 - d)];
            }
            part1[(blk * 4 * C + (size_t)c * 4 + ub) * (KK + 1) + d] = v;
        }
    }
}

// Normalised LL band of level 1 (the sub-problem's input), one thread per
// level-1 position: ll[p][j] = (a + b + c + d) / 2 of the 2 x 2 block (zero
// beyond the plane).
template <typename T>
__global__ void __launch_bounds__(kTopThreads) k_top_ll(const T* __restrict__ x, uint32_t n, int H, int W,
                                                        float* __restrict__ ll) {
    const int h1 = (H + 1) >> 1, w1 = (W + 1) >> 1;
    for (uint32_t e = blockIdx.x * kTopThreads + threadIdx.x; e < n; e += gridDim.x * kTopThreads) {
        const uint32_t jx = e % (uint32_t)w1, t = e / (uint32_t)w1;
        const uint32_t jy = t % (uint32_t)h1, p = t / (uint32_t)h1;
        const T* xp = x + (size_t)p * H * W;
        const int y = 2 * (int)jy, xg = 2 * (int)jx;
        const bool rx = xg + 1 < W, ry = y + 1 < H;
        const float a = tld(xp, (uint32_t)(y * W + xg));
        const float b = rx ? tld(xp, (uint32_t)(y * W + xg + 1)) : 0.f;
        const float cc = ry ? tld(xp, (uint32_t)((y + 1) * W + xg)) : 0.f;
        const float d = (rx && ry) ? tld(xp, (uint32_t)((y + 1) * W + xg + 1)) : 0.f;
        ll[e] = 0.5f * ((a + b) + (cc + d));
    }
}

// fp32 planes with W % 4 == 0: one workgroup per LL row (plane p, row jy), a
// thread per two LL positions (one 16-byte load from each of the two x rows),
// no per-element index divisions; same sums in the same order as k_top_ll
__global__ void __launch_bounds__(64) k_top_ll4(const float* __restrict__ x, int H, int W, float* __restrict__ ll) {
    const int h1 = (H + 1) >> 1, w1 = W >> 1;
    const int row = blockIdx.x;   // p h1 + jy
    const int p = row / h1, jy = row - p * h1;
    const float* xr = x + (size_t)p * H * W + (size_t)(2 * jy) * W;
    const bool ry = 2 * jy + 1 < H;
    float* lr = ll + (size_t)row * w1;
    for (int q = threadIdx.x; q < (W >> 2); q += 64) {
        const float4 a = *reinterpret_cast<const float4*>(xr + 4 * q);
        const float4 b = ry ? *reinterpret_cast<const float4*>(xr + W + 4 * q) : make_float4(0.f, 0.f, 0.f, 0.f);
        float2 o;
        o.x = 0.5f * ((a.x + a.y) + (b.x + b.y));
        o.y = 0.5f * ((a.z + a.w) + (b.z + b.w));
        *reinterpret_cast<float2*>(lr + 2 * q) = o;
    }
}

template <int K, typename T>
int top_fwd_k(const wtc_desc* d, const void* x, const float* w0, const float* s0, const float* b0, const float* wl,
              const float* sl, const float* zext, void* out, hipStream_t st) {
    const int ntx = (d->W + kTop - 1) / kTop, nty = (d->H + kTop - 1) / kTop;
    const uint32_t nunit = (uint32_t)d->B * d->C * ntx * nty, grid = 8 * ((nunit + 7) / 8);
    hipLaunchKernelGGL((k_top_fwd<K, T>), dim3(grid), dim3(kTopThreads), 0, st, reinterpret_cast<const T*>(x), d->C,
                       d->H, d->W, ntx, nty, w0, s0, b0, wl, sl, zext, reinterpret_cast<T*>(out), nunit);
    return hipGetLastError() == hipSuccess ? WTC_OK : WTC_EHIP;
}

template <typename T>
int top_fwd_t(const wtc_desc* d, const void* x, const float* w0, const float* s0, const float* b0, const float* wl,
              const float* sl, const float* zext, void* out, hipStream_t st) {
    switch (d->k) {
        case 1: return top_fwd_k<1, T>(d, x, w0, s0, b0, wl, sl, zext, out, st);
        case 3: return top_fwd_k<3, T>(d, x, w0, s0, b0, wl, sl, zext, out, st);
        case 5: return top_fwd_k<5, T>(d, x, w0, s0, b0, wl, sl, zext, out, st);
        case 7: return top_fwd_k<7, T>(d, x, w0, s0, b0, wl, sl, zext, out, st);
        default: return WTC_ESHAPE;
    }
}

template <int K, typename T>
int top_bwd_k(const wtc_desc* d, const void* x, const void* g, const float* w0, const float* s0, const float* wl,
              const float* sl, const float* dll, void* dx, float* part0, float* part1, hipStream_t st) {
    const int ntx = (d->W + kTop - 1) / kTop, nty = (d->H + kTop - 1) / kTop;
    const uint32_t nunit = (uint32_t)d->B * d->C * ntx * nty, grid = 8 * ((nunit + 7) / 8);
    hipLaunchKernelGGL((k_top_bwd<K, T>), dim3(grid), dim3(kTopThreads), 0, st, reinterpret_cast<const T*>(x),
                       reinterpret_cast<const T*>(g), d->C, d->H, d->W, ntx, nty, w0, s0, wl, sl, dll,
                       reinterpret_cast<T*>(dx), part0, part1, nunit);
    return hipGetLastError() == hipSuccess ? WTC_OK : WTC_EHIP;
}

template <typename T>
int top_bwd_t(const wtc_desc* d, const void* x, const void* g, const float* w0, const float* s0, const float* wl,
              const float* sl, const float* dll, void* dx, float* part0, float* part1, hipStream_t st) {
    switch (d->k) {
        case 1: return top_bwd_k<1, T>(d, x, g, w0, s0, wl, sl, dll, dx, part0, part1, st);
        case 3: return top_bwd_k<3, T>(d, x, g, w0, s0, wl, sl, dll, dx, part0, part1, st);
        case 5: return top_bwd_k<5, T>(d, x, g, w0, s0, wl, sl, dll, dx, part0, part1, st);
        case 7: return top_bwd_k<7, T>(d, x, g, w0, s0, wl, sl, dll, dx, part0, part1, st);
        default: return WTC_ESHAPE;
    }
}

}  // namespace

int top_backward(const wtc_desc* d, const void* x, const void* g, const float* w0, const float* s0, const float* wl,
                 const float* sl, const float* dll, void* dx, float* part0, float* part1, void* stream) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    return d->dtype == WTC_BF16 ? top_bwd_t<uint16_t>(d, x, g, w0, s0, wl, sl, dll, dx, part0, part1, st)
                                : top_bwd_t<float>(d, x, g, w0, s0, wl, sl, dll, dx, part0, part1, st);
}

int top_forward(const wtc_desc* d, const void* x, const float* w0, const float* s0, const float* b0,
                const float* wl, const float* sl, const float* zext, void* out, void* stream) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    return d->dtype == WTC_BF16 ? top_fwd_t<uint16_t>(d, x, w0, s0, b0, wl, sl, zext, out, st)
                                : top_fwd_t<float>(d, x, w0, s0, b0, wl, sl, zext, out, st);
}

int top_ll(const wtc_desc* d, const void* x, float* ll, void* stream) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const uint32_t n = (uint32_t)d->B * d->C * ((d->H + 1) / 2) * ((d->W + 1) / 2);
    const uint32_t grid = std::max<uint32_t>(1, std::min<uint32_t>((n + kTopThreads - 1) / kTopThreads, 1u << 20));
    if (d->dtype == WTC_BF16)
        hipLaunchKernelGGL(k_top_ll<uint16_t>, dim3(grid), dim3(kTopThreads), 0, st,
                           reinterpret_cast<const uint16_t*>(x), n, d->H, d->W, ll);
    else if (d->W % 4 == 0)
        hipLaunchKernelGGL(k_top_ll4, dim3((uint32_t)d->B * d->C * ((d->H + 1) / 2)), dim3(64), 0, st,
                           reinterpret_cast<const float*>(x), d->H, d->W, ll);
    else
        hipLaunchKernelGGL(k_top_ll<float>, dim3(grid), dim3(kTopThreads), 0, st, reinterpret_cast<const float*>(x),
                           n, d->H, d->W, ll);
    return hipGetLastError() == hipSuccess ? WTC_OK : WTC_EHIP;
}

}  // namespace wtc
