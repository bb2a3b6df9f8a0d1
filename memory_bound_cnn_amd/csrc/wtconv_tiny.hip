// Register-resident WTConv for planes of at most 8 x 8 pixels (gfx950).
//
// Same operator and reformulations as the LDS plane pipeline (analysis
// recomputed on chip, closed-form synthesis, scales and Haar factors folded
// into the weights), organised for tiny planes: one quad of lanes holds one
// plane zero-extended to 8 x 8, each lane a 4 x 4 quadrant.  Convolution
// halos and subband exchanges travel between the four lanes of the quad by
// DPP quad permutes; a workgroup is one wave, 16 planes of 16 consecutive
// channels in flight, and LDS holds only the group's folded weights.
//
// Level 1 (4 x 4 grid) and level 2 (2 x 2 grid) use the band-per-lane scheme:
// lane t gathers subband t over the whole grid in canonical order, convolves
// it with its own folded weights (taps that fall outside the grid are skipped
// at compile time) and, for the synthesis, hands every other lane the values
// at that lane's positions.  Supported: k = 5, 1 <= L = Lm <= 2, H, W <= 8.
#include <hip/hip_runtime.h>

#include "wtc_internal.h"
#include "wtc_numeric.h"

namespace wtc {
namespace tiny {

constexpr int K = 5, R = K / 2, KK = K * K;
constexpr int WN = 4 + 2 * R;   // window side of a 4 x 4 block

struct bf16v {
    uint16_t bits;
};

// Plane I/O through raw buffer resources: the hardware range check returns 0 for
// a load at or beyond `num_records` bytes and drops such a store, so every load
// and store of a pass is issued unconditionally (a pixel outside the plane, or a
// quad past the end of the batch, simply addresses beyond the range).
using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr uint32_t kRsrcWord3 = 0x00020000;   // raw 32-bit data format (gfx9)
constexpr int kOutOfRange = 0x7FFFFFF0;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ float bload(rsrc_t r, int off, float*) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ float bload(rsrc_t r, int off, bf16v*) {
    return __uint_as_float(((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0)) << 16);
}
__device__ __forceinline__ void bstore(rsrc_t r, int off, float v, float*) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}
__device__ __forceinline__ void bstore(rsrc_t r, int off, float v, bf16v*) {
    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)bf16_rne(v), r, off, 0, 0);
}

// Value of `v` in quad lane (lane ^ X); X = 0 is the lane itself.
constexpr int quad_xor_ctrl(int x) {
    // quad_perm selector: lane i of each quad reads lane sel[i]
    return ((0 ^ x) << 0) | ((1 ^ x) << 2) | ((2 ^ x) << 4) | ((3 ^ x) << 6);
}
template <int X>
__device__ __forceinline__ float qx(float v) {
    if constexpr (X == 0) {
        return v;
    } else {
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), quad_xor_ctrl(X), 0xF, 0xF, true));
    }
}

// a[i] for a lane-dependent index 0 <= i < 4 (two selects on its bits).  The
// candidates are pinned to registers first: otherwise the optimizer may turn the
// selects into a dynamically indexed (hence memory-resident) array.
__device__ __forceinline__ float sel4(const float (&a)[4], int i) {
    float a0 = a[0], a1 = a[1], a2 = a[2], a3 = a[3];
    asm volatile("" : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3));
    const float lo = (i & 1) ? a1 : a0;
    const float hi = (i & 1) ? a3 : a2;
    return (i & 2) ? hi : lo;
}

// c ? x : y on register values (pinned, for the same reason as sel4)
__device__ __forceinline__ float selv(bool c, float x, float y) {
    asm volatile("" : "+v"(x), "+v"(y));
    return c ? x : y;
}

// Raw +-1 butterfly of a 2 x 2 block a=(0,0), b=(0,1), c=(1,0), d=(1,1).
__device__ __forceinline__ void haar4(float a, float b, float c, float d, float (&r)[4]) {
    const float s01 = a + b, d01 = a - b, s23 = c + d, d23 = c - d;
    r[0] = s01 + s23;
    r[1] = d01 + d23;
    r[2] = s01 - s23;
    r[3] = d01 - d23;
}

// Halo of this lane's 4 x 4 block of a plane held by the quad (block of lane t
// at quadrant (t >> 1, t & 1)): the vertical partner (lane ^ 2) sends its R rows
// next to us, the horizontal one (lane ^ 1) its R columns, the diagonal one
// (lane ^ 3) its R x R corner.  Zero where the partner lies outside the plane.
struct Halo {
    float vr[R][4], hc[4][R], dg[R][R];
};
__device__ __forceinline__ void exchange_halo(const float (&X)[4][4], int sy, int sx, Halo& h) {
    auto& vr = h.vr;
    auto& hc = h.hc;
    auto& dg = h.dg;
#pragma unroll
    for (int k = 0; k < R; ++k)
#pragma unroll
        for (int j = 0; j < 4; ++j) vr[k][j] = qx<2>(selv(sy != 0, X[k][j], X[4 - R + k][j]));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < R; ++k) hc[i][k] = qx<1>(selv(sx != 0, X[i][k], X[i][4 - R + k]));
#pragma unroll
    for (int k = 0; k < R; ++k)
#pragma unroll
        for (int l = 0; l < R; ++l)
            dg[k][l] = qx<3>(selv(sy != 0, selv(sx != 0, X[k][l], X[k][4 - R + l]),
                                  selv(sx != 0, X[4 - R + k][l], X[4 - R + k][4 - R + l])));
    // keep only the halo that lies inside the plane: the partners' blocks are above
    // (sy = 1) or below, left (sx = 1) or right; the other side is the plane border
}

// Row r of the (4 + 2R)^2 window around the lane's block (rows/cols -R .. 3+R).
__device__ __forceinline__ void window_row(const float (&X)[4][4], const Halo& h, bool above, bool left, int r,
                                           float (&row)[WN]) {
    const int rb = r < R ? 0 : (r < R + 4 ? 1 : 2);   // 0 above, 1 own, 2 below
    const int rr = rb == 0 ? r : (rb == 1 ? r - R : r - R - 4);
#pragma unroll
    for (int c = 0; c < WN; ++c) {
        const int cb = c < R ? 0 : (c < R + 4 ? 1 : 2);
        const int cc = cb == 0 ? c : (cb == 1 ? c - R : c - R - 4);
        float v;
        if (rb == 1 && cb == 1) {
            v = X[rr][cc];
        } else if (cb == 1) {
            v = ((rb == 0) == above) ? h.vr[rr][cc] : 0.f;
        } else if (rb == 1) {
            v = ((cb == 0) == left) ? h.hc[rr][cc] : 0.f;
        } else {
            v = ((rb == 0) == above && (cb == 0) == left) ? h.dg[rr][cc] : 0.f;
        }
        row[c] = v;
    }
}

// Gather subband t of the quad's N x N level grid in canonical order: lane q
// holds bands[jy][jx][u] at its (N/2 x N/2) block (quadrant (q >> 1, q & 1)).
template <int NB>   // block side (N = 2 NB)
__device__ __forceinline__ void gather_band(const float (&bands)[NB][NB][4], int t, float (&G)[2 * NB][2 * NB]) {
    float rv[4][NB][NB];
#pragma unroll
    for (int jy = 0; jy < NB; ++jy)
#pragma unroll
        for (int jx = 0; jx < NB; ++jx) {
            // round r: the partner t ^ r receives its own band (t ^ r) of our block
            rv[0][jy][jx] = sel4(bands[jy][jx], t);
            rv[1][jy][jx] = qx<1>(sel4(bands[jy][jx], t ^ 1));
            rv[2][jy][jx] = qx<2>(sel4(bands[jy][jx], t ^ 2));
            rv[3][jy][jx] = qx<3>(sel4(bands[jy][jx], t ^ 3));
        }
    // block (Y, X) came from lane (Y, X), i.e. in round ((Y << 1) | X) ^ t
#pragma unroll
    for (int Y = 0; Y < 2; ++Y)
#pragma unroll
        for (int Xb = 0; Xb < 2; ++Xb)
#pragma unroll
            for (int jy = 0; jy < NB; ++jy)
#pragma unroll
                for (int jx = 0; jx < NB; ++jx) {
                    const float c4[4] = {rv[0][jy][jx], rv[1][jy][jx], rv[2][jy][jx], rv[3][jy][jx]};
                    G[Y * NB + jy][Xb * NB + jx] = sel4(c4, ((Y << 1) | Xb) ^ t);
                }
}

// Depthwise K x K correlation on an N x N grid with zero padding, taps outside
// the grid skipped at compile time.  CORR: also cr[ky][kx] += xs[y][x] g[y+ky-R][x+kx-R].
template <int N, bool CORR>
__device__ __forceinline__ void grid_conv(const float (&G)[N][N], const float (&w)[KK], float (&Y)[N][N],
                                          const float (&xs)[N][N], float (&cr)[KK]) {
#pragma unroll
    for (int y = 0; y < N; ++y)
#pragma unroll
        for (int x = 0; x < N; ++x) {
            float acc = 0.f;
#pragma unroll
            for (int ky = 0; ky < K; ++ky)
#pragma unroll
                for (int kx = 0; kx < K; ++kx) {
                    const int gy = y + ky - R, gx = x + kx - R;
                    if (gy < 0 || gy >= N || gx < 0 || gx >= N) continue;
                    acc = fmaf(w[ky * K + kx], G[gy][gx], acc);
                    if constexpr (CORR) cr[ky * K + kx] = fmaf(xs[y][x], G[gy][gx], cr[ky * K + kx]);
                }
            Y[y][x] = acc;
        }
}

// Synthesis hand-over: lane t holds band t on the canonical N x N grid; every lane
// receives, for each band u, the values at its own block and adds them with the
// signs of the inverse butterfly: z[2jy+dy][2jx+dx] += (-1)^(u_y dy + u_x dx) Y^u[jy][jx]
// (NB x NB positions per block, z is 2NB x 2NB).
template <int NB>
__device__ __forceinline__ void synth_band(const float (&Yc)[2 * NB][2 * NB], int t, float (&z)[2 * NB][2 * NB]) {
    float rv[4][NB][NB];
#pragma unroll
    for (int jy = 0; jy < NB; ++jy)
#pragma unroll
        for (int jx = 0; jx < NB; ++jx) {
            // round r: the partner p = t ^ r needs our band at its block (p >> 1, p & 1)
            float blk[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) blk[b] = Yc[(b >> 1) * NB + jy][(b & 1) * NB + jx];
            rv[0][jy][jx] = sel4(blk, t);
            rv[1][jy][jx] = qx<1>(sel4(blk, t ^ 1));
            rv[2][jy][jx] = qx<2>(sel4(blk, t ^ 2));
            rv[3][jy][jx] = qx<3>(sel4(blk, t ^ 3));
        }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int u = t ^ r;   // band received in round r
        const float sgx = (u & 1) ? -1.f : 1.f, sgy = (u & 2) ? -1.f : 1.f, sgxy = sgx * sgy;
#pragma unroll
        for (int jy = 0; jy < NB; ++jy)
#pragma unroll
            for (int jx = 0; jx < NB; ++jx) {
                const float v = rv[r][jy][jx];
                z[2 * jy][2 * jx] += v;
                z[2 * jy][2 * jx + 1] = fmaf(sgx, v, z[2 * jy][2 * jx + 1]);
                z[2 * jy + 1][2 * jx] = fmaf(sgy, v, z[2 * jy + 1][2 * jx]);
                z[2 * jy + 1][2 * jx + 1] = fmaf(sgxy, v, z[2 * jy + 1][2 * jx + 1]);
            }
    }
}

__device__ __forceinline__ float wave_sum(float v, int from) {
    for (int m = from; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Byte offset of pixel (i, j) of the lane's quadrant in a plane starting at
// byte `pbyte` of the resource; out of range outside H x W.
template <typename ST>
__device__ __forceinline__ int pix_off(int pbyte, int H, int W, int sy, int sx, int i, int j) {
    const int y = 4 * sy + i, x = 4 * sx + j;
    return (y < H && x < W) ? pbyte + (y * W + x) * (int)sizeof(ST) : kOutOfRange;
}

// The lane's 4 x 4 quadrant of the plane at byte `pbyte` (zero outside H x W and
// beyond the resource's range).
template <typename ST>
__device__ __forceinline__ void load_quadrant(rsrc_t r, int pbyte, int H, int W, int sy, int sx, float (&X)[4][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) X[i][j] = bload(r, pix_off<ST>(pbyte, H, W, sy, sx, i, j), (ST*)nullptr);
}

// Opaque copy: keeps the compiler from hoisting lane-dependent values out of
// the plane loop (they are cheap to recompute, expensive to keep live).
__device__ __forceinline__ int opaque(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

// One wave per workgroup: 16 consecutive channels c0 .. c0 + 15 (quad i takes
// channel c0 + i) and the batch entries of one chunk, one pass per entry.  The
// 16 planes of a pass are adjacent in memory, so a pass reads and writes one
// contiguous span; each quad keeps its channel, hence its weights and its
// weight-gradient accumulators, for the whole workgroup.
template <typename ST, bool BWD, int LM>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(BWD ? 2 : 3)))
wtc_tiny_kernel(const FusedArgs a) {
    constexpr int WPC = KK * (1 + 4 * LM);   // weights per channel: base, then the bands of each level
    __shared__ float wsh[16 * WPC];
    const int lane = threadIdx.x;
    const int ngrp = (a.C + 15) >> 4;
    const int grp = blockIdx.x % ngrp, chunk = blockIdx.x / ngrp;
    const int c0 = grp * 16, nch = min(16, a.C - c0);
    const int b_lo = chunk * a.ppw, b_hi = min(a.B, b_lo + a.ppw);
    const int HW = a.H * a.W;
    const int pbytes = HW * (int)sizeof(ST);
    const ST* srcp = reinterpret_cast<const ST*>(a.src);
    const ST* auxp = reinterpret_cast<const ST*>(a.aux);
    ST* dstp = reinterpret_cast<ST*>(a.dst);

    // weights of the group's channels: base (unfolded; s0 is applied at the
    // output) and every band of every level folded with its scale and 4^-i;
    // rotated by 180 degrees for the backward
    for (int e = lane; e < nch * WPC; e += 64) {
        const int cq = e / WPC, r = e - cq * WPC;
        const int blk = r / KK, q = r - blk * KK, tap = BWD ? KK - 1 - q : q;
        const int c = c0 + cq;
        float v;
        if (blk == 0) {
            v = a.w0[(size_t)c * KK + tap];
        } else {
            const int i = (blk - 1) >> 2, u = (blk - 1) & 3;   // level i + 1, band u
            const size_t pu = ((size_t)i * a.C + c) * 4 + u;
            v = ldexpf(a.sl[pu], -2 * (i + 1)) * a.wl[pu * KK + tap];
        }
        wsh[e] = v;
    }
    __syncthreads();
    const int quad0 = lane >> 2;
    const bool cok = quad0 < nch;   // quad-uniform
    const int cme = c0 + (cok ? quad0 : 0);
    const float s0 = cok ? a.s0[cme] : 0.f;
    const float bias = (BWD || !cok) ? 0.f : a.b0[cme];
    float corr0[KK], corr1[KK], corr2[KK];
#pragma unroll
    for (int q = 0; q < KK; ++q) corr0[q] = corr1[q] = corr2[q] = 0.f;
    float sumg = 0.f;

    // pass b covers planes (b, c0) .. (b, c0 + nch - 1): one resource per pass
    auto pass_rsrc = [&](const ST* base, int b) { return make_rsrc(base + ((size_t)b * a.C + c0) * HW, nch * pbytes); };
    float Xn[4][4], xn[4][4];
    {
        const int ln = opaque(lane), t = ln & 3, pb = (ln >> 2) * pbytes;
        load_quadrant<ST>(pass_rsrc(srcp, b_lo), pb, a.H, a.W, t >> 1, t & 1, Xn);
        if constexpr (BWD) load_quadrant<ST>(pass_rsrc(auxp, b_lo), pb, a.H, a.W, t >> 1, t & 1, xn);
    }
    for (int b = b_lo; b < b_hi; ++b) {
        const int ln = opaque(lane);
        const int t = ln & 3, quad = ln >> 2;
        const int sy = t >> 1, sx = t & 1;
        const int pbyte = quad * pbytes;   // beyond the pass's range for a quad past the last channel
        const float* wq = wsh + quad * WPC;
        float X[4][4], xs[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                X[i][j] = Xn[i][j];
                if constexpr (BWD) xs[i][j] = xn[i][j];
            }
        if (b + 1 < b_hi) {
            load_quadrant<ST>(pass_rsrc(srcp, b + 1), pbyte, a.H, a.W, sy, sx, Xn);
            if constexpr (BWD) load_quadrant<ST>(pass_rsrc(auxp, b + 1), pbyte, a.H, a.W, sy, sx, xn);
        }

        // ---- base convolution (and correlation of x with g), one window row at a time ----
        float acc[4][4];
        {
            Halo h;
            exchange_halo(X, sy, sx, h);
            float w0[KK];
#pragma unroll
            for (int q = 0; q < KK; ++q) w0[q] = wq[q];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
#pragma unroll
            for (int r = 0; r < WN; ++r) {
                float row[WN];
                window_row(X, h, sy != 0, sx != 0, r, row);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ky = r - i;
                    if (ky < 0 || ky >= K) continue;
#pragma unroll
                    for (int kx = 0; kx < K; ++kx)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            acc[i][j] = fmaf(w0[ky * K + kx], row[j + kx], acc[i][j]);
                            if constexpr (BWD)
                                corr0[ky * K + kx] = fmaf(xs[i][j], row[j + kx], corr0[ky * K + kx]);
                        }
                }
            }
        }
        if constexpr (BWD) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) sumg += X[i][j];
        }
        // phase boundary: keeps the scheduler from overlapping the phases' live ranges
        __builtin_amdgcn_sched_barrier(0);

        // ---- level 1: raw bands of this lane's 2 x 2 positions ----
        float hv[2][2][4], hx[2][2][4];
#pragma unroll
        for (int jy = 0; jy < 2; ++jy)
#pragma unroll
            for (int jx = 0; jx < 2; ++jx) {
                haar4(X[2 * jy][2 * jx], X[2 * jy][2 * jx + 1], X[2 * jy + 1][2 * jx], X[2 * jy + 1][2 * jx + 1],
                      hv[jy][jx]);
                if constexpr (BWD)
                    haar4(xs[2 * jy][2 * jx], xs[2 * jy][2 * jx + 1], xs[2 * jy + 1][2 * jx], xs[2 * jy + 1][2 * jx + 1],
                          hx[jy][jx]);
            }
        float G1[4][4], Y1[4][4], X1[4][4];
        gather_band<2>(hv, t, G1);
        if constexpr (BWD) gather_band<2>(hx, t, X1);
        __builtin_amdgcn_sched_barrier(0);
        {
            float w1[KK];
#pragma unroll
            for (int q = 0; q < KK; ++q) w1[q] = wq[KK + t * KK + q];
            grid_conv<4, BWD>(G1, w1, Y1, X1, corr1);
        }
        __builtin_amdgcn_sched_barrier(0);

        float z[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) z[i][j] = 0.f;

        // ---- level 2 (this lane's block is one level-2 position) ----
        if constexpr (LM >= 2) {
            float h2[1][1][4], x2[1][1][4];
            haar4(hv[0][0][0], hv[0][1][0], hv[1][0][0], hv[1][1][0], h2[0][0]);
            if constexpr (BWD) haar4(hx[0][0][0], hx[0][1][0], hx[1][0][0], hx[1][1][0], x2[0][0]);
            float G2[2][2], Y2[2][2], X2[2][2];
            gather_band<1>(h2, t, G2);
            if constexpr (BWD) gather_band<1>(x2, t, X2);
            float w2[KK];
#pragma unroll
            for (int q = 0; q < KK; ++q) w2[q] = wq[5 * KK + t * KK + q];
            grid_conv<2, BWD>(G2, w2, Y2, X2, corr2);
            // level-2 synthesis: the LL input of level 1 at this lane's 2 x 2 positions
            float z2[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
            synth_band<1>(Y2, t, z2);
            // enters the level-1 butterfly through band 0: +z2 at all four pixels
#pragma unroll
            for (int jy = 0; jy < 2; ++jy)
#pragma unroll
                for (int jx = 0; jx < 2; ++jx)
#pragma unroll
                    for (int dy = 0; dy < 2; ++dy)
#pragma unroll
                        for (int dx = 0; dx < 2; ++dx) z[2 * jy + dy][2 * jx + dx] += z2[jy][jx];
        }
        __builtin_amdgcn_sched_barrier(0);
        // ---- level-1 synthesis fused with the output ----
        synth_band<2>(Y1, t, z);
        const rsrc_t rd = pass_rsrc(dstp, b);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bstore(rd, pix_off<ST>(pbyte, a.H, a.W, sy, sx, i, j), fmaf(s0, acc[i][j], bias + z[i][j]),
                       (ST*)nullptr);
    }

    if constexpr (BWD) {
        // record of (chunk, channel): [C_0][level 1: 4 bands][level 2: 4 bands][sum g]
        // [tail = 0], correlations in weight-gradient tap order (accumulator q holds
        // tap KK-1-q); lane t of a quad holds band t of levels 1, 2
        const int t = lane & 3;
        float* rec = a.partials + ((size_t)chunk * a.C + cme) * a.P;
#pragma unroll
        for (int q = 0; q < KK; ++q) {
            float v0 = corr0[q];
            v0 += qx<1>(v0);
            v0 += qx<2>(v0);
            if (cok) {
                if (t == 0) rec[KK - 1 - q] = v0;
                rec[KK + t * KK + (KK - 1 - q)] = corr1[q];
                if constexpr (LM >= 2) rec[5 * KK + t * KK + (KK - 1 - q)] = corr2[q];
            }
        }
        float vs = sumg;
        vs += qx<1>(vs);
        vs += qx<2>(vs);
        if (cok && t == 0) {
            rec[a.P - 2] = vs;
            rec[a.P - 1] = 0.f;
        }
    }
}

template <typename ST, bool BWD>
hipError_t launch_dt(const FusedArgs& a, int grid, hipStream_t st) {
    if (a.Lm == 1)
        hipLaunchKernelGGL((wtc_tiny_kernel<ST, BWD, 1>), dim3(grid), dim3(64), 0, st, a);
    else
        hipLaunchKernelGGL((wtc_tiny_kernel<ST, BWD, 2>), dim3(grid), dim3(64), 0, st, a);
    return hipGetLastError();
}

}  // namespace tiny

int launch_tiny(const FusedArgs& a, int dtype, int bwd, int grid, void* stream) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    using namespace tiny;
    if (dtype == WTC_BF16) return (int)(bwd ? launch_dt<bf16v, true>(a, grid, st) : launch_dt<bf16v, false>(a, grid, st));
    return (int)(bwd ? launch_dt<float, true>(a, grid, st) : launch_dt<float, false>(a, grid, st));
}

}  // namespace wtc
