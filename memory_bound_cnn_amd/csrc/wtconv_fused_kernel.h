// Fused WTConv forward / backward for gfx950 (MI355X): kernel template.
// Instantiated once per kernel size in wtconv_fused_k<k>.hip.
//
// Method: "Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware
// Reformulation" (arXiv 2608.10805, Abstract) names three reformulations of
// the WTConv operator; all three are used here, re-derived for CDNA4:
//   (1) the Haar analysis butterfly is recomputed on chip (LDS / registers)
//       instead of storing subbands in HBM;
//   (2) the multi-level synthesis is one pass whose signs are indexed by the
//       output-coordinate bits (evaluated deepest level first, one LDS pass per
//       level, the last one fused with the output store);
//   (3) the per-channel scales -- and the 2^-i Haar normalisations of analysis
//       and synthesis -- are folded into the convolution weights,
//       W'_i = 4^-i * s_i * W_i and W'_0 = s0 * W0, so every butterfly is a raw
//       +-1 sum.
// HBM traffic is one read of the convolved tensor, one write of the result
// and, in the backward pass, one read of x.
//
// Work decomposition (one workgroup = one channel, a chunk of the batch):
//   * each plane is staged in LDS with a zero halo of k/2 and zero-extended to
//     Hq x Wq (multiples of max(8, 2^Lm)); zero extension is exactly the
//     "pad to even before each analysis, crop after each synthesis" rule;
//   * 4 lanes ("a quad") own an 8x8 pixel block.  At level 0 each lane owns a
//     4x4 sub-block; at levels 1 and 2 lane t convolves subband t over the
//     whole quad block (4x4 resp. 2x2 positions), so one lane needs one set
//     of k*k weights and one set of correlation accumulators per level;
//   * levels >= 3 (grids of at most one position per quad) are flat loops;
//     their weight-gradient correlations are output-stationary (one thread
//     per subband x tap x position subset) so they need one register each.
// The backward pass is the same pipeline applied to g with 180-degree-rotated
// weights (the adjoint: the orthonormal Haar matrix is symmetric, so analysis
// and synthesis are each other's transpose), plus the correlations
//   C_0[d] = sum g[p] x[p+d],   C_i^u[d] = sum R_i^u(g)[j] R_i^u(x)[j+d]
// accumulated in registers across the workgroup's planes and reduced once.
#pragma once
#include <hip/hip_runtime.h>

#include "wtc_internal.h"

namespace wtc {
namespace fused_detail {

// ---------------------------------------------------------------------------
// storage <-> float32
// ---------------------------------------------------------------------------
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return __uint_as_float(((uint32_t)v.bits) << 16); }

__device__ __forceinline__ void from_f32(float& d, float v) { d = v; }
__device__ __forceinline__ void from_f32(bf16_t& d, float v) {
    // round to nearest, ties to even (finite inputs)
    uint32_t u = __float_as_uint(v);
    u += 0x7FFFu + ((u >> 16) & 1u);
    d.bits = (uint16_t)(u >> 16);
}

// Four consecutive pixels (the caller guarantees 4-pixel alignment).
__device__ __forceinline__ void load4(const float* p, float (&v)[4]) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}
__device__ __forceinline__ void load4(const bf16_t* p, float (&v)[4]) {
    const uint2 q = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(q.x << 16);
    v[1] = __uint_as_float(q.x & 0xFFFF0000u);
    v[2] = __uint_as_float(q.y << 16);
    v[3] = __uint_as_float(q.y & 0xFFFF0000u);
}
__device__ __forceinline__ void store4(float* p, const float (&v)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store4(bf16_t* p, const float (&v)[4]) {
    bf16_t b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) from_f32(b[i], v[i]);
    uint2 q;
    q.x = (uint32_t)b[0].bits | ((uint32_t)b[1].bits << 16);
    q.y = (uint32_t)b[2].bits | ((uint32_t)b[3].bits << 16);
    *reinterpret_cast<uint2*>(p) = q;
}

// ---------------------------------------------------------------------------
// LDS helpers
// ---------------------------------------------------------------------------
// Read WW consecutive floats; AL = guaranteed alignment of p in floats (4, 2, 1).
template <int WW, int AL>
__device__ __forceinline__ void lds_row(const float* p, float (&row)[WW]) {
    if constexpr (AL == 4) {
#pragma unroll
        for (int q = 0; q + 4 <= WW; q += 4) {
            const float4 v = *reinterpret_cast<const float4*>(p + q);
            row[q] = v.x; row[q + 1] = v.y; row[q + 2] = v.z; row[q + 3] = v.w;
        }
        constexpr int done = (WW / 4) * 4;
        if constexpr (WW - done >= 2) {
            const float2 v = *reinterpret_cast<const float2*>(p + done);
            row[done] = v.x; row[done + 1] = v.y;
        }
        if constexpr ((WW - done) % 2 == 1) row[WW - 1] = p[WW - 1];
    } else if constexpr (AL == 2) {
#pragma unroll
        for (int q = 0; q + 2 <= WW; q += 2) {
            const float2 v = *reinterpret_cast<const float2*>(p + q);
            row[q] = v.x; row[q + 1] = v.y;
        }
        if constexpr (WW % 2 == 1) row[WW - 1] = p[WW - 1];
    } else {
#pragma unroll
        for (int q = 0; q < WW; ++q) row[q] = p[q];
    }
}

// Zero every element of a rows x S array outside the rectangle [r0,r1) x [c0,c1).
__device__ void zero_ring(float* base, int rows, int S, int r0, int r1, int c0, int c1, int tid,
                          int nthr) {
    const int top = r0 * S;
    const int bot = (rows - r1) * S;
    const int side = c0 + (S - c1);
    const int mid = (r1 - r0) * side;
    const int n = top + bot + mid;
    for (int e = tid; e < n; e += nthr) {
        int idx;
        if (e < top) {
            idx = e;
        } else if (e < top + bot) {
            idx = r1 * S + (e - top);
        } else {
            const int m = e - top - bot;
            const int row = r0 + m / side;
            const int col = m % side;
            idx = row * S + (col < c0 ? col : c1 + (col - c0));
        }
        base[idx] = 0.f;
    }
}

// ---------------------------------------------------------------------------
// Register-blocked stencil: OH x OW outputs from an (OH+K-1) x (OW+K-1) LDS
// window, one window row live at a time.
//   acc[oy][ox]   += w[ky][kx] * win[oy+ky][ox+kx]
//   corr[ky][kx]  += xv[oy][ox] * win[oy+ky][ox+kx]     (CORR only)
// ---------------------------------------------------------------------------
template <int K, int OH, int OW, int AL, bool CORR>
__device__ __forceinline__ void stencil(const float* win, int S, const float (&w)[K * K],
                                        float (&acc)[OH][OW], const float (&xv)[OH][OW],
                                        float (&corr)[K * K]) {
    constexpr int WH = OH + K - 1, WW = OW + K - 1;
    // Two window rows live: row wy+1 is read while row wy is consumed.  The
    // scheduling barrier keeps the compiler from hoisting every row's LDS
    // read to the top (which would hold the whole window in registers).
    float rows[2][WW];
    lds_row<WW, AL>(win, rows[0]);
#pragma unroll
    for (int wy = 0; wy < WH; ++wy) {
        float (&row)[WW] = rows[wy & 1];
        if (wy + 1 < WH) lds_row<WW, AL>(win + (wy + 1) * S, rows[(wy + 1) & 1]);
#pragma unroll
        for (int oy = 0; oy < OH; ++oy) {
            const int ky = wy - oy;
            if (ky < 0 || ky >= K) continue;
#pragma unroll
            for (int kx = 0; kx < K; ++kx) {
#pragma unroll
                for (int ox = 0; ox < OW; ++ox) {
                    acc[oy][ox] = fmaf(w[ky * K + kx], row[ox + kx], acc[oy][ox]);
                    if constexpr (CORR)
                        corr[ky * K + kx] = fmaf(xv[oy][ox], row[ox + kx], corr[ky * K + kx]);
                }
            }
        }
        // Pin this row's results before the next row is read (keeps the live
        // window to two rows instead of the whole window).
#pragma unroll
        for (int oy = 0; oy < OH; ++oy)
#pragma unroll
            for (int ox = 0; ox < OW; ++ox) asm volatile("" : "+v"(acc[oy][ox]));
        if constexpr (CORR) {
#pragma unroll
            for (int q = 0; q < K * K; ++q) asm volatile("" : "+v"(corr[q]));
        }
        asm volatile("" ::: "memory");
    }
}

// Folded weights of one (level, band) from LDS; ROT = 180-degree rotation.
template <int K, bool ROT>
__device__ __forceinline__ void load_w(const float* p, float (&w)[K * K]) {
#pragma unroll
    for (int t = 0; t < K * K; ++t) w[t] = p[ROT ? (K * K - 1 - t) : t];
}

// Pixel (y, x) of a plane, zero outside [0,H) x [0,W).
template <typename ST>
__device__ __forceinline__ float ld_px(const ST* plane, int y, int x, int H, int W) {
    return (y < H && x < W) ? to_f32(plane[y * W + x]) : 0.f;
}

// Four pixels starting at `rowp` (= image pixel (y, x), x % 4 == 0); zero where
// the row is outside the image (row_ok false) or a column is >= W.
template <bool VEC, typename ST>
__device__ __forceinline__ void ld_row4(const ST* rowp, bool row_ok, int x, int W, float (&v)[4]) {
    if constexpr (VEC) {
        if (row_ok && x < W) {
            load4(rowp, v);
        } else {
            v[0] = v[1] = v[2] = v[3] = 0.f;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (row_ok && x + i < W) ? to_f32(rowp[i]) : 0.f;
    }
}

// Opaque copy of a per-thread offset: keeps the compiler from hoisting the
// addresses derived from it out of the plane loop as 64-bit pointers.
__device__ __forceinline__ int opaque(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

__device__ __forceinline__ float wave_sum(float v, int width_mask_from) {
    // xor-butterfly over lane bits >= log2(width_mask_from)
    for (int m = width_mask_from; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// ---------------------------------------------------------------------------
// The fused kernel
// ---------------------------------------------------------------------------
template <int K, typename ST, bool BWD, int BPQ, bool VEC>
__global__ void __launch_bounds__(512) wtc_fused_kernel(const FusedArgs a) {
    constexpr int R = K / 2, KK = K * K;
    extern __shared__ __align__(16) float lds[];

    const int tid = threadIdx.x, nthr = blockDim.x, nquads = nthr >> 2;
    const int c = blockIdx.x % a.C, chunk = blockIdx.x / a.C;
    const int b_begin = chunk * a.bpc;
    const int b_end = min(a.B, b_begin + a.bpc);
    const int t = tid & 3, Q = tid >> 2;
    const int sy = t >> 1, sx = t & 1;
    const float sgx = (t & 1) ? -1.f : 1.f;   // sign of the W-direction high-pass for band t
    const float sgy = (t & 2) ? -1.f : 1.f;   // sign of the H-direction high-pass for band t
    const int Lm = a.Lm;
    const size_t plane_sz = (size_t)a.H * a.W;

    int slot, qpb[BPQ];
    if constexpr (BPQ == 1) {
        slot = Q / a.qpp;
        qpb[0] = Q - slot * a.qpp;
    } else {
        slot = 0;
#pragma unroll
        for (int s = 0; s < BPQ; ++s) qpb[s] = Q + s * nquads;
    }
    bool qok[BPQ];
#pragma unroll
    for (int s = 0; s < BPQ; ++s) qok[s] = (slot < a.NP) && (qpb[s] < a.qpp);

    // ---- fold scales (and Haar normalisations) into the level weights ----
    // The base weights stay unfolded in scalar registers; s0 is applied once
    // per output pixel, fused with the synthesis add: out = s0 * (W0 * x) + Z.
    float* wts = lds + a.wts_off;
    const int wlev = 0;                        // level i (1-based) band u at wlev + ((i-1)*4+u)*KK
    for (int e = tid; e < 4 * a.L * KK; e += nthr) {
        const int i = e / (4 * KK), rem = e - i * 4 * KK, u = rem / KK, tap = rem - u * KK;
        const float sc = ldexpf(a.sl[((size_t)i * a.C + c) * 4 + u], -2 * (i + 1));
        wts[wlev + e] = sc * a.wl[(((size_t)i * a.C + c) * 4 + u) * KK + tap];
    }

    // ---- zero the halo rings that nothing else writes ----
    for (int s2 = 0; s2 < a.NP; ++s2) {
        float* S = lds + s2 * a.slot_stride;
        zero_ring(S + a.a0_off, a.a0_rows, a.a0_S, R, R + a.H, R, R + a.W, tid, nthr);
        if (Lm >= 1)
            for (int u = 0; u < 4; ++u)
                zero_ring(S + a.b_off[1] + u * a.b_bs[1], a.b_rows[1], a.b_S[1], R,
                          R + (a.Hq >> 1), R, R + (a.Wq >> 1), tid, nthr);
    }
    __syncthreads();
    float kappa = 0.f;
    for (int i = Lm; i < a.L; ++i)
        for (int u = 0; u < 4; ++u) kappa += wts[wlev + (i * 4 + u) * KK + (KK >> 1)];

    // ---- persistent backward accumulators ----
    float corr0[KK], corr1[KK], corr2[KK], cdeep[kMaxLm];
#pragma unroll
    for (int i = 0; i < KK; ++i) corr0[i] = corr1[i] = corr2[i] = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxLm; ++i) cdeep[i] = 0.f;
    float sumg = 0.f, tailc = 0.f;
    // deep-level correlation role: subband du, tap (dty, dtx), position subset dsb
    const int drole = tid;
    const bool dactive = BWD && drole < 4 * KK * a.dsub;
    const int du = drole & 3, dtap = (drole >> 2) % KK, dsb = (drole >> 2) / KK;
    const int ddy = dtap / K - R, ddx = dtap % K - R;

    const ST* srcp = reinterpret_cast<const ST*>(a.src);
    const ST* auxp = reinterpret_cast<const ST*>(a.aux);
    ST* dstp = reinterpret_cast<ST*>(a.dst);
    constexpr bool vec = VEC;

    for (int bb = b_begin; bb < b_end; bb += a.NP) {
        const int b = bb + slot;
        const bool pok = (slot < a.NP) && (b < b_end);
        float* S = lds + (slot < a.NP ? slot : 0) * a.slot_stride;
        const size_t poff = ((size_t)b * a.C + c) * plane_sz;

        __syncthreads();  // the previous plane is fully consumed

        // ---------------- phase 1: stage the planes in LDS ----------------
        {
            const int per = vec ? a.H * (a.W >> 2) : a.H * a.W;
            const int wv = vec ? (a.W >> 2) : a.W;
            for (int e = tid; e < a.NP * per; e += nthr) {
                const int s2 = e / per, m = e - s2 * per;
                const int b2 = bb + s2;
                if (b2 >= b_end) continue;
                const int y = m / wv, xq = m - y * wv;
                const ST* pl = srcp + ((size_t)b2 * a.C + c) * plane_sz;
                float* dstl = lds + s2 * a.slot_stride + a.a0_off + (y + R) * a.a0_S + R;
                if constexpr (VEC) {
                    float v[4];
                    load4(pl + (size_t)y * a.W + 4 * xq, v);
#pragma unroll
                    for (int i = 0; i < 4; ++i) dstl[4 * xq + i] = v[i];
                } else {
                    dstl[xq] = to_f32(pl[(size_t)y * a.W + xq]);
                }
            }
            if (a.overlap)
                for (int s2 = 0; s2 < a.NP; ++s2)
                    zero_ring(lds + s2 * a.slot_stride + a.a0_off, a.a0_rows, a.a0_S, R, R + a.H,
                              R, R + a.W, tid, nthr);
        }
        __syncthreads();

        // ---------------- phase 2: base conv, level-1 analysis ----------------
        float acc[BPQ][4][4];
#pragma unroll
        for (int s = 0; s < BPQ; ++s) {
            if (!(pok && qok[s])) continue;
            const int qy = qpb[s] / a.nqx, qx = qpb[s] - (qpb[s] / a.nqx) * a.nqx;
            const int py0 = 8 * qy + 4 * sy, px0 = 8 * qx + 4 * sx;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[s][i][j] = 0.f;
            float w[KK];
            load_w<K, BWD>(a.w0 + (size_t)c * KK, w);
            float xo[4][4];
            if constexpr (BWD) {
                const ST* xp = auxp + poff + opaque(py0 * a.W + px0);
#pragma unroll
                for (int i = 0; i < 4; ++i) ld_row4<VEC>(xp + i * a.W, py0 + i < a.H, px0, a.W, xo[i]);
            }
            const float* win = S + a.a0_off + py0 * a.a0_S + px0;
            stencil<K, 4, 4, 4, BWD>(win, a.a0_S, w, acc[s], xo, corr0);
            // the block itself (window centre) -> level-1 raw bands, sum of g
            float ctr[4][4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float rowv[4];
                lds_row<4, (R % 4 == 0) ? 4 : ((R % 2 == 0) ? 2 : 1)>(win + (i + R) * a.a0_S + R, rowv);
#pragma unroll
                for (int j = 0; j < 4; ++j) ctr[i][j] = rowv[j];
            }
            if constexpr (BWD) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) sumg += ctr[i][j];
            }
            if (Lm >= 1) {
                float* B1 = S + a.b_off[1];
                const int S1 = a.b_S[1], bs1 = a.b_bs[1];
#pragma unroll
                for (int jy = 0; jy < 2; ++jy)
#pragma unroll
                    for (int jx = 0; jx < 2; ++jx) {
                        const float p0 = ctr[2 * jy][2 * jx], p1 = ctr[2 * jy][2 * jx + 1];
                        const float p2 = ctr[2 * jy + 1][2 * jx], p3 = ctr[2 * jy + 1][2 * jx + 1];
                        const float s01 = p0 + p1, d01 = p0 - p1, s23 = p2 + p3, d23 = p2 - p3;
                        const int off = (py0 / 2 + jy + R) * S1 + (px0 / 2 + jx + R);
                        B1[off] = s01 + s23;
                        B1[bs1 + off] = d01 + d23;
                        B1[2 * bs1 + off] = s01 - s23;
                        B1[3 * bs1 + off] = d01 - d23;
                    }
            } else if (a.L > 0 && py0 == 0 && px0 == 0) {
                // every level is a 1x1 grid: tail term enters at pixel (0, 0)
                S[a.tail_off] = ctr[0][0] * kappa;
                if constexpr (BWD) tailc = fmaf(ctr[0][0], xo[0][0], tailc);
            }
        }
        __syncthreads();

        // ---------------- phase 3: analysis of levels 2..Lm ----------------
        for (int i = 2; i <= Lm; ++i) {
            const int hi = a.Hq >> i, wi = a.Wq >> i, Si = a.b_S[i], rows = a.b_rows[i];
            const int per = rows * Si;
            for (int e = tid; e < a.NP * per; e += nthr) {
                const int s2 = e / per, m = e - s2 * per;
                if (bb + s2 >= b_end) continue;
                float* Sl = lds + s2 * a.slot_stride;
                const int ry = m / Si, rx = m - ry * Si;
                const int jy = ry - R, jx = rx - R;
                float v0 = 0.f, v1 = 0.f, v2 = 0.f, v3 = 0.f;
                if (jy >= 0 && jy < hi && jx >= 0 && jx < wi) {
                    const float* LL = Sl + a.b_off[i - 1];
                    const int Sp = a.b_S[i - 1];
                    const int o = (2 * jy + R) * Sp + 2 * jx + R;
                    const float p0 = LL[o], p1 = LL[o + 1], p2 = LL[o + Sp], p3 = LL[o + Sp + 1];
                    const float s01 = p0 + p1, d01 = p0 - p1, s23 = p2 + p3, d23 = p2 - p3;
                    v0 = s01 + s23; v1 = d01 + d23; v2 = s01 - s23; v3 = d01 - d23;
                }
                float* Bi = Sl + a.b_off[i];
                Bi[m] = v0;
                Bi[a.b_bs[i] + m] = v1;
                Bi[2 * a.b_bs[i] + m] = v2;
                Bi[3 * a.b_bs[i] + m] = v3;
            }
            __syncthreads();
        }

        // ---------------- phase 4a: levels 1 and 2, subband per lane ----------------
        float y1[BPQ][4][4], y2[BPQ][2][2];
#pragma unroll
        for (int s = 0; s < BPQ; ++s) {
            if (!(pok && qok[s]) || Lm < 1) continue;
            const int qy = qpb[s] / a.nqx, qx = qpb[s] - (qpb[s] / a.nqx) * a.nqx;
            float rx1[4][4], ll1[4][4];
            if constexpr (BWD) {
                // x over the quad's 8x8 block -> band t and LL at level 1
                const ST* xp = auxp + poff + opaque(8 * qy * a.W + 8 * qx);
#pragma unroll
                for (int jy = 0; jy < 4; ++jy) {
                    float r0[2][4], r1[2][4];
                    const int y0 = 8 * qy + 2 * jy;
                    const ST* p0r = xp + (2 * jy) * a.W;
                    ld_row4<VEC>(p0r, y0 < a.H, 8 * qx, a.W, r0[0]);
                    ld_row4<VEC>(p0r + 4, y0 < a.H, 8 * qx + 4, a.W, r0[1]);
                    ld_row4<VEC>(p0r + a.W, y0 + 1 < a.H, 8 * qx, a.W, r1[0]);
                    ld_row4<VEC>(p0r + a.W + 4, y0 + 1 < a.H, 8 * qx + 4, a.W, r1[1]);
#pragma unroll
                    for (int jx = 0; jx < 4; ++jx) {
                        const float p0 = r0[jx >> 1][(2 * jx) & 3], p1 = r0[jx >> 1][(2 * jx + 1) & 3];
                        const float p2 = r1[jx >> 1][(2 * jx) & 3], p3 = r1[jx >> 1][(2 * jx + 1) & 3];
                        ll1[jy][jx] = (p0 + p1) + (p2 + p3);
                        rx1[jy][jx] = fmaf(sgy, fmaf(sgx, p3, p2), fmaf(sgx, p1, p0));
                    }
                    // two input rows live at a time
#pragma unroll
                    for (int jx = 0; jx < 4; ++jx) asm volatile("" : "+v"(ll1[jy][jx]), "+v"(rx1[jy][jx]));
                    asm volatile("" ::: "memory");
                }
            }
            float ll2[2][2], rx2[2][2];
            if constexpr (BWD) {
#pragma unroll
                for (int jy = 0; jy < 2; ++jy)
#pragma unroll
                    for (int jx = 0; jx < 2; ++jx) {
                        const float p0 = ll1[2 * jy][2 * jx], p1 = ll1[2 * jy][2 * jx + 1];
                        const float p2 = ll1[2 * jy + 1][2 * jx], p3 = ll1[2 * jy + 1][2 * jx + 1];
                        ll2[jy][jx] = (p0 + p1) + (p2 + p3);
                        rx2[jy][jx] = fmaf(sgy, fmaf(sgx, p3, p2), fmaf(sgx, p1, p0));
                    }
            }
            {
                float w[KK];
                load_w<K, BWD>(wts + wlev + t * KK, w);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) y1[s][i][j] = 0.f;
                const float* win = S + a.b_off[1] + t * a.b_bs[1] + (4 * qy) * a.b_S[1] + 4 * qx;
                stencil<K, 4, 4, 4, BWD>(win, a.b_S[1], w, y1[s], rx1, corr1);
            }
            if (Lm >= 2) {
                float w[KK];
                load_w<K, BWD>(wts + wlev + (4 + t) * KK, w);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) y2[s][i][j] = 0.f;
                const float* win = S + a.b_off[2] + t * a.b_bs[2] + (2 * qy) * a.b_S[2] + 2 * qx;
                stencil<K, 2, 2, 2, BWD>(win, a.b_S[2], w, y2[s], rx2, corr2);
                if constexpr (BWD) {
                    if (Lm >= 3 && t == 0) {
                        float* xl2 = S + a.xl2_off;
                        const int w2 = a.Wq >> 2;
#pragma unroll
                        for (int jy = 0; jy < 2; ++jy)
#pragma unroll
                            for (int jx = 0; jx < 2; ++jx) xl2[(2 * qy + jy) * w2 + 2 * qx + jx] = ll2[jy][jx];
                    }
                }
            }
            // tail term: rho = raw LL of the convolved tensor at level Lm, position (0,0)
            if (a.L > Lm && qpb[s] == 0 && t == 0) {
                const float rho = S[a.b_off[Lm] + R * a.b_S[Lm] + R];
                S[a.tail_off] = rho * kappa;
                if constexpr (BWD) {
                    if (Lm == 1) tailc = fmaf(rho, ll1[0][0], tailc);
                    if (Lm == 2) tailc = fmaf(rho, ll2[0][0], tailc);
                }
            }
        }

        // ---------------- phase 4b: x bands of levels >= 3 (backward) ----------------
        if constexpr (BWD) {
            if (Lm >= 3) {
                __syncthreads();
                for (int i = 3; i <= Lm; ++i) {
                    const int hi = a.Hq >> i, wi = a.Wq >> i, wp = a.Wq >> (i - 1);
                    const int per = hi * wi;
                    for (int e = tid; e < a.NP * per; e += nthr) {
                        const int s2 = e / per, m = e - s2 * per;
                        if (bb + s2 >= b_end) continue;
                        float* Sl = lds + s2 * a.slot_stride;
                        const float* LL = (i == 3) ? (Sl + a.xl2_off) : (Sl + a.xb_off[i - 1]);
                        const int jy = m / wi, jx = m - jy * wi;
                        const int o = 2 * jy * wp + 2 * jx;
                        const float p0 = LL[o], p1 = LL[o + 1], p2 = LL[o + wp], p3 = LL[o + wp + 1];
                        const float s01 = p0 + p1, d01 = p0 - p1, s23 = p2 + p3, d23 = p2 - p3;
                        float* XB = Sl + a.xb_off[i];
                        XB[m] = s01 + s23;
                        XB[per + m] = d01 + d23;
                        XB[2 * per + m] = s01 - s23;
                        XB[3 * per + m] = d01 - d23;
                    }
                    __syncthreads();
                }
                if (a.L > Lm && pok && qok[0] && qpb[0] == 0 && t == 0) {
                    const float rho = S[a.b_off[Lm] + R * a.b_S[Lm] + R];
                    tailc = fmaf(rho, S[a.xb_off[Lm]], tailc);
                }
            }
        }

        // ---------------- phase 4c: levels >= 3, flat ----------------
        for (int i = 3; i <= Lm; ++i) {
            const int hi = a.Hq >> i, wi = a.Wq >> i, Si = a.b_S[i], bs = a.b_bs[i];
            const int per = 4 * hi * wi;
            for (int e = tid; e < a.NP * per; e += nthr) {
                const int s2 = e / per, m = e - s2 * per;
                if (bb + s2 >= b_end) continue;
                float* Sl = lds + s2 * a.slot_stride;
                const int u = m & 3, j = m >> 2;
                const int jy = j / wi, jx = j - jy * wi;
                float w[KK];
                load_w<K, BWD>(wts + wlev + ((i - 1) * 4 + u) * KK, w);
                const float* win = Sl + a.b_off[i] + u * bs + jy * Si + jx;
                float accv = 0.f;
#pragma unroll
                for (int ky = 0; ky < K; ++ky)
#pragma unroll
                    for (int kx = 0; kx < K; ++kx) accv = fmaf(w[ky * K + kx], win[ky * Si + kx], accv);
                Sl[a.yd_off[i] + u * hi * wi + j] = accv;
            }
            if constexpr (BWD) {
                // output-stationary correlation: C_i^du[d] over this role's positions
                if (dactive) {
                    float cv = 0.f;
                    for (int s2 = 0; s2 < a.NP; ++s2) {
                        if (bb + s2 >= b_end) break;
                        const float* Sl = lds + s2 * a.slot_stride;
                        const float* XB = Sl + a.xb_off[i] + du * hi * wi;
                        const float* G = Sl + a.b_off[i] + du * bs;
                        for (int m = dsb; m < hi * wi; m += a.dsub) {
                            const int my = m / wi, mx = m - my * wi;
                            cv = fmaf(XB[m], G[(my - ddy + R) * Si + (mx - ddx + R)], cv);
                        }
                    }
#pragma unroll
                    for (int q = 0; q < kMaxLm; ++q)
                        if (q == i - 3) cdeep[q] += cv;
                }
            }
        }
        __syncthreads();

        // ---------------- phase 4d: levels 1, 2 results in place ----------------
#pragma unroll
        for (int s = 0; s < BPQ; ++s) {
            if (!(pok && qok[s]) || Lm < 1) continue;
            const int qy = qpb[s] / a.nqx, qx = qpb[s] - (qpb[s] / a.nqx) * a.nqx;
            float* B1 = S + a.b_off[1] + t * a.b_bs[1];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) B1[(4 * qy + i + R) * a.b_S[1] + 4 * qx + j + R] = y1[s][i][j];
            if (Lm >= 2) {
                float* B2 = S + a.b_off[2] + t * a.b_bs[2];
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) B2[(2 * qy + i + R) * a.b_S[2] + 2 * qx + j + R] = y2[s][i][j];
            }
        }
        __syncthreads();

        // ---------------- phase 5: synthesis of levels Lm..2 ----------------
        for (int i = Lm; i >= 2; --i) {
            const int hi = a.Hq >> i, wi = a.Wq >> i;
            const int per = hi * wi, wz = a.Wq >> (i - 1);
            for (int e = tid; e < a.NP * per; e += nthr) {
                const int s2 = e / per, j = e - s2 * per;
                if (bb + s2 >= b_end) continue;
                float* Sl = lds + s2 * a.slot_stride;
                const int jy = j / wi, jx = j - jy * wi;
                float T0, T1, T2, T3;
                if (i == 2) {
                    const float* B2 = Sl + a.b_off[2];
                    const int o = (jy + R) * a.b_S[2] + jx + R, bs = a.b_bs[2];
                    T0 = B2[o]; T1 = B2[bs + o]; T2 = B2[2 * bs + o]; T3 = B2[3 * bs + o];
                } else {
                    const float* Y = Sl + a.yd_off[i];
                    T0 = Y[j]; T1 = Y[per + j]; T2 = Y[2 * per + j]; T3 = Y[3 * per + j];
                }
                if (i < Lm) T0 += Sl[a.z_off[i + 1] + j];
                if (i == Lm && j == 0 && a.L > Lm) T0 += Sl[a.tail_off];
                const float s01 = T0 + T1, d01 = T0 - T1, s23 = T2 + T3, d23 = T2 - T3;
                float* Z = Sl + a.z_off[i] + (2 * jy) * wz + 2 * jx;
                Z[0] = s01 + s23;
                Z[1] = d01 + d23;
                Z[wz] = s01 - s23;
                Z[wz + 1] = d01 - d23;
            }
            __syncthreads();
        }

        // ---------------- phase 6: level-1 synthesis fused with the store ----------------
#pragma unroll
        for (int s = 0; s < BPQ; ++s) {
            if (!(pok && qok[s])) continue;
            const int qy = qpb[s] / a.nqx, qx = qpb[s] - (qpb[s] / a.nqx) * a.nqx;
            const int py0 = 8 * qy + 4 * sy, px0 = 8 * qx + 4 * sx;
            const float bias = BWD ? 0.f : a.b0[c];
            float z[4][4];
            if (Lm >= 1) {
                const float* B1 = S + a.b_off[1];
                const int S1 = a.b_S[1], bs1 = a.b_bs[1], w1 = a.Wq >> 1;
#pragma unroll
                for (int dy = 0; dy < 2; ++dy)
#pragma unroll
                    for (int dx = 0; dx < 2; ++dx) {
                        const int jy = py0 / 2 + dy, jx = px0 / 2 + dx;
                        const int o = (jy + R) * S1 + jx + R;
                        float T0 = B1[o] + bias;
                        const float T1 = B1[bs1 + o], T2 = B1[2 * bs1 + o], T3 = B1[3 * bs1 + o];
                        if (Lm >= 2) T0 += S[a.z_off[2] + jy * w1 + jx];
                        if (Lm == 1 && a.L > 1 && jy == 0 && jx == 0) T0 += S[a.tail_off];
                        const float s01 = T0 + T1, d01 = T0 - T1, s23 = T2 + T3, d23 = T2 - T3;
                        z[2 * dy][2 * dx] = s01 + s23;
                        z[2 * dy][2 * dx + 1] = d01 + d23;
                        z[2 * dy + 1][2 * dx] = s01 - s23;
                        z[2 * dy + 1][2 * dx + 1] = d01 - d23;
                    }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) z[i][j] = bias;
                if (a.L > 0 && py0 == 0 && px0 == 0) z[0][0] += S[a.tail_off];
            }
            const float s0c = a.s0[c];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[s][i][j] = fmaf(s0c, acc[s][i][j], z[i][j]);
            ST* op = dstp + poff + opaque(py0 * a.W + px0);
            if constexpr (VEC) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (py0 + i < a.H && px0 < a.W) store4(op + i * a.W, acc[s][i]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (py0 + i < a.H && px0 + j < a.W) from_f32(op[i * a.W + j], acc[s][i][j]);
            }
        }
    }

    if constexpr (BWD) {
        // ---------------- reduction of the correlation accumulators ----------------
        __syncthreads();
        float* red = lds + a.red_off;
        const int nw = nthr >> 6, wave = tid >> 6, lane = tid & 63;
        // per-wave record: [C_0 (KK)][C_1 u=0..3 (KK each)][C_2 u=0..3][sumg][tail]
        const int WR = KK * 9 + 2;
#pragma unroll
        for (int q = 0; q < KK; ++q) {
            const float v0 = wave_sum(corr0[q], 1);
            const float v1 = wave_sum(corr1[q], 4);
            const float v2 = wave_sum(corr2[q], 4);
            // un-rotate: accumulator q holds tap KK-1-q
            if (lane == 0) red[wave * WR + (KK - 1 - q)] = v0;
            if (lane < 4) {
                red[wave * WR + KK + lane * KK + (KK - 1 - q)] = v1;
                red[wave * WR + 5 * KK + lane * KK + (KK - 1 - q)] = v2;
            }
        }
        {
            const float vs = wave_sum(sumg, 1), vt = wave_sum(tailc, 1);
            if (lane == 0) {
                red[wave * WR + 9 * KK] = vs;
                red[wave * WR + 9 * KK + 1] = vt;
            }
        }
        float* dred = red + nw * WR;   // deep: [q][role]
        if (dactive)
            for (int q = 0; q + 3 <= Lm; ++q) dred[q * 4 * KK * a.dsub + drole] = cdeep[q];
        __syncthreads();
        float* rec = a.partials + ((size_t)chunk * a.C + c) * a.P;
        for (int e = tid; e < a.P; e += nthr) {
            float v = 0.f;
            if (e < KK) {
                for (int wv = 0; wv < nw; ++wv) v += red[wv * WR + e];
            } else if (e < KK + 4 * KK * Lm) {
                const int lvl = (e - KK) / (4 * KK) + 1;
                const int rem = (e - KK) - (lvl - 1) * 4 * KK;
                if (lvl <= 2) {
                    const int base = (lvl == 1) ? KK : 5 * KK;
                    for (int wv = 0; wv < nw; ++wv) v += red[wv * WR + base + rem];
                } else {
                    const int u = rem / KK, tap = rem - u * KK;
                    for (int sb = 0; sb < a.dsub; ++sb)
                        v += dred[(lvl - 3) * 4 * KK * a.dsub + (sb * KK + tap) * 4 + u];
                }
            } else if (e == a.P - 2) {
                for (int wv = 0; wv < nw; ++wv) v += red[wv * WR + 9 * KK];
            } else {
                for (int wv = 0; wv < nw; ++wv) v += red[wv * WR + 9 * KK + 1];
            }
            rec[e] = v;
        }
    }
}

template <int K, typename ST, bool BWD, int BPQ, bool VEC>
hipError_t launch_t(const FusedArgs& a, int nthr, size_t lds, int grid, hipStream_t st) {
    auto kern = wtc_fused_kernel<K, ST, BWD, BPQ, VEC>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(nthr), lds, st, a);
    return hipGetLastError();
}

template <int K, typename ST, bool BWD>
hipError_t launch_b(const FusedArgs& a, int bpq, int nthr, size_t lds, int grid, hipStream_t st) {
    if (a.vec) {
        if (bpq == 1) return launch_t<K, ST, BWD, 1, true>(a, nthr, lds, grid, st);
        return launch_t<K, ST, BWD, 2, true>(a, nthr, lds, grid, st);
    }
    if (bpq == 1) return launch_t<K, ST, BWD, 1, false>(a, nthr, lds, grid, st);
    return launch_t<K, ST, BWD, 2, false>(a, nthr, lds, grid, st);
}

template <int K, typename ST>
hipError_t launch_d(const FusedArgs& a, int bwd, int bpq, int nthr, size_t lds, int grid, hipStream_t st) {
    return bwd ? launch_b<K, ST, true>(a, bpq, nthr, lds, grid, st)
               : launch_b<K, ST, false>(a, bpq, nthr, lds, grid, st);
}

template <int K>
hipError_t launch_k(const FusedArgs& a, int dtype, int bwd, int bpq, int nthr, size_t lds, int grid,
                    hipStream_t st) {
    return dtype == WTC_BF16 ? launch_d<K, bf16_t>(a, bwd, bpq, nthr, lds, grid, st)
                             : launch_d<K, float>(a, bwd, bpq, nthr, lds, grid, st);
}

}  // namespace fused_detail
}  // namespace wtc
