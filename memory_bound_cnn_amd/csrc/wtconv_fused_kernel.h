// Fused WTConv forward / backward for gfx950 (MI355X): kernel template.
// Instantiated once per kernel size in wtconv_fused_k<k>.hip.
//
// Method: "Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware
// Reformulation" (arXiv 2608.10805, Abstract) names three reformulations of
// the WTConv operator; all three are used here, re-derived for CDNA4:
//   (1) the Haar analysis butterfly is recomputed on chip (LDS / registers)
//       instead of storing subbands in HBM;
//   (2) the multi-level synthesis is one pass whose signs are indexed by the
//       output-coordinate bits: each lane sums, for its own 4x4 output block,
//       one subband quadruple per level (with signs from the bits of the
//       block's coordinates) and one 2x2 butterfly per level-1 position, fused
//       with the output store;
//   (3) the per-channel scales -- and the 2^-i Haar normalisations of analysis
//       and synthesis -- are folded into the convolution weights,
//       W'_i = 4^-i * s_i * W_i and W'_0 = s0 * W0, so every butterfly is a raw
//       +-1 sum.
// HBM traffic is one read of the convolved tensor, one write of the result
// and, in the backward pass, one read of x.
//
// Work decomposition (one workgroup = a contiguous range of planes in
// channel-major order, at most two channel segments):
//   * each plane is staged in LDS with a zero halo of k/2 and zero-extended to
//     Hq x Wq (multiples of max(8, 2^Lm)); zero extension is exactly the
//     "pad to even before each analysis, crop after each synthesis" rule;
//   * 4 lanes ("a quad") own an 8x8 pixel block.  At level 0 each lane owns a
//     4x4 sub-block; at levels 1 and 2 lane t convolves subband t over the
//     whole quad block (4x4 resp. 2x2 positions), so one lane needs one set
//     of k*k weights and one set of correlation accumulators per level;
//   * the analysis of levels 1..3 happens in registers while the base conv
//     runs (a lane's 4x4 block is one level-2 position, a quad's 8x8 block one
//     level-3 position); deeper levels (large planes only) are flat loops;
//   * levels >= 3 (at most one position per quad) are convolved in flat
//     loops; their weight-gradient correlations are output-stationary (one
//     thread per subband x tap x position subset), one register each;
//   * the next planes are prefetched into registers while the current one is
//     computed.
// The backward pass is the same pipeline applied to g with 180-degree-rotated
// weights (the adjoint: the orthonormal Haar matrix is symmetric, so analysis
// and synthesis are each other's transpose), plus the correlations
//   C_0[d] = sum g[p] x[p+d],   C_i^u[d] = sum R_i^u(g)[j] R_i^u(x)[j+d]
// accumulated in registers across the workgroup's planes and reduced once.
#pragma once
#include <hip/hip_runtime.h>

#include <type_traits>

#include "wtc_internal.h"
#include "wtc_numeric.h"

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
__device__ __forceinline__ void from_f32(bf16_t& d, float v) { d.bits = bf16_rne(v); }

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
// Two consecutive pixels (the caller guarantees 2-pixel alignment).
__device__ __forceinline__ void store2(float* p, float v0, float v1) {
    *reinterpret_cast<float2*>(p) = make_float2(v0, v1);
}
__device__ __forceinline__ void store2(bf16_t* p, float v0, float v1) {
    *reinterpret_cast<uint32_t*>(p) = bf16x2_rne(v0, v1);
}
__device__ __forceinline__ void store4(float* p, const float (&v)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store4(bf16_t* p, const float (&v)[4]) {
    uint2 q;
    q.x = bf16x2_rne(v[0], v[1]);
    q.y = bf16x2_rne(v[2], v[3]);
    *reinterpret_cast<uint2*>(p) = q;
}

// ---------------------------------------------------------------------------
// LDS helpers
// ---------------------------------------------------------------------------
// Native vector types: their loads keep the float type-alias tag, which lets
// the compiler see that they cannot overlap a pending LDS DMA into another
// region (it would otherwise wait for the DMA before each of them).
typedef float lds_f4 __attribute__((ext_vector_type(4)));
typedef float lds_f2 __attribute__((ext_vector_type(2)));

// Read WW consecutive floats; AL = guaranteed alignment of p in floats (4, 2, 1).
template <int WW, int AL>
__device__ __forceinline__ void lds_row(const float* p, float (&row)[WW]) {
    if constexpr (AL == 4) {
#pragma unroll
        for (int q = 0; q + 4 <= WW; q += 4) {
            const lds_f4 v = *reinterpret_cast<const lds_f4*>(p + q);
            row[q] = v.x; row[q + 1] = v.y; row[q + 2] = v.z; row[q + 3] = v.w;
        }
        constexpr int done = (WW / 4) * 4;
        if constexpr (WW - done >= 2) {
            const lds_f2 v = *reinterpret_cast<const lds_f2*>(p + done);
            row[done] = v.x; row[done + 1] = v.y;
        }
        if constexpr ((WW - done) % 2 == 1) row[WW - 1] = p[WW - 1];
    } else if constexpr (AL == 2) {
#pragma unroll
        for (int q = 0; q + 2 <= WW; q += 2) {
            const lds_f2 v = *reinterpret_cast<const lds_f2*>(p + q);
            row[q] = v.x; row[q + 1] = v.y;
        }
        if constexpr (WW % 2 == 1) row[WW - 1] = p[WW - 1];
    } else {
#pragma unroll
        for (int q = 0; q < WW; ++q) row[q] = p[q];
    }
}

// Zero every element of a rows x S array outside the interior [r0, r0+h) x
// [c0, c0+w) (c0 + w <= S).  The ring is a prefix, a suffix and one gap of
// S - w elements between consecutive interior rows: no divisions needed.
__device__ void zero_ring(float* base, int rows, int S, int r0, int h, int c0, int w, int tid,
                          int nthr) {
    const int pre = r0 * S + c0;
    const int suf0 = (r0 + h - 1) * S + c0 + w;
    const int suf = rows * S - suf0;
    for (int e = tid; e < pre; e += nthr) base[e] = 0.f;
    for (int e = tid; e < suf; e += nthr) base[suf0 + e] = 0.f;
    const int gap = S - w;
    for (int y = tid; y < h - 1; y += nthr) {
        float* g = base + (r0 + y) * S + c0 + w;
        for (int j = 0; j < gap; ++j) g[j] = 0.f;
    }
}

// Zero the rings of `na` arrays in every plane slot (array j of a slot at
// off + j * astride; rows x S floats, interior [R, R+h) x [R, R+w)), one work
// item per array row: a halo row is cleared whole with 16-byte stores, an
// interior row only left and right of the interior.  Rows start 16-byte
// aligned (slot, offsets, strides and S are multiples of 4 floats).
template <int R, class G>
__device__ __forceinline__ void zero_rings(float* lds, const G& g, int off, int astride, int na, int rows, int S, int h, int w,
                           int tid, int nthr);

// (FastDiv, make_div, fdiv: integer division by a float reciprocal, wtc_numeric.h)

template <int R, class G>
__device__ __forceinline__ void zero_rings(float* lds, const G& g, int off, int astride, int na, int rows, int S, int h, int w,
                           int tid, int nthr) {
    const int per_slot = na * rows;
    const FastDiv dps = make_div(per_slot), drows = make_div(rows);
    for (int e = tid; e < g.NP() * per_slot; e += nthr) {
        const int s2 = fdiv(e, dps), rem = e - s2 * per_slot;
        const int j = fdiv(rem, drows), r = rem - j * rows;
        float* row = lds + s2 * g.slot() + off + j * astride + r * S;
        if (r < R || r >= R + h) {
            for (int c = 0; c < S; c += 4) *reinterpret_cast<lds_f4*>(row + c) = lds_f4{0.f, 0.f, 0.f, 0.f};
        } else {
#pragma unroll
            for (int c = 0; c < R; ++c) row[c] = 0.f;
            for (int c = R + w; c < S; ++c) row[c] = 0.f;
        }
    }
}

// ---------------------------------------------------------------------------
// Register-blocked stencil: OH x OW outputs from an (OH+K-1) x (OW+K-1) LDS
// window, one window row live at a time.
//   acc[oy][ox]   += w[ky][kx] * win[oy+ky][ox+kx]
//   corr[ky][kx]  += xv[oy][ox] * win[oy+ky][ox+kx]     (CORR only)
// ---------------------------------------------------------------------------
// CTR: also hand back the window's centre, ctr[oy][ox] = win[oy+K/2][ox+K/2]
// (the block itself), taken from the rows as they pass instead of read again.
template <int K, int OH, int OW, int AL, bool CORR, bool CTR = false>
__device__ __forceinline__ void stencil(const float* win, int S, const float (&w)[K * K],
                                        float (&acc)[OH][OW], const float (&xv)[OH][OW],
                                        float (&corr)[K * K], float (*ctr)[OW] = nullptr) {
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
        if constexpr (CTR) {
            if (wy >= K / 2 && wy < K / 2 + OH) {
#pragma unroll
                for (int ox = 0; ox < OW; ++ox) ctr[wy - K / 2][ox] = row[K / 2 + ox];
            }
        }
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
// Same from a 16-byte aligned set padded to a multiple of 4 floats: 16-byte
// LDS reads from one base address (immediate offsets).
template <int K, bool ROT>
__device__ __forceinline__ void load_w4(const float* p, float (&w)[K * K]) {
    constexpr int KK = K * K, KKP = (KK + 3) & ~3;
    float v[KKP];
#pragma unroll
    for (int q = 0; q < KKP; q += 4) {
        const lds_f4 f = *reinterpret_cast<const lds_f4*>(p + q);
        v[q] = f.x; v[q + 1] = f.y; v[q + 2] = f.z; v[q + 3] = f.w;
    }
#pragma unroll
    for (int t = 0; t < KK; ++t) w[t] = v[ROT ? (KK - 1 - t) : t];
}

// Four pixels of one row at pixel stride ps: consecutive (load4 / store4) in
// NCHW planes, ps = C elements apart in channels-last tensors.
template <bool NHWC, typename ST>
__device__ __forceinline__ void gload4(const ST* p, size_t ps, float (&v)[4]) {
    if constexpr (NHWC) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = to_f32(p[i * ps]);
    } else {
        load4(p, v);
    }
}
template <bool NHWC, typename ST>
__device__ __forceinline__ void gstore4(ST* p, size_t ps, const float (&v)[4]) {
    if constexpr (NHWC) {
#pragma unroll
        for (int i = 0; i < 4; ++i) from_f32(p[i * ps], v[i]);
    } else {
        store4(p, v);
    }
}

// Raw buffer resource over `bytes` bytes at `base`: the hardware range check
// drops stores at offsets past the range, so out-of-plane lanes need no branch.
using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr uint32_t kRsrcWord3 = 0x00020000;   // raw 32-bit data format
constexpr int kOutOfRange = 0x7FFFFFF0;       // past every range used here (< 2^31 bytes)
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}
// four pixels at byte offset `off` of the resource: one 16-byte store of
// floats, or one 8-byte store of bfloat16 (rounded to nearest even)
__device__ __forceinline__ void bstore4(rsrc_t r, int off, const float (&v)[4], float*) {
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    const u4 d = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
    __builtin_amdgcn_raw_buffer_store_b128(d, r, off, 0, 0);
}
__device__ __forceinline__ void bstore4(rsrc_t r, int off, const float (&v)[4], bf16_t*) {
    typedef unsigned int u2 __attribute__((ext_vector_type(2)));
    const u2 d = {bf16x2_rne(v[0], v[1]), bf16x2_rne(v[2], v[3])};
    __builtin_amdgcn_raw_buffer_store_b64(d, r, off, 0, 0);
}

// Pixel (y, x) of a plane, zero outside [0,H) x [0,W).
template <typename ST>
__device__ __forceinline__ float ld_px(const ST* plane, int y, int x, int H, int W) {
    return (y < H && x < W) ? to_f32(plane[y * W + x]) : 0.f;
}

// Four pixels starting at `rowp` (= image pixel (y, x), x % 4 == 0); zero where
// the row is outside the image (row_ok false) or a column is >= W.
template <bool VEC, bool NHWC = false, typename ST>
__device__ __forceinline__ void ld_row4(const ST* rowp, bool row_ok, int x, int W, float (&v)[4], size_t ps = 1) {
    if constexpr (VEC) {
        if (row_ok && x < W) {
            gload4<NHWC>(rowp, ps, v);
        } else {
            v[0] = v[1] = v[2] = v[3] = 0.f;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (row_ok && x + i < W) ? to_f32(rowp[NHWC ? i * ps : i]) : 0.f;
    }
}

// Opaque copy of a per-thread offset: keeps the compiler from hoisting the
// addresses derived from it out of the plane loop as 64-bit pointers.
__device__ __forceinline__ int opaque(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

// Value of v in lane l - N of the same 16-lane row (0 for the row's first N
// lanes): a DPP row shift, plain VALU with no LDS round trip.
template <int N>
__device__ __forceinline__ float row_shr(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x110 | N, 0xF, 0xF, true));
}
// Lanes 12..15 of every 16-lane row: the sum of v over the row's four lanes
// with the same lane index mod 4 (lane 12 + r holds residue r).
__device__ __forceinline__ float row_sum_by_residue(float v) {
    v += row_shr<4>(v);
    return v + row_shr<8>(v);
}
// Lane 15 of every 16-lane row: the sum of v over the row.
__device__ __forceinline__ float row_sum(float v) {
    v = row_sum_by_residue(v);
    v += row_shr<1>(v);
    return v + row_shr<2>(v);
}

// ---------------------------------------------------------------------------
// Plane geometry.  RtGeom reads it from the kernel arguments (any plane size);
// CtGeom fixes it at compile time, so LDS strides and offsets become
// immediates and the per-level loops unroll.  Both describe the same layout
// (make_layout), so one kernel body serves both.  kDeep = deep levels (>= 3)
// whose backward correlation accumulators a thread holds across planes: the
// runtime-geometry kernel is compiled for Lm <= 3 (one set) and for any Lm,
// so that the common shallow plans keep 20 registers free.
// ---------------------------------------------------------------------------
template <bool DLM, int LMX, bool NHWC = false>
struct RtGeom {
    static constexpr bool kDL = DLM;     // planes by DMA (layout mode 1) or staged through registers
    static constexpr bool kNHWC = NHWC;  // activations channels-last: pixel stride C
    static constexpr bool kXSeg = false;
    static constexpr bool kFixed = false;
    static constexpr bool kWhole = false;
    static constexpr int kPH = 0, kPW = 0;
    static constexpr bool kNoLevels = false;
    static constexpr int kDeep = LMX > 3 ? LMX - 2 : 1;
    static constexpr bool kSub = true;   // may run the LL problem of a peeled plane
    static constexpr int kMaxThreads = 512;
    static constexpr int kHq = 0, kWq = 0, kNP = 0, kNthr = 0;   // known at run time only
    const FusedArgs& a;
    __device__ RtGeom(const FusedArgs& args) : a(args) {}
    __device__ int Lm() const { return a.Lm; }
    __device__ int early() const { return a.lay.early_lv; }
    __device__ int Hq() const { return a.Hq; }
    __device__ int Wq() const { return a.Wq; }
    __device__ int NP() const { return a.NP; }
    __device__ int qpp() const { return a.qpp; }
    __device__ int nqx() const { return a.nqx; }
    __device__ int nthr() const { return blockDim.x; }
    __device__ bool ovl() const { return a.lay.overlap != 0; }
    __device__ int bovl() const { return a.lay.bovl; }
    __device__ int slot() const { return a.lay.slot; }
    __device__ int a0_off() const { return a.lay.a0_off; }
    __device__ int a0_S() const { return a.lay.a0_S; }
    __device__ int a0_rows() const { return a.lay.a0_rows; }
    __device__ int b_off(int i) const { return a.lay.b_off[i]; }
    __device__ int b_S(int i) const { return a.lay.b_S[i]; }
    __device__ int b_bs(int i) const { return a.lay.b_bs[i]; }
    __device__ int b_rows(int i) const { return a.lay.b_rows[i]; }
    __device__ int yd_off(int i) const { return a.lay.yd_off[i]; }
    __device__ int xb_off(int i) const { return a.lay.xb_off[i]; }
    __device__ int tail_off() const { return a.lay.tail_off; }
    __device__ int xp_off() const { return a.lay.xp_off; }
    __device__ int xp_S() const { return a.lay.xp_S; }
    __device__ int st_off() const { return a.lay.st_off; }
    __device__ int wts_off() const { return a.wts_off; }
    __device__ int red_off() const { return a.red_off; }
    __device__ int dsub() const { return a.dsub; }
    __device__ int P() const { return a.P; }
};

template <int K, int HQ, int WQ, int LM, int EARLY, int NPV, int NTHR, bool BWDL, int BOVL, int MODE, int ESZ,
          bool NHWC = false, bool WHOLE = false, int PH = 0, int PW = 0>
struct CtGeom {
    static constexpr Layout lay = make_layout(K, HQ, WQ, LM, EARLY, BWDL, BOVL, MODE, ESZ);
    static constexpr bool kDL = MODE == 1;
    static constexpr bool kNHWC = NHWC;
    // direct loads may run ahead into the next channel segment: the backward
    // reduction scratch (from offset 0) ends before the first copy target
    static constexpr bool kXSeg =
        MODE == 1 && (!BWDL || red_len(NTHR, K, LM, NTHR / (4 * K) > 0 ? NTHR / (4 * K) : 1) <= lay.a0_off);
    static constexpr bool kFixed = true;
    static constexpr bool kWhole = WHOLE;   // the plane is exactly HQ x WQ
    static constexpr int kPH = WHOLE ? HQ : PH, kPW = WHOLE ? WQ : PW;   // plane size, if fixed (else 0)
    static constexpr bool kNoLevels = LM == 0;
    static constexpr int kDeep = kMaxLm - 2;
    // the LL problem of a peeled plane is over 64 pixels wide (its parent did
    // not fit the pipeline): the smaller classes never check for it
    static constexpr bool kSub = HQ > 64;
    static constexpr int kMaxThreads = NTHR > 512 ? NTHR : 512;
    static constexpr int kHq = HQ, kWq = WQ, kNP = NPV, kNthr = NTHR;
    const FusedArgs& a;
    __device__ CtGeom(const FusedArgs& args) : a(args) {}
    __device__ static constexpr int Lm() { return LM; }
    __device__ static constexpr int early() { return lay.early_lv; }
    __device__ static constexpr int Hq() { return HQ; }
    __device__ static constexpr int Wq() { return WQ; }
    __device__ static constexpr int NP() { return NPV; }
    __device__ static constexpr int qpp() { return (HQ / 8) * (WQ / 8); }
    __device__ static constexpr int nqx() { return WQ / 8; }
    __device__ static constexpr int nthr() { return NTHR; }
    __device__ static constexpr bool ovl() { return lay.overlap != 0; }
    __device__ static constexpr int bovl() { return lay.bovl; }
    __device__ static constexpr int slot() { return lay.slot; }
    __device__ static constexpr int a0_off() { return lay.a0_off; }
    __device__ static constexpr int a0_S() { return lay.a0_S; }
    __device__ static constexpr int a0_rows() { return lay.a0_rows; }
    __device__ static constexpr int b_off(int i) { return lay.b_off[i]; }
    __device__ static constexpr int b_S(int i) { return lay.b_S[i]; }
    __device__ static constexpr int b_bs(int i) { return lay.b_bs[i]; }
    __device__ static constexpr int b_rows(int i) { return lay.b_rows[i]; }
    __device__ static constexpr int yd_off(int i) { return lay.yd_off[i]; }
    __device__ static constexpr int xb_off(int i) { return lay.xb_off[i]; }
    __device__ static constexpr int tail_off() { return lay.tail_off; }
    __device__ static constexpr int xp_off() { return lay.xp_off; }
    __device__ static constexpr int xp_S() { return lay.xp_S; }
    __device__ static constexpr int st_off() { return lay.st_off; }
    __device__ static constexpr int wts_off() { return NPV * lay.slot; }
    __device__ static constexpr int red_off() { return 0; }
    __device__ static constexpr int dsub() { return NTHR / (4 * K) > 0 ? NTHR / (4 * K) : 1; }
    __device__ static constexpr int P() { return partial_len(K, LM); }
};

// Workgroup barrier for LDS communication only: waits for this wave's LDS
// operations (lgkmcnt) and meets the other waves at s_barrier, leaving global
// loads (the next planes' prefetch) and stores in flight.  All inter-wave
// communication in these kernels goes through LDS.  Unlike __syncthreads() it
// carries no memory-model fence, so what it waits for does not depend on how
// the compiler lowers one; the empty asm statements keep the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0); vmcnt and expcnt untouched
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// The fused kernel
// ---------------------------------------------------------------------------
// Sign of subband u at the position with low bits (py, px): (-1)^(u_y py + u_x px).
__device__ __forceinline__ float band_sign(int u, int py, int px) {
    return (((u >> 1) & py) ^ (u & px & 1)) ? -1.f : 1.f;
}

// Raw +-1 butterfly of a 2x2 block a=(0,0), b=(0,1), c=(1,0), d=(1,1):
// r[u] = sum over the block of (-1)^(u_y py + u_x px) * pixel.
__device__ __forceinline__ void haar4(float a, float b, float c, float d, float (&r)[4]) {
    const float s01 = a + b, d01 = a - b, s23 = c + d, d23 = c - d;
    r[0] = s01 + s23;
    r[1] = d01 + d23;
    r[2] = s01 - s23;
    r[3] = d01 - d23;
}

// Value of v in lane L of this lane's quad (DPP quad permute: every lane of
// the quad reads lane L).
template <int L>
__device__ __forceinline__ float quad_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), L | (L << 2) | (L << 4) | (L << 6), 0xF, 0xF,
                                                   false));
}

// Rows 2*JY and 2*JY + 1 of a quad's 8x8 block, from the four lanes' 4x4
// blocks xk (lane 2*sy + sx holds rows 4*sy.., columns 4*sx..): r0/r1[h] are
// columns 4*h .. 4*h + 3.
template <int JY>
__device__ __forceinline__ void quad_rows(const float (&xk)[4][4], float (&r0)[2][4], float (&r1)[2][4]) {
    constexpr int ra = 2 * JY, rb = 2 * JY + 1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        r0[0][q] = quad_bcast<(ra >> 2) * 2>(xk[ra & 3][q]);
        r0[1][q] = quad_bcast<(ra >> 2) * 2 + 1>(xk[ra & 3][q]);
        r1[0][q] = quad_bcast<(rb >> 2) * 2>(xk[rb & 3][q]);
        r1[1][q] = quad_bcast<(rb >> 2) * 2 + 1>(xk[rb & 3][q]);
    }
}

// Level count of a fixed geometry (compile time); -1 for the runtime one.
template <class G>
constexpr int fixed_lm() {
    if constexpr (G::kFixed) {
        return G::Lm();
    } else {
        return -1;
    }
}

// Waves per SIMD a kernel is compiled for: a workgroup of 1024 threads (one
// per CU) needs 4; otherwise the register budget of fused_waves_per_simd.
template <class G, bool BWD, int BPQ>
constexpr int kernel_waves() {
    return G::kMaxThreads > 512 ? 4 : fused_waves_per_simd(BWD, BPQ, G::kNoLevels && BPQ == 1);
}

// Units of four pixels per thread of the next plane that the two-blocks-per-
// quad backward prefetches (fixed geometry, one plane per workgroup, the plane
// an exact number of unit steps); 0: no prefetch.
template <class G, bool BWD, int BPQ, bool VEC>
constexpr int next_plane_units() {
    if constexpr (G::kFixed && !G::kNHWC && VEC && BWD && BPQ > 1) {
        constexpr int wv = G::kWq / 4;
        if (G::kNP == 1 && G::kNthr % wv == 0 && (G::kHq * wv) % G::kNthr == 0) return G::kHq * wv / G::kNthr;
    }
    return 0;
}

// The plane's height and width: fixed at compile time in the instances for
// planes that fill their zero-extended size exactly ("whole" planes) or for
// one benchmark plane size, so that their bounds tests fold away and their
// row strides are shifts.
template <class G>
__device__ __forceinline__ int plane_h(const FusedArgs& a) {
    if constexpr (G::kPH > 0) return G::kPH;
    else return a.H;
}
template <class G>
__device__ __forceinline__ int plane_w(const FusedArgs& a) {
    if constexpr (G::kPW > 0) return G::kPW;
    else return a.W;
}

template <class G>
constexpr bool tail_possible() {
    if constexpr (G::kFixed) {
        constexpr int T = G::Lm() >= 3 ? (1 << G::Lm()) : 8;
        return G::kHq == T && G::kWq == T;
    }
    return true;
}

// Fixed-geometry forward whose register prefetch holds every 4-pixel unit of
// its plane group: the prefetch is on for every plane (the last plane of a
// segment loads its own group again, which is in L2) and the output stores go
// through a buffer resource whose range check drops the lanes outside the
// plane, so no memory instruction of the plane loop sits under a branch.
// The compiler then counts the stores issued after a prefetch load and waits
// for that load alone, instead of for every store of the previous plane.
template <class G, bool BWD, bool VEC, int PFU>
constexpr bool static_prefetch() {
    if constexpr (G::kFixed && !G::kDL && !BWD && VEC)
        return PFU * G::kNthr >= G::kNP * G::kHq * (G::kWq / 4);
    return false;
}

// With a static prefetch and a layout in which no other array overlaps the
// level-0 plane, that plane is dead once phase 2 ends: the next plane is
// committed there and then (and the one after it issued), so the plane loop
// needs no barrier and no staging at its top.  (Measured on 128x128 planes:
// one level 249.6 -> 241.2 us; without levels 169.4 -> 180.0 us, so the plain
// depthwise convolution keeps the staging at the loop top.)
template <class G, bool PFS>
constexpr bool early_commit() {
    if constexpr (PFS && G::kFixed) return !G::ovl() && G::bovl() == 0 && G::Lm() >= 1;
    return false;
}

template <int K, typename ST, bool BWD, int BPQ, bool VEC, class G>
__global__ void __launch_bounds__(G::kMaxThreads) __attribute__((amdgpu_waves_per_eu(kernel_waves<G, BWD, BPQ>())))
wtc_fused_kernel(const FusedArgs a) {
    constexpr int R = K / 2, KK = K * K;
    constexpr int KKP = (KK + 3) & ~3;   // LDS stride of one (level, band) weight set
    // Direct-load mode: planes are copied from device memory into their LDS slot
    // by DMA (global_load_lds), one plane ahead, with no register staging.
    constexpr bool DL = G::kDL;
    static_assert(!DL || (VEC && BPQ == 1), "direct loads: 4-pixel rows, one block per quad");
    constexpr bool SDL = DL && sizeof(ST) == 2;           // bf16: raw plane staged, widened per plane
    constexpr bool XDL = DL && BWD && sizeof(ST) == 4;    // fp32 backward: x plane in LDS too
    // x block of phase 2 reused in phase 4a (fixed geometry only: the
    // runtime-geometry kernel has no registers to spare)
    constexpr bool XQB = BWD && !XDL && BPQ == 1 && G::kFixed;
    constexpr int PFF = pf_capacity(BWD, BPQ);  // prefetch capacity, floats per thread
    constexpr int PFU = DL ? 1 : (VEC ? PFF / 4 : PFF);   // prefetch units (4-pixel groups or pixels)
    constexpr int UW = VEC ? 4 : 1;
    extern __shared__ __align__(16) float lds[];

    const G g(a);
    // plane size: a compile-time constant in whole-plane instances
    const int aH = plane_h<G>(a), aW = plane_w<G>(a);
    const int tid0 = threadIdx.x;
    const int nthr = g.nthr(), nquads = nthr >> 2;
    // This workgroup's planes: [q0, q1) in channel-major order (q = c*B + b),
    // at most two channel segments.
    const long qtot = (long)a.C * a.B;
    long q0, q1;
    int unit = 0;
    if (a.units) {
        // one (batch chunk, channel) unit, chunk-major, the units dealt to the
        // XCDs in contiguous ranges (workgroup i runs on XCD i % 8): the planes
        // of neighbouring channels, which share cache lines (channels-last
        // tensors, small odd planes), go through one L2 at about the same time
        const int U = a.C * a.nchunk, per = (U + 7) / 8, k8 = blockIdx.x >> 3;
        unit = (blockIdx.x & 7) * per + k8;
        if (k8 >= per || unit >= U) return;   // whole workgroup, before any barrier
        const int cu = unit % a.C, chunk = unit / a.C;
        q0 = (long)cu * a.B + (long)chunk * a.ppw;
        q1 = min(q0 + (long)a.ppw, (long)(cu + 1) * a.B);
    } else {
        q0 = (long)blockIdx.x * a.ppw;
        q1 = min(q0 + (long)a.ppw, qtot);
    }
    const int c_first = (int)(q0 / a.B);
    const int Lm = g.Lm();
    // Levels past the last one with a grid above 1 x 1 (the tail) exist only
    // when the whole plane fits one level-Lm cell, i.e. when the plane is
    // zero-extended to max(8, 2^Lm) on both sides: a fixed geometry of any
    // other size never has a tail, and its kernel carries no tail term.
    constexpr bool TAILS = !G::kFixed || tail_possible<G>();
    const bool tail = TAILS && a.L > Lm;
    const size_t plane_sz = (size_t)aH * aW;
    // global addressing: plane (b, c) starts at b C H W + c (channels-last) or
    // (b C + c) H W (NCHW); pixel (y, x) of a plane is (y W + x) ps further
    constexpr bool NHWC = G::kNHWC;
    static_assert(!(NHWC && DL && sizeof(ST) == 2), "channels-last bf16 planes are staged through registers");
    const size_t ps = NHWC ? (size_t)a.C : 1;
    auto plane_at = [&](const ST* base, long b, int ch) {
        return base + (size_t)b * a.C * plane_sz + (NHWC ? (size_t)ch : (size_t)ch * plane_sz);
    };
    const FastDiv dqpp = make_div(g.qpp()), dnqx = make_div(g.nqx());

    // Per-thread roles.  Recomputed at the top of every plane iteration from an
    // opaque copy of the thread index, so that the compiler does not hoist every
    // per-thread address out of the plane loop and keep them all live.
    int tid, t, sy, sx, slot, qpb[BPQ], qyv[BPQ], qxv[BPQ];
    float sgx, sgy;   // signs of the W- and H-direction high-pass of band t
    bool qok[BPQ];
    auto roles = [&](int tid_in) {
        tid = tid_in;
        t = tid & 3;
        const int Q = tid >> 2;
        sy = t >> 1;
        sx = t & 1;
        sgx = (t & 1) ? -1.f : 1.f;
        sgy = (t & 2) ? -1.f : 1.f;
        if constexpr (BPQ == 1) {
            slot = fdiv(Q, dqpp);
            qpb[0] = Q - slot * g.qpp();
        } else {
            slot = 0;
#pragma unroll
            for (int s = 0; s < BPQ; ++s) qpb[s] = Q + s * nquads;
        }
#pragma unroll
        for (int s = 0; s < BPQ; ++s) {
            qok[s] = (slot < g.NP()) && (qpb[s] < g.qpp());
            qyv[s] = fdiv(qpb[s], dnqx);
            qxv[s] = qpb[s] - qyv[s] * g.nqx();
        }
    };
    roles(tid0);

    for (int seg = 0; seg < 2; ++seg) {
    const int c = c_first + seg;
    const long qs = max(q0, (long)c * a.B), qe = min(q1, (long)(c + 1) * a.B);
    if (qs >= qe) break;
    const int b_begin = (int)(qs - (long)c * a.B);
    const int b_end = (int)(qe - (long)c * a.B);
    lds_barrier();  // the previous segment is done with the weights and the slots
    const ST* srcp = reinterpret_cast<const ST*>(a.src);
    const ST* auxp = reinterpret_cast<const ST*>(a.aux);
    ST* dstp = reinterpret_cast<ST*>(a.dst);

    // ---- plane staging: units of UW pixels, unit e -> (slot, row, column) ----
    const int wv = VEC ? (aW >> 2) : aW;
    const int per = aH * wv;
    const FastDiv dper = make_div(per), dwv = make_div(wv);
    // (the backward kernel with two blocks per quad never has the capacity; the
    // runtime-geometry backward stages synchronously: with a plane held in
    // registers beside its correlation accumulators it spills, measured 5-13 %
    // slower on 14x14 to 30x30 planes)
    constexpr bool PFS = static_prefetch<G, BWD, VEC, PFU>();
    // buffer-resource output stores (NCHW planes, byte offsets < 2^31)
    // (also the two-blocks-per-quad backward whose next plane is loaded
    // during the current one: the loop-top wait for those loads then leaves
    // this plane's dx stores outstanding)
    constexpr bool BST = (PFS || next_plane_units<G, BWD, BPQ, VEC>() > 0) && VEC && !G::kNHWC;
    constexpr bool EC = early_commit<G, PFS>();
    const bool pf_on = PFS || (!DL && !(BWD && BPQ > 1) && !(BWD && !G::kFixed) && a.pf_on != 0);
    float pf[PFU][UW];
    // With 4-pixel units the decode of each unit is done once per segment: its
    // offset within a plane group in device memory, and (packed) its plane
    // slot (bits 16+) and LDS offset (bits 0-15; slots fit in 64K floats);
    // -1 = no unit.  Single-pixel units decode on the fly (16 of them would
    // take too many registers): each is decoded once, when its load is issued,
    // and keeps its LDS destination until the commit.
    const int cplane = a.C * (int)plane_sz;   // < 2^31 / NP when prefetching
    int pf_goff[VEC ? PFU : 1], pf_lds[VEC ? PFU : 1];
    int pf_dst[VEC ? 1 : PFU];
    if (VEC && pf_on) {
#pragma unroll
        for (int k = 0; k < PFU; ++k) {
            const int e = tid + k * nthr;
            pf_goff[k] = 0;
            pf_lds[k] = -1;
            if (e < g.NP() * per) {
                const int s2 = fdiv(e, dper), m = e - s2 * per;
                const int y = fdiv(m, dwv), xq = m - y * wv;
                pf_goff[k] = s2 * cplane + (y * aW + xq * UW) * (NHWC ? a.C : 1);
                pf_lds[k] = (s2 << 16) | (s2 * g.slot() + g.a0_off() + (y + R) * g.a0_S() + R + xq * UW);
            }
        }
    }
    // issue the global loads of the NP planes starting at batch index bbn
    auto pf_issue = [&](int bbn) {
        if constexpr (VEC) {
            // Every unit's load is issued, a missing unit reading the plane's
            // first pixels (the caller issues only for planes that exist), and
            // the commit waits for every unit: no load of these registers is
            // then left in flight on any path, so the compiler needs no
            // wait-for-everything before this plane's loads.
            const ST* base = plane_at(srcp, bbn, c);
#pragma unroll
            for (int k = 0; k < PFU; ++k) {
                const bool ok = pf_lds[k] >= 0 && bbn + (pf_lds[k] >> 16) < b_end;
                gload4<NHWC>(base + (ok ? pf_goff[k] : 0), ps, pf[k]);
            }
        } else if constexpr (G::kFixed) {
            // unit k: plane k % NP, in-plane pixel tid + (k / NP) * nthr, so one
            // row/column decode serves the NP planes (NP is a constant here; the
            // planner prefetches only when NP * ceil(H W / nthr) units fit)
            constexpr int NPc = G::NP(), NJ = (PFU + NPc - 1) / NPc;
            const ST* base = plane_at(srcp, bbn, c);
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj) {
                const int m = tid + jj * nthr;
                const int y = fdiv(m, dwv), xq = m - y * wv;
                const int dst0 = g.a0_off() + (y + R) * g.a0_S() + R + xq;
#pragma unroll
                for (int s2 = 0; s2 < NPc; ++s2) {
                    const int k = jj * NPc + s2;
                    if (k >= PFU) continue;
                    pf_dst[k] = -1;
                    if (m < per && bbn + s2 < b_end) {
                        pf[k][0] = to_f32(base[s2 * cplane + m * ps]);
                        pf_dst[k] = s2 * g.slot() + dst0;
                    }
                }
            }
        } else {
            const ST* base = plane_at(srcp, bbn, c);
#pragma unroll
            for (int k = 0; k < PFU; ++k) {
                const int e = tid + k * nthr;
                pf_dst[k] = -1;
                if (e < g.NP() * per) {
                    const int s2 = fdiv(e, dper), m = e - s2 * per;
                    if (bbn + s2 < b_end) {
                        pf[k][0] = to_f32(base[s2 * cplane + m * ps]);
                        const int y = fdiv(m, dwv), xq = m - y * wv;
                        pf_dst[k] = s2 * g.slot() + g.a0_off() + (y + R) * g.a0_S() + R + xq;
                    }
                }
            }
        }
    };
    auto pf_commit = [&](int bbn) {
        if constexpr (VEC) {
#pragma unroll
            for (int k = 0; k < PFU; ++k) {
#pragma unroll
                for (int i = 0; i < UW; ++i) asm volatile("" : "+v"(pf[k][i]));   // waited for on every path
            }
#pragma unroll
            for (int k = 0; k < PFU; ++k)
                if (pf_lds[k] >= 0 && bbn + (pf_lds[k] >> 16) < b_end) {
                    float* d = lds + (pf_lds[k] & 0xFFFF);
#pragma unroll
                    for (int i = 0; i < UW; ++i) d[i] = pf[k][i];
                }
        } else {
            (void)bbn;
#pragma unroll
            for (int k = 0; k < PFU; ++k)
                if (pf_dst[k] >= 0) lds[pf_dst[k]] = pf[k][0];
        }
    };
    // Direct loads: rows [0, H) of the NP planes starting at batch index bbn go to
    // region `roff` of their slots (row stride rS, interior at row rr, column rc),
    // one 64-pixel row chunk per wave instruction; the LDS destination of lane l
    // is the chunk start + 4 l bytes, so lanes past the row end are masked off.
    // Cells outside the interior are never written (zeroed once per segment).
    auto dl_issue = [&](const ST* base, int roff, int rS, int rr, int rc, int bbn, int ch, int bend) {
        if constexpr (DL && !SDL && G::kFixed) {
            // fixed geometry: the row loop is unrolled (no branches between the
            // copies); rows of a plane are dealt to the waves round-robin
            static_assert(G::Wq() <= 64, "direct loads: one 64-lane row chunk");
            constexpr int NW = G::nthr() / 64, NPc = G::NP(), JT = NPc * G::Hq();
            constexpr int NJ = (JT + NW - 1) / NW;
            const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6), lane = tid0 & 63;
            auto rows = [&](auto full) {
#pragma unroll
                for (int jj = 0; jj < NJ; ++jj) {
                    const int j = wave + jj * NW;
                    const int s2 = NPc == 1 ? 0 : j / G::Hq();
                    const int r = j - s2 * G::Hq();
                    if (JT % NW != 0 && j >= JT) continue;
                    if (!decltype(full)::value && r >= aH) continue;
                    if (NPc > 1 && bbn + s2 >= bend) continue;
                    __builtin_amdgcn_global_load_lds(
                        (const void*)(plane_at(base, bbn + s2, ch) + ((size_t)r * aW + lane) * ps),
                        (__attribute__((address_space(3))) void*)(lds + s2 * g.slot() + roff + (r + rr) * rS + rc),
                        4, 0, 0);
                }
            };
            if (lane < aW) {
                if (aH == G::Hq()) rows(std::true_type{});
                else rows(std::false_type{});
            }
        } else if constexpr (DL && !SDL) {
            // runtime geometry: one plane (the planner's direct-load plans have
            // NP = 1), addressed once; rows dealt to the waves round-robin, each
            // row in 64-pixel chunks
            if (bbn >= bend) return;
            // (lane from an opaque copy: no per-lane address is kept live across the plane loop)
            const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6), lane = opaque(tid0) & 63;
            const int nw = nthr >> 6;
            const ST* pb = plane_at(base, bbn, ch);
            float* lb = lds + roff + rr * rS + rc;
            for (int c0 = 0; c0 < aW; c0 += 64) {
                if (c0 + lane >= aW) break;
                const ST* src = pb + ((size_t)wave * aW + c0 + lane) * ps;
                float* dst = lb + wave * rS + c0;
                for (int r = wave; r < aH; r += nw, src += (size_t)nw * aW * ps, dst += nw * rS)
                    __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)dst,
                                                     4, 0, 0);
            }
        }
    };
    // bf16: the raw planes (H*W 16-bit pixels, contiguous) are copied word by
    // word into the staging area, 64 words per wave instruction
    auto stage_issue = [&](int bbn, int ch, int bend) {
        if constexpr (SDL && G::kFixed) {
            // fixed geometry: unrolled over the plane's 64-word chunks
            constexpr int NW = G::nthr() / 64, NPc = G::NP();
            constexpr int CH = (G::Hq() * G::Wq() / 2 + 63) / 64, JT = NPc * CH;
            constexpr int NJ = (JT + NW - 1) / NW;
            const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6), lane = tid0 & 63;
            const int words = (aH * aW) >> 1;
            auto chunks = [&](auto full) {
#pragma unroll
                for (int jj = 0; jj < NJ; ++jj) {
                    const int j = wave + jj * NW;
                    const int s2 = NPc == 1 ? 0 : j / CH, k = j - s2 * CH;
                    if (JT % NW != 0 && j >= JT) continue;
                    if (NPc > 1 && bbn + s2 >= bend) continue;
                    const int i = k * 64 + lane;
                    if (!decltype(full)::value && i >= words) continue;
                    __builtin_amdgcn_global_load_lds(
                        (const void*)(reinterpret_cast<const uint32_t*>(srcp + ((size_t)(bbn + s2) * a.C + ch) * plane_sz) +
                                      i),
                        (__attribute__((address_space(3))) void*)(lds + s2 * g.slot() + g.st_off() + k * 64), 4, 0, 0);
                }
            };
            if (words == G::Hq() * G::Wq() / 2 && words % 64 == 0) chunks(std::true_type{});
            else chunks(std::false_type{});
        } else if constexpr (SDL) {
            // runtime geometry, one plane (NP = 1 with direct loads)
            if (bbn >= bend) return;
            const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6), lane = opaque(tid0) & 63;
            const int nw = nthr >> 6;
            const int words = (aH * aW) >> 1;
            const uint32_t* src = reinterpret_cast<const uint32_t*>(srcp + ((size_t)bbn * a.C + ch) * plane_sz);
            float* dst = lds + g.st_off();
            for (int k = wave * 64; k < words; k += nw * 64)
                if (k + lane < words)
                    __builtin_amdgcn_global_load_lds((const void*)(src + k + lane),
                                                     (__attribute__((address_space(3))) void*)(dst + k), 4, 0, 0);
        }
    };
    // the first planes' copies are issued before the set-up below, which they
    // do not touch (interiors of the staging areas vs rings and weights)
    // (a second channel segment's first copies were issued at the end of the
    // first segment, where the layout allows it)
    constexpr bool XSEG = DL && G::kXSeg;
    const bool pre = XSEG && seg == 1;
    if (pf_on) pf_issue(b_begin);
    if constexpr (XDL) {
        for (int s2 = 0; s2 < g.NP(); ++s2)
            zero_ring(lds + s2 * g.slot() + g.xp_off(), g.Hq(), g.xp_S(), 0, aH, 0, aW, tid, nthr);
        if (!pre) dl_issue(auxp, g.xp_off(), g.xp_S(), 0, 0, b_begin, c, b_end);
    }
    if constexpr (DL && !SDL) {
        if (!pre) dl_issue(srcp, g.a0_off(), g.a0_S(), R, R, b_begin, c, b_end);
    }
    if constexpr (SDL) {
        if (!pre) stage_issue(b_begin, c, b_end);
    }

    // ---- zero the halo rings: per segment (the backward reduction reuses the
    // slots), and per plane where regions overlap ----
    for (int s2 = 0; s2 < g.NP(); ++s2) {
        float* S = lds + s2 * g.slot();
        zero_ring(S + g.a0_off(), g.a0_rows(), g.a0_S(), R, aH, R, aW, tid, nthr);
        for (int i = 1; i <= Lm; ++i)
            for (int u = 0; u < 4; ++u)
                zero_ring(S + g.b_off(i) + u * g.b_bs(i), g.b_rows(i), g.b_S(i), R, g.Hq() >> i, R,
                          g.Wq() >> i, tid, nthr);
    }
    // ---- fold scales and Haar normalisations into the level weights ----
    // W'_i = 4^-i s_i W_i (LDS, per workgroup).  The base weights stay unfolded;
    // s0 is applied once per output pixel, fused with the synthesis add.
    // Every parameter is read from device memory here, once per workgroup: no
    // vector-memory load may sit behind the next planes' prefetch in the plane
    // loop (vector-memory completions are counted in order).
    float* wts = lds + g.wts_off();
    // (level i, band u) at wts + (4 i + u) KKP: 16-byte aligned sets
    float* wbase = wts + 4 * a.L * KKP;         // unfolded base weights W0[c]
    for (int e = tid; e < 4 * a.L * KK; e += nthr) {
        const int i = e / (4 * KK), rem = e - i * 4 * KK, u = rem / KK, tap = rem - u * KK;
        const float sc = ldexpf(a.sl[((size_t)i * a.C + c) * 4 + u], -2 * (i + 1));
        wts[(i * 4 + u) * KKP + tap] = sc * a.wl[(((size_t)i * a.C + c) * 4 + u) * KK + tap];
    }
    for (int e = tid; e < KK; e += nthr) wbase[e] = a.w0[(size_t)c * KK + e];
    if (tid == 0) {
        wbase[KK] = BWD ? 0.f : a.b0[c];
        wbase[KK + 1] = a.s0[c];
    }
    // two blocks per quad, backward, three levels or more (where 25 persistent
    // accumulators spilled): per-row C_0 accumulators after the weights (rows
    // of 16 lanes; each slot has one writer, lane 15 of its row)
    const bool flush0 = BWD && BPQ > 1 && Lm >= 3;
    float* c0acc = wts + ((KKP * 4 * a.L + KK + 4 + 3) & ~3);
    if (flush0)
        for (int e = tid; e < (nthr >> 4) * KK; e += nthr) c0acc[e] = 0.f;

    lds_barrier();
    // tail levels (1x1 grids): kappa = sum of their folded centre taps
    float kappa = 0.f;
    for (int i = Lm; i < a.L; ++i)
        for (int u = 0; u < 4; ++u) kappa += wts[(i * 4 + u) * KKP + (KK >> 1)];

    // ---- persistent backward accumulators ----
    constexpr int ND = G::kDeep;
    float corr0[KK], corr1[KK], corr2[KK], cdeep[ND][K];
#pragma unroll
    for (int i = 0; i < KK; ++i) corr0[i] = corr1[i] = corr2[i] = 0.f;
#pragma unroll
    for (int q = 0; q < ND; ++q)
#pragma unroll
        for (int kx = 0; kx < K; ++kx) cdeep[q][kx] = 0.f;
    float sumg = 0.f, tailc = 0.f;
    // deep-level (>= 3) correlation role: subband du, kernel row dky, band rows
    // dsb, dsb + dsub, ...; one accumulator per kernel column
    const int drole = tid;
    const int droles = 4 * K * g.dsub();
    const bool dactive = BWD && drole < droles;
    const int du = drole & 3, dky = (drole >> 2) % K, dsb = (drole >> 2) / K;

    // Two-blocks-per-quad backward with one or three levels, on a plane that
    // fills its zero-extended size: the next plane's loads are issued when the
    // synthesis phase starts and stored at the top of the next iteration, so
    // their round trip passes during the synthesis and the stores of this
    // plane (the registers are free there; a prefetch that lived through the
    // whole plane would spill).  Unit k of a thread is pixel 4 (tid + k nthr).
    constexpr int XPU0 = next_plane_units<G, BWD, BPQ, VEC>();
    constexpr bool XPF = XPU0 > 0;
    constexpr int XPU = XPF ? XPU0 : 1;
    constexpr int XWV = XPF ? G::kWq / 4 : 1;   // 4-pixel units per plane row
    constexpr int XRPK = XPF ? G::kNthr / XWV : 1;   // plane rows per unit step
    const bool xwhole = XPF && aH == g.Hq() && aW == g.Wq();
    float xpf[XPU][4];
#pragma unroll
    for (int k = 0; k < XPU; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) xpf[k][i] = 0.f;
    bool xpf_ok = false;   // this plane was prefetched by the previous iteration

    // the segment's first prefetch has landed: no load is pending on entry to
    // the plane loop, so the loop-top wait counts only the previous
    // iteration's prefetch loads and the stores issued after them
    if constexpr (PFS || XPF) __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
    if constexpr (EC) {
        // the segment's first planes go in here; the loop commits the others
        pf_commit(b_begin);
        lds_barrier();
        pf_issue(b_begin + g.NP() < b_end ? b_begin + g.NP() : b_begin);
    }
    for (int bb = b_begin; bb < b_end; bb += g.NP()) {
        roles(opaque(tid0));
        const int b = bb + slot;
        const bool pok = (slot < g.NP()) && (b < b_end);
        float* S = lds + (slot < g.NP() ? slot : 0) * g.slot();
        const size_t poff = (size_t)b * a.C * plane_sz + (NHWC ? (size_t)c : (size_t)c * plane_sz);

        if constexpr (DL) {
            // this plane's direct loads have landed (every wave's), and the
            // previous plane is fully consumed
            __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
            lds_barrier();
            if constexpr (SDL) {
                // widen the staged 16-bit pixels into the level-0 plane (4 per unit)
                typedef uint32_t lds_u2 __attribute__((ext_vector_type(2)));
                const int wq = aW >> 2, per_plane = aH * wq;
                for (int e = tid; e < g.NP() * per_plane; e += nthr) {
                    const int s2 = g.NP() == 1 ? 0 : e / per_plane, m = e - s2 * per_plane;
                    if (bb + s2 >= b_end) continue;
                    const int y = m / wq, xq = m - y * wq;
                    float* Sl = lds + s2 * g.slot();
                    const lds_u2 v = *reinterpret_cast<const lds_u2*>(Sl + g.st_off() + 2 * m);
                    float* d = Sl + g.a0_off() + (y + R) * g.a0_S() + R + 4 * xq;
                    *reinterpret_cast<lds_f2*>(d) = lds_f2{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u)};
                    *reinterpret_cast<lds_f2*>(d + 2) =
                        lds_f2{__uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u)};
                }
                lds_barrier();
                // the staging area is free: the next planes' copies land meanwhile
                // (backward: after this plane's last x load, whose wait would
                // otherwise also wait for the copy, vector-memory counts being in order)
                if (!BWD && bb + g.NP() < b_end) stage_issue(bb + g.NP(), c, b_end);
            }
        } else if constexpr (!EC) {
        lds_barrier();  // the previous plane is fully consumed

        // ---------------- phase 1: stage the planes in LDS ----------------
        if constexpr (XPF) {
            // the prefetch registers are consumed on every path, so no load
            // into them is left in flight when the next ones are issued
#pragma unroll
            for (int k = 0; k < XPU; ++k)
#pragma unroll
                for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(xpf[k][i]));
        }
        if (pf_on) {
            pf_commit(bb);
        } else if (XPF && xpf_ok) {
            // this plane, loaded by the previous iteration
            const int t1 = opaque(tid);
            float* dst0 = lds + g.a0_off() + ((t1 / XWV) + R) * g.a0_S() + R + (t1 % XWV) * 4;
#pragma unroll
            for (int k = 0; k < XPU; ++k)
#pragma unroll
                for (int i = 0; i < 4; ++i) dst0[k * XRPK * g.a0_S() + i] = xpf[k][i];
        } else if constexpr (VEC && BWD && BPQ > 1 && (fixed_lm<G>() == 1 || fixed_lm<G>() == 3)) {
            // the units' loads are issued in batches of SB before their stores:
            // one memory latency per batch instead of one per unit.  The
            // two-blocks-per-quad backward has no registers for a prefetch that
            // lives through a plane; a batch of four fits beside its
            // accumulators with one or three levels (128x128 planes, L = 3:
            // 642 -> 585 us), while with two, four or five levels even a batch of
            // two spills 24-48 VGPRs and measured slower.
            constexpr int SU = (G::NP() * G::Hq() * (G::Wq() / UW) + G::nthr() - 1) / G::nthr();
            constexpr int SB = 4;
#pragma unroll
            for (int k0 = 0; k0 < SU; k0 += SB) {
                float sv[SB][4];
#pragma unroll
                for (int k = 0; k < SB && k0 + k < SU; ++k) {
                    const int e = tid + (k0 + k) * nthr;
                    const int s2 = fdiv(e, dper), m = e - s2 * per;
                    const int y = fdiv(m, dwv), xq = m - y * wv;
                    if (e < g.NP() * per && bb + s2 < b_end)
                        gload4<NHWC>(plane_at(srcp, bb + s2, c) + ((size_t)y * aW + xq * UW) * ps, ps, sv[k]);
                }
#pragma unroll
                for (int k = 0; k < SB && k0 + k < SU; ++k) {
                    const int e = tid + (k0 + k) * nthr;
                    const int s2 = fdiv(e, dper), m = e - s2 * per;
                    const int y = fdiv(m, dwv), xq = m - y * wv;
                    if (e < g.NP() * per && bb + s2 < b_end) {
                        float* d = lds + s2 * g.slot() + g.a0_off() + (y + R) * g.a0_S() + R + xq * UW;
#pragma unroll
                        for (int i = 0; i < 4; ++i) d[i] = sv[k][i];
                    }
                }
            }
        } else {
            for (int e = tid; e < g.NP() * per; e += nthr) {
                const int s2 = fdiv(e, dper), m = e - s2 * per;
                if (bb + s2 >= b_end) continue;
                const int y = fdiv(m, dwv), xq = m - y * wv;
                const ST* pl = plane_at(srcp, bb + s2, c) + ((size_t)y * aW + xq * UW) * ps;
                float* d = lds + s2 * g.slot() + g.a0_off() + (y + R) * g.a0_S() + R + xq * UW;
                if constexpr (VEC) {
                    float v[4];
                    gload4<NHWC>(pl, ps, v);
#pragma unroll
                    for (int i = 0; i < 4; ++i) d[i] = v[i];
                } else {
                    d[0] = to_f32(pl[0]);
                }
            }
        }
        if (g.bovl() > 0) {
            zero_rings<R>(lds, g, g.a0_off(), 0, 1, g.a0_rows(), g.a0_S(), aH, aW, tid, nthr);
        } else if (g.ovl()) {
            for (int s2 = 0; s2 < g.NP(); ++s2)
                zero_ring(lds + s2 * g.slot() + g.a0_off(), g.a0_rows(), g.a0_S(), R, aH, R, aW, tid, nthr);
        }
        lds_barrier();
        // the next planes' loads fly while this plane is computed
        if constexpr (PFS) pf_issue(bb + g.NP() < b_end ? bb + g.NP() : bb);
        else if (pf_on && bb + g.NP() < b_end) pf_issue(bb + g.NP());
        }

        // ---------------- phase 2: base conv; analysis of levels 1..3 ----------------
        float acc[BPQ][4][4];
        // backward without an LDS copy of x, one block per quad: this lane's 4x4
        // block of x, kept for phase 4a (the quad's 8x8 block by quad broadcasts)
        float xkeep[XQB ? 4 : 1][4];
        // raw bands of this lane's block: level 1 at its 2x2 positions [jy][jx][u],
        // level 2 at its position [u], level 3 (band t) at the quad's position
        float hv1[BPQ][2][2][4], hv2[BPQ][4], hv3[BPQ];
        // write the early bands of levels lo..hi of block s
        auto put_bands = [&](int s, int lo, int hi) {
            const int qy = qyv[s], qx = qxv[s];
            const int py0 = 8 * qy + 4 * sy, px0 = 8 * qx + 4 * sx;
            if (lo <= 1 && 1 <= hi) {
                float* B1 = S + g.b_off(1);
#pragma unroll
                for (int jy = 0; jy < 2; ++jy)
#pragma unroll
                    for (int jx = 0; jx < 2; ++jx) {
                        const int off = (py0 / 2 + jy + R) * g.b_S(1) + (px0 / 2 + jx + R);
#pragma unroll
                        for (int u = 0; u < 4; ++u) B1[u * g.b_bs(1) + off] = hv1[s][jy][jx][u];
                    }
            }
            if (g.early() >= 2 && lo <= 2 && 2 <= hi) {
                float* B2 = S + g.b_off(2);
                const int off2 = (2 * qy + sy + R) * g.b_S(2) + 2 * qx + sx + R;
#pragma unroll
                for (int u = 0; u < 4; ++u) B2[u * g.b_bs(2) + off2] = hv2[s][u];
            }
            if (g.early() >= 3 && lo <= 3 && 3 <= hi)
                S[g.b_off(3) + t * g.b_bs(3) + (qy + R) * g.b_S(3) + qx + R] = hv3[s];
        };
#pragma unroll
        for (int s = 0; s < BPQ; ++s) {
            if (!(pok && qok[s])) continue;
            const int qy = qyv[s], qx = qxv[s];
            const int py0 = 8 * qy + 4 * sy, px0 = 8 * qx + 4 * sx;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[s][i][j] = 0.f;
            float w[KK];
            load_w4<K, BWD>(wbase, w);
            float xo[4][4];
            if constexpr (XDL) {
                const float* xr = S + g.xp_off() + py0 * g.xp_S() + px0;
#pragma unroll
                for (int i = 0; i < 4; ++i) lds_row<4, 4>(xr + i * g.xp_S(), xo[i]);
            } else if constexpr (BWD) {
                const ST* xp = auxp + poff + (size_t)opaque(py0 * aW + px0) * ps;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    ld_row4<VEC, NHWC>(xp + (size_t)i * aW * ps, py0 + i < aH, px0, aW, xo[i], ps);
                if constexpr (XQB) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j) xkeep[i][j] = xo[i][j];
                }
            }
            const float* win = S + g.a0_off() + py0 * g.a0_S() + px0;
            // the block itself (window centre), for the raw analysis cascade in
            // registers: handed back by the stencil as its rows pass (except in
            // the two-blocks-per-quad backward, where keeping it live through
            // the stencil spills: read again there)
            constexpr bool CTRS = !(BWD && BPQ > 1);
            float ctr[4][4];
            if (CTRS && !(G::kSub && a.nobase)) {
                stencil<K, 4, 4, 4, BWD, CTRS>(win, g.a0_S(), w, acc[s], xo, corr0, ctr);
            } else {
                if (!(G::kSub && a.nobase)) stencil<K, 4, 4, 4, BWD>(win, g.a0_S(), w, acc[s], xo, corr0);
                // (the LL problem of a peeled plane has no base conv: scale and bias 0)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float rowv[4];
                    lds_row<4, (R % 4 == 0) ? 4 : ((R % 2 == 0) ? 2 : 1)>(win + (i + R) * g.a0_S() + R, rowv);
#pragma unroll
                    for (int j = 0; j < 4; ++j) ctr[i][j] = rowv[j];
                }
            }
            if constexpr (BWD) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) sumg += ctr[i][j];
            }
            if (Lm >= 1) {
#pragma unroll
                for (int jy = 0; jy < 2; ++jy)
#pragma unroll
                    for (int jx = 0; jx < 2; ++jx) {
                        haar4(ctr[2 * jy][2 * jx], ctr[2 * jy][2 * jx + 1], ctr[2 * jy + 1][2 * jx],
                              ctr[2 * jy + 1][2 * jx + 1], hv1[s][jy][jx]);
                        if (g.bovl() != 1) {   // level 1 is not over the level-0 plane: write at once
                            const int off = (py0 / 2 + jy + R) * g.b_S(1) + (px0 / 2 + jx + R);
#pragma unroll
                            for (int u = 0; u < 4; ++u) S[g.b_off(1) + u * g.b_bs(1) + off] = hv1[s][jy][jx][u];
                        }
                    }
                if (g.early() >= 2) {
                    // this lane's 4x4 block is one level-2 position
                    haar4(hv1[s][0][0][0], hv1[s][0][1][0], hv1[s][1][0][0], hv1[s][1][1][0], hv2[s]);
                    if (g.bovl() == 0 || g.bovl() > 2) put_bands(s, 2, 2);
                    if (g.early() >= 3) {
                        // the quad's 8x8 block is one level-3 position: lane t
                        // gathers the quad's four level-2 LL values, keeps band t
                        const int qb = (tid & 63) & ~3;
                        const float l0 = __shfl(hv2[s][0], qb + 0, 64), l1 = __shfl(hv2[s][0], qb + 1, 64);
                        const float l2 = __shfl(hv2[s][0], qb + 2, 64), l3 = __shfl(hv2[s][0], qb + 3, 64);
                        hv3[s] = fmaf(sgy, fmaf(sgx, l3, l2), fmaf(sgx, l1, l0));
                        if (g.bovl() == 0 || g.bovl() > 3) put_bands(s, 3, 3);
                    }
                }
            } else if (tail && py0 == 0 && px0 == 0) {
                // every level is a 1x1 grid: the tail term enters at pixel (0, 0)
                S[g.tail_off()] = ctr[0][0] * kappa;
                if constexpr (BWD) tailc = fmaf(ctr[0][0], xo[0][0], tailc);
            }
        }
        if (flush0) {
            // this plane's C_0 into the row accumulators: the 25 accumulators
            // are live through phase 2 only, not across the levels.  A
            // no-return LDS add per value; each slot has a single writer, so
            // the order of the sums is fixed.
            const int crow = tid >> 4;
#pragma unroll
            for (int q = 0; q < KK; ++q) {
                const float v = row_sum(corr0[q]);
                if ((tid & 15) == 15)
                    __hip_atomic_fetch_add(c0acc + crow * KK + q, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                corr0[q] = 0.f;
            }
        }
        if (g.bovl() >= 1 && g.bovl() <= Lm) {
            // these bands live over the level-0 plane: write them once every wave
            // is done reading it, and restore the zero rings the plane covered
            lds_barrier();
#pragma unroll
            for (int s = 0; s < BPQ; ++s)
                if (pok && qok[s]) put_bands(s, g.bovl(), 3);
            for (int i = g.bovl(); i <= Lm; ++i)
                zero_rings<R>(lds, g, g.b_off(i), g.b_bs(i), 4, g.b_rows(i), g.b_S(i), g.Hq() >> i, g.Wq() >> i, tid,
                              nthr);
        }
        lds_barrier();
        // the level-0 plane is dead: the next planes' copies land during the rest
        if (DL && !SDL && bb + g.NP() < b_end) dl_issue(srcp, g.a0_off(), g.a0_S(), R, R, bb + g.NP(), c, b_end);
        if constexpr (EC) {
            // the next planes (prefetched during this plane's phase 2) go in
            // now -- phases 3..6 never read the level-0 plane, and their
            // barriers order these writes before the next phase 2 -- and the
            // planes after them are issued (a segment's last planes reload
            // the group loaded most recently, which exists and is in L2)
            pf_commit(bb + g.NP());
            const int nb2 = bb + 2 * g.NP();
            pf_issue(nb2 < b_end ? nb2 : (bb + g.NP() < b_end ? bb + g.NP() : bb));
        }

        // Two-blocks-per-quad backward: the first block's first two x row pairs
        // for the level-1 analysis below are loaded now, so their round trip
        // passes during phase 3 and the deep levels (fixed geometry: every
        // thread owns both its blocks).  With one or three levels (128x128
        // planes: L = 1 511 -> 484 us, L = 3 -1 %); with two levels it spills
        // and measured 2 % slower, with four or five no change.
        constexpr bool XPRE = BWD && !XDL && !XQB && BPQ > 1 && VEC && !NHWC &&
                              (fixed_lm<G>() == 1 || fixed_lm<G>() == 3);
        float xpre0[XPRE ? 2 : 1][2][4], xpre1[XPRE ? 2 : 1][2][4];
        if constexpr (XPRE) {
            const int qy = qyv[0], qx = qxv[0];
            const ST* xp = auxp + poff + (size_t)opaque(8 * qy * aW + 8 * qx);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const ST* p0r = xp + (size_t)(2 * h) * aW;
                const int yh = 8 * qy + 2 * h;
                ld_row4<VEC, NHWC>(p0r, yh < aH, 8 * qx, aW, xpre0[h][0]);
                ld_row4<VEC, NHWC>(p0r + 4, yh < aH, 8 * qx + 4, aW, xpre0[h][1]);
                ld_row4<VEC, NHWC>(p0r + (size_t)aW, yh + 1 < aH, 8 * qx, aW, xpre1[h][0]);
                ld_row4<VEC, NHWC>(p0r + (size_t)(aW + 4), yh + 1 < aH, 8 * qx + 4, aW, xpre1[h][1]);
            }
        }

        // ---------------- phase 3: analysis of levels early_lv+1..Lm ----------------
        for (int i = g.early() + 1; i <= Lm; ++i) {
            const int hi = g.Hq() >> i, wi = g.Wq() >> i, Si = g.b_S(i), bs = g.b_bs(i);
            const int pi = hi * wi;
            const FastDiv dpi = make_div(pi), dwi = make_div(wi);
            const int Sp = g.b_S(i - 1);
            for (int e = tid; e < g.NP() * pi; e += nthr) {
                const int s2 = fdiv(e, dpi), m = e - s2 * pi;
                if (bb + s2 >= b_end) continue;
                float* Sl = lds + s2 * g.slot();
                const int jy = fdiv(m, dwi), jx = m - jy * wi;
                const float* LL = Sl + g.b_off(i - 1) + (2 * jy + R) * Sp + 2 * jx + R;
                float r[4];
                haar4(LL[0], LL[1], LL[Sp], LL[Sp + 1], r);
                float* Bi = Sl + g.b_off(i) + (jy + R) * Si + jx + R;
#pragma unroll
                for (int u = 0; u < 4; ++u) Bi[u * bs] = r[u];
            }
            if (g.ovl() && g.bovl() == 0)  // this level lives where the level-0 plane was staged
                zero_rings<R>(lds, g, g.b_off(i), bs, 4, g.b_rows(i), Si, hi, wi, tid, nthr);
            lds_barrier();
        }

        // ---------------- phase 4a: levels >= 3 flat, then levels 1 and 2 subband per lane ----------------
        // The deep convolutions (their bands are complete after phase 2/3) come
        // first, in the same phase as the band-per-lane stencils: their short
        // chains of LDS reads overlap the stencils' arithmetic.
        for (int i = 3; i <= Lm; ++i) {
            const int hi = g.Hq() >> i, wi = g.Wq() >> i, Si = g.b_S(i), bs = g.b_bs(i);
            const int pi4 = 4 * hi * wi;
            const FastDiv dpi = make_div(pi4), dwi = make_div(wi);
            for (int e = tid; e < g.NP() * pi4; e += nthr) {
                const int s2 = fdiv(e, dpi), m = e - s2 * pi4;
                if (bb + s2 >= b_end) continue;
                float* Sl = lds + s2 * g.slot();
                const int u = m & 3, j = m >> 2;
                const int jy = fdiv(j, dwi), jx = j - jy * wi;
                float w[KK];
                load_w4<K, BWD>(wts + ((i - 1) * 4 + u) * KKP, w);
                const float* win = Sl + g.b_off(i) + u * bs + jy * Si + jx;
                float accv = 0.f;
#pragma unroll
                for (int ky = 0; ky < K; ++ky)
#pragma unroll
                    for (int kx = 0; kx < K; ++kx) accv = fmaf(w[ky * K + kx], win[ky * Si + kx], accv);
                Sl[g.yd_off(i) + u * hi * wi + j] = accv;
            }
        }
        float y1[BPQ][4][4], y2[BPQ][2][2];
#pragma unroll
        for (int s = 0; s < BPQ; ++s) {
            if (!(pok && qok[s]) || Lm < 1) continue;
            const int qy = qyv[s], qx = qxv[s];
            float rx1[4][4], rx2[2][2];
            float ll2[2][2];
            if constexpr (BWD) {
                // x over the quad's 8x8 block -> band t (and LL) at levels 1, 2, 3
                float ll1[4][4];
                float xr0[2][2][4], xr1[2][2][4];
                const ST* xp = auxp + poff + (size_t)opaque(8 * qy * aW + 8 * qx) * ps;
#pragma unroll
                for (int jy = 0; jy < 4; ++jy) {
                    float r0[2][4], r1[2][4];
                    const int y0 = 8 * qy + 2 * jy;
                    if constexpr (XDL) {
                        const float* xr = S + g.xp_off() + y0 * g.xp_S() + 8 * qx;
                        lds_row<4, 4>(xr, r0[0]);
                        lds_row<4, 4>(xr + 4, r0[1]);
                        lds_row<4, 4>(xr + g.xp_S(), r1[0]);
                        lds_row<4, 4>(xr + g.xp_S() + 4, r1[1]);
                    } else if constexpr (XQB) {
                        if (jy == 0) quad_rows<0>(xkeep, r0, r1);
                        if (jy == 1) quad_rows<1>(xkeep, r0, r1);
                        if (jy == 2) quad_rows<2>(xkeep, r0, r1);
                        if (jy == 3) quad_rows<3>(xkeep, r0, r1);
                    } else {
                    // row pairs loaded two at a time: one memory round trip per two pairs
                    if (XPRE && s == 0 && jy == 0) {
#pragma unroll
                        for (int h = 0; h < 2; ++h)
#pragma unroll
                            for (int q = 0; q < 2; ++q)
#pragma unroll
                                for (int i = 0; i < 4; ++i) {
                                    xr0[h][q][i] = xpre0[XPRE ? h : 0][q][i];
                                    xr1[h][q][i] = xpre1[XPRE ? h : 0][q][i];
                                }
                    } else if ((jy & 1) == 0) {
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const ST* p0r = xp + (size_t)(2 * (jy + h)) * aW * ps;
                            const int yh = y0 + 2 * h;
                            ld_row4<VEC, NHWC>(p0r, yh < aH, 8 * qx, aW, xr0[h][0], ps);
                            ld_row4<VEC, NHWC>(p0r + 4 * ps, yh < aH, 8 * qx + 4, aW, xr0[h][1], ps);
                            ld_row4<VEC, NHWC>(p0r + (size_t)aW * ps, yh + 1 < aH, 8 * qx, aW, xr1[h][0], ps);
                            ld_row4<VEC, NHWC>(p0r + (size_t)(aW + 4) * ps, yh + 1 < aH, 8 * qx + 4, aW, xr1[h][1], ps);
                        }
                    }
#pragma unroll
                    for (int q = 0; q < 2; ++q)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            r0[q][i] = xr0[jy & 1][q][i];
                            r1[q][i] = xr1[jy & 1][q][i];
                        }
                    }
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
#pragma unroll
                for (int jy = 0; jy < 2; ++jy)
#pragma unroll
                    for (int jx = 0; jx < 2; ++jx) {
                        const float p0 = ll1[2 * jy][2 * jx], p1 = ll1[2 * jy][2 * jx + 1];
                        const float p2 = ll1[2 * jy + 1][2 * jx], p3 = ll1[2 * jy + 1][2 * jx + 1];
                        ll2[jy][jx] = (p0 + p1) + (p2 + p3);
                        rx2[jy][jx] = fmaf(sgy, fmaf(sgx, p3, p2), fmaf(sgx, p1, p0));
                    }
                if (Lm >= 3) {
                    const float rx3 = fmaf(sgy, fmaf(sgx, ll2[1][1], ll2[1][0]), fmaf(sgx, ll2[0][1], ll2[0][0]));
                    const int h3 = g.Hq() >> 3, w3 = g.Wq() >> 3;
                    S[g.xb_off(3) + t * h3 * w3 + qy * w3 + qx] = rx3;
                }
                if (tail && qpb[s] == 0 && t == 0) {
                    // tail correlation: raw LL of g and of x at level Lm, position (0, 0)
                    const float rho = S[g.b_off(Lm) + R * g.b_S(Lm) + R];
                    if (Lm == 1) tailc = fmaf(rho, ll1[0][0], tailc);
                    if (Lm == 2) tailc = fmaf(rho, ll2[0][0], tailc);
                }
            }
            {
                float w[KK];
                load_w4<K, BWD>(wts + t * KKP, w);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) y1[s][i][j] = 0.f;
                const float* win = S + g.b_off(1) + t * g.b_bs(1) + (4 * qy) * g.b_S(1) + 4 * qx;
                stencil<K, 4, 4, 4, BWD>(win, g.b_S(1), w, y1[s], rx1, corr1);
            }
            if (Lm >= 2) {
                float w[KK];
                load_w4<K, BWD>(wts + (4 + t) * KKP, w);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) y2[s][i][j] = 0.f;
                const float* win = S + g.b_off(2) + t * g.b_bs(2) + (2 * qy) * g.b_S(2) + 2 * qx;
                stencil<K, 2, 2, 2, BWD>(win, g.b_S(2), w, y2[s], rx2, corr2);
            }
            // tail term: rho = raw LL of the convolved tensor at level Lm, position (0,0)
            if (tail && qpb[s] == 0 && t == 0) S[g.tail_off()] = S[g.b_off(Lm) + R * g.b_S(Lm) + R] * kappa;
        }

        if (SDL && BWD && bb + g.NP() < b_end) stage_issue(bb + g.NP(), c, b_end);

        if constexpr (XPF) {
            xpf_ok = xwhole && bb + 1 < b_end;
            if (xpf_ok) {
                const ST* src0 = plane_at(srcp, bb + 1, c) + (size_t)opaque(tid) * 4;
#pragma unroll
                for (int k = 0; k < XPU; ++k) load4(src0 + (size_t)k * XWV * XRPK * 4, xpf[k]);
            } else {
                // (defined on every path: no value of these registers lives
                // through the next plane)
#pragma unroll
                for (int k = 0; k < XPU; ++k)
#pragma unroll
                    for (int i = 0; i < 4; ++i) xpf[k][i] = 0.f;
            }
        }


        // ---------------- phase 4b: x bands of levels >= 4 (backward) ----------------
        if constexpr (BWD) {
            if (Lm >= 3) {
                lds_barrier();  // band 0 of level 3 (x) written in phase 4a
                // every wave is done with the x plane: the next one lands meanwhile
                if (XDL && bb + g.NP() < b_end) dl_issue(auxp, g.xp_off(), g.xp_S(), 0, 0, bb + g.NP(), c, b_end);
                for (int i = 4; i <= Lm; ++i) {
                    const int hi = g.Hq() >> i, wi = g.Wq() >> i, wp = g.Wq() >> (i - 1);
                    const int pi = hi * wi;
                    const FastDiv dpi = make_div(pi), dwi = make_div(wi);
                    for (int e = tid; e < g.NP() * pi; e += nthr) {
                        const int s2 = fdiv(e, dpi), m = e - s2 * pi;
                        if (bb + s2 >= b_end) continue;
                        float* Sl = lds + s2 * g.slot();
                        const float* LL = Sl + g.xb_off(i - 1);
                        const int jy = fdiv(m, dwi), jx = m - jy * wi;
                        const int o = 2 * jy * wp + 2 * jx;
                        float r[4];
                        haar4(LL[o], LL[o + 1], LL[o + wp], LL[o + wp + 1], r);
                        float* XB = Sl + g.xb_off(i);
#pragma unroll
                        for (int u = 0; u < 4; ++u) XB[u * pi + m] = r[u];
                    }
                    lds_barrier();
                }
                if (tail && pok && qok[0] && qpb[0] == 0 && t == 0) {
                    const float rho = S[g.b_off(Lm) + R * g.b_S(Lm) + R];
                    tailc = fmaf(rho, S[g.xb_off(Lm)], tailc);
                }
            }
        }

        // ---------------- phase 4c: levels >= 3, flat (correlations) ----------------
        for (int i = 3; i <= Lm; ++i) {
            const int hi = g.Hq() >> i, wi = g.Wq() >> i, Si = g.b_S(i), bs = g.b_bs(i);
            if constexpr (BWD) {
                // C_i^du[ky][kx] = sum_m X[m] G[m - (ky - R, kx - R)] (G with its zero
                // halo): this role takes kernel row dky and its band rows; a chunk of
                // 4 X values and 4 + 2R values of one G row serve all K columns.
                // (the role is decoded here from an opaque copy of tid, so none
                // of it is held in registers through the rest of the plane)
                const int drl = opaque(tid);
                const int du4 = drl & 3, dky4 = (drl >> 2) % K, dsb4 = (drl >> 2) / K;
                if (drl < droles) {
                    float cv[K];
#pragma unroll
                    for (int kx = 0; kx < K; ++kx) cv[kx] = 0.f;
                    for (int s2 = 0; s2 < g.NP(); ++s2) {
                        if (bb + s2 >= b_end) break;
                        const float* Sl = lds + s2 * g.slot();
                        for (int my = dsb4; my < hi; my += g.dsub()) {
                            const float* XR = Sl + g.xb_off(i) + du4 * hi * wi + my * wi;
                            const float* GR = Sl + g.b_off(i) + du4 * bs + (my - dky4 + 2 * R) * Si;
#pragma unroll
                            for (int mx0 = 0; mx0 < wi; mx0 += 4) {
                                float xv[4], gv[4 + 2 * R];
#pragma unroll
                                for (int q = 0; q < 4; ++q) xv[q] = (mx0 + q < wi) ? XR[mx0 + q] : 0.f;
#pragma unroll
                                for (int q = 0; q < 4 + 2 * R; ++q)
                                    gv[q] = (mx0 + q < wi + 2 * R) ? GR[mx0 + q] : 0.f;
#pragma unroll
                                for (int kx = 0; kx < K; ++kx)
#pragma unroll
                                    for (int q = 0; q < 4; ++q) cv[kx] = fmaf(xv[q], gv[q + 2 * R - kx], cv[kx]);
                            }
                        }
                    }
#pragma unroll
                    for (int q = 0; q < ND; ++q)
                        if (q == i - 3)
#pragma unroll
                            for (int kx = 0; kx < K; ++kx) cdeep[q][kx] += cv[kx];
                }
            }
        }
        lds_barrier();
        if (XDL && Lm < 3 && bb + g.NP() < b_end) dl_issue(auxp, g.xp_off(), g.xp_S(), 0, 0, bb + g.NP(), c, b_end);

        // ---------------- phase 4d: levels 1, 2 results in place ----------------
#pragma unroll
        for (int s = 0; s < BPQ; ++s) {
            if (!(pok && qok[s]) || Lm < 1) continue;
            const int qy = qyv[s], qx = qxv[s];
            float* B1 = S + g.b_off(1) + t * g.b_bs(1);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) B1[(4 * qy + i + R) * g.b_S(1) + 4 * qx + j + R] = y1[s][i][j];
            if (Lm >= 2) {
                float* B2 = S + g.b_off(2) + t * g.b_bs(2);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) B2[(2 * qy + i + R) * g.b_S(2) + 2 * qx + j + R] = y2[s][i][j];
            }
        }
        lds_barrier();

        // ---------------- phase 6: closed-form synthesis fused with the store ----------------
        // Every level >= 2 contributes to this lane's 4x4 block through a single
        // position per level (the block is 2^i-aligned for i <= 2 and the quad's
        // block for i = 3 ...), with signs given by the bits of the block's
        // level-(i-1) coordinate; level 1 adds one 2x2 butterfly per position.
#pragma unroll
        for (int s = 0; s < BPQ; ++s) {
            const bool sok = pok && qok[s];
            if (!BST && !sok) continue;
            const int qy = qyv[s], qx = qxv[s];
            const int py0 = 8 * qy + 4 * sy, px0 = 8 * qx + 4 * sx;
            if (sok) {
                const float bias = wbase[KK];
                float z[4][4];
                if (Lm >= 1) {
                    // levels Lm..3: v = Z_3 at this lane's level-2 position
                    float v = 0.f;
                    for (int i = Lm; i >= 3; --i) {
                        const int wi = g.Wq() >> i, pi = (g.Hq() >> i) * wi;
                        const int jy = py0 >> i, jx = px0 >> i;
                        const int by = (py0 >> (i - 1)) & 1, bx = (px0 >> (i - 1)) & 1;
                        const float* Y = S + g.yd_off(i) + jy * wi + jx;
                        float T0 = Y[0] + v;
                        if (i == Lm && tail && jy == 0 && jx == 0) T0 += S[g.tail_off()];
                        const float sxb = bx ? -1.f : 1.f, syb = by ? -1.f : 1.f;
                        v = T0 + sxb * Y[pi] + syb * Y[2 * pi] + (sxb * syb) * Y[3 * pi];
                    }
                    float z2[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
                    if (Lm >= 2) {
                        const float* B2 = S + g.b_off(2) + (py0 / 4 + R) * g.b_S(2) + px0 / 4 + R;
                        const int bs2 = g.b_bs(2);
                        float T0 = B2[0] + v;
                        if (Lm == 2 && tail && py0 == 0 && px0 == 0) T0 += S[g.tail_off()];
                        float r[4];
                        haar4(T0, B2[bs2], B2[2 * bs2], B2[3 * bs2], r);
                        z2[0][0] = r[0]; z2[0][1] = r[1]; z2[1][0] = r[2]; z2[1][1] = r[3];
                    }
                    const float* B1 = S + g.b_off(1);
                    const int S1 = g.b_S(1), bs1 = g.b_bs(1);
#pragma unroll
                    for (int dy = 0; dy < 2; ++dy)
#pragma unroll
                        for (int dx = 0; dx < 2; ++dx) {
                            const int jy = py0 / 2 + dy, jx = px0 / 2 + dx;
                            const int o = (jy + R) * S1 + jx + R;
                            float T0 = B1[o] + bias + z2[dy][dx];
                            if (Lm == 1 && tail && jy == 0 && jx == 0) T0 += S[g.tail_off()];
                            float r[4];
                            haar4(T0, B1[bs1 + o], B1[2 * bs1 + o], B1[3 * bs1 + o], r);
                            z[2 * dy][2 * dx] = r[0];
                            z[2 * dy][2 * dx + 1] = r[1];
                            z[2 * dy + 1][2 * dx] = r[2];
                            z[2 * dy + 1][2 * dx + 1] = r[3];
                        }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j) z[i][j] = bias;
                    if (tail && py0 == 0 && px0 == 0) z[0][0] += S[g.tail_off()];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[s][i][j] = fmaf(wbase[KK + 1], acc[s][i][j], z[i][j]);
            }
            if constexpr (BST) {
                // One resource over the workgroup's NP planes of channel c
                // (uniform, so no loop over distinct descriptors); a lane's
                // plane starts slot * C planes in.  Rows outside the plane, and
                // blocks or planes that do not exist, get an offset past the
                // range: dropped.
                constexpr int EB = (int)sizeof(ST);
                const rsrc_t ro = make_rsrc(dstp + (size_t)bb * cplane + (size_t)c * plane_sz,
                                            (uint32_t)((g.NP() - 1) * cplane + aH * aW) * (uint32_t)EB);
                const int soff = (g.NP() == 1 ? 0 : slot * cplane) * EB;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool rok = sok && py0 + i < aH && px0 < aW;
                    // (opaque: one store per row, not a branch per side of the select)
                    const int off = opaque(rok ? soff + ((py0 + i) * aW + px0) * EB : kOutOfRange);
                    bstore4(ro, off, acc[s][i], (ST*)nullptr);
                }
            } else {
                ST* op = dstp + poff + (size_t)opaque(py0 * aW + px0) * ps;
                if constexpr (VEC) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (py0 + i < aH && px0 < aW) gstore4<NHWC>(op + (size_t)i * aW * ps, ps, acc[s][i]);
                } else if (NHWC) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            if (py0 + i < aH && px0 + j < aW) from_f32(op[((size_t)i * aW + j) * ps], acc[s][i][j]);
                } else if ((aW & 1) == 0) {
                    // even width: pixel pairs
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int p = 0; p < 2; ++p)
                            if (py0 + i < aH && px0 + 2 * p < aW)
                                store2(op + i * aW + 2 * p, acc[s][i][2 * p], acc[s][i][2 * p + 1]);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            if (py0 + i < aH && px0 + j < aW) from_f32(op[i * aW + j], acc[s][i][j]);
                }
            }
        }
    }
    if constexpr (XSEG) {
        // every wave is past this segment's last phase 2 and 4b, so the copy
        // targets are free: the next segment's first planes land during the
        // reduction and set-up
        if (seg == 0 && q1 > (long)(c + 1) * a.B) {
            const int bend_next = (int)(min(q1, (long)(c + 2) * a.B) - (long)(c + 1) * a.B);
            if constexpr (XDL) dl_issue(auxp, g.xp_off(), g.xp_S(), 0, 0, 0, c + 1, bend_next);
            if constexpr (!SDL) dl_issue(srcp, g.a0_off(), g.a0_S(), R, R, 0, c + 1, bend_next);
            if constexpr (SDL) stage_issue(0, c + 1, bend_next);
        }
    }
    if constexpr (BWD) {
        // ---------------- reduction of the correlation accumulators ----------------
        // Row sums by DPP (four steps per accumulator, all independent), then
        // one partial per 16-lane row in LDS, summed in a fixed order.
        lds_barrier();
        float* red = lds + g.red_off();
        const int nw = nthr >> 6, lane = tid & 63;
        const int NR = nw * 4, row = (tid >> 6) * 4 + ((lane >> 4) & 3);
        // [C_0: NR x KK][C_1: NR x 4 x KK][C_2: NR x 4 x KK][sum g: NR][tail: NR][deep]
        float* r0 = red;
        float* r1 = r0 + NR * KK;
        float* r2 = r1 + NR * 4 * KK;
        float* rs = r2 + NR * 4 * KK;
        float* rt = rs + NR;
        float* dred = rt + NR;   // deep: [q][role]
#pragma unroll
        for (int q = 0; q < KK; ++q) {
            corr0[q] = row_sum(corr0[q]);
            corr1[q] = row_sum_by_residue(corr1[q]);
            corr2[q] = row_sum_by_residue(corr2[q]);
        }
        sumg = row_sum(sumg);
        tailc = row_sum(tailc);
        // un-rotate: accumulator q holds tap KK-1-q; band u = lane mod 4
        if ((lane & 15) >= 12) {
            const int u = lane & 3;
#pragma unroll
            for (int q = 0; q < KK; ++q) {
                r1[(row * 4 + u) * KK + (KK - 1 - q)] = corr1[q];
                r2[(row * 4 + u) * KK + (KK - 1 - q)] = corr2[q];
            }
            if (u == 3) {
#pragma unroll
                for (int q = 0; q < KK; ++q) r0[row * KK + (KK - 1 - q)] = flush0 ? c0acc[row * KK + q] : corr0[q];
                rs[row] = sumg;
                rt[row] = tailc;
            }
        }
        if (dactive) {
#pragma unroll
            for (int q = 0; q < ND; ++q)
                if (q + 3 <= Lm)
#pragma unroll
                    for (int kx = 0; kx < K; ++kx) dred[(q * droles + drole) * K + kx] = cdeep[q][kx];
        }
        lds_barrier();
        float* rec = a.partials + (a.units ? (size_t)unit : (size_t)blockIdx.x * 2 + seg) * g.P();
        for (int e = tid; e < g.P(); e += nthr) {
            float v = 0.f;
            if (e < KK) {
                for (int i = 0; i < NR; ++i) v += r0[i * KK + e];
            } else if (e < KK + 4 * KK * Lm) {
                const int lvl = (e - KK) / (4 * KK) + 1;
                const int rem = (e - KK) - (lvl - 1) * 4 * KK;
                if (lvl <= 2) {
                    const float* rl = lvl == 1 ? r1 : r2;
                    const int u = rem / KK, tap = rem - u * KK;
                    for (int i = 0; i < NR; ++i) v += rl[(i * 4 + u) * KK + tap];
                } else {
                    const int u = rem / KK, tap = rem - u * KK, ky = tap / K, kx = tap - ky * K;
                    for (int sb = 0; sb < g.dsub(); ++sb)
                        v += dred[((lvl - 3) * droles + (sb * K + ky) * 4 + u) * K + kx];
                }
            } else if (e == g.P() - 2) {
                for (int i = 0; i < NR; ++i) v += rs[i];
            } else {
                for (int i = 0; i < NR; ++i) v += rt[i];
            }
            rec[e] = v;
        }
    }
    }  // channel segments
}

template <int K, typename ST, bool BWD, int BPQ, bool VEC, class G>
hipError_t launch_t(const FusedArgs& a, int nthr, size_t lds, int grid, hipStream_t st) {
    auto kern = wtc_fused_kernel<K, ST, BWD, BPQ, VEC, G>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(nthr), lds, st, a);
    return hipGetLastError();
}

// Runtime-geometry kernel of one activation layout (NH: channels-last).
template <int K, bool NH>
hipError_t launch_rt_l(const FusedArgs& a, int dtype, int bwd, int bpq, int nthr, size_t lds, int grid,
                       hipStream_t st) {
    if (a.Lm > kMaxLm) return hipErrorInvalidValue;
    const bool shallow = a.Lm <= 3;
    if (a.lay.dl) {
        if (!a.vec || bpq != 1 || a.NP != 1 || (dtype == WTC_BF16 && !bwd)) return hipErrorInvalidValue;
        if (!bwd) return launch_t<K, float, false, 1, true, RtGeom<true, kMaxLm, NH>>(a, nthr, lds, grid, st);
        if (dtype == WTC_BF16) {
            if constexpr (NH) {
                return hipErrorInvalidValue;   // channels-last bf16 planes are staged through registers
            } else {
                if (shallow) return launch_t<K, bf16_t, true, 1, true, RtGeom<true, 3>>(a, nthr, lds, grid, st);
                return launch_t<K, bf16_t, true, 1, true, RtGeom<true, kMaxLm>>(a, nthr, lds, grid, st);
            }
        }
        if (shallow) return launch_t<K, float, true, 1, true, RtGeom<true, 3, NH>>(a, nthr, lds, grid, st);
        return launch_t<K, float, true, 1, true, RtGeom<true, kMaxLm, NH>>(a, nthr, lds, grid, st);
    }
#define WTC_RT(ST_, BWD_, LMX_)                                                                           \
    do {                                                                                                 \
        using G_ = RtGeom<false, LMX_, NH>;                                                              \
        if (a.vec) {                                                                                     \
            if (bpq == 1) return launch_t<K, ST_, BWD_, 1, true, G_>(a, nthr, lds, grid, st);            \
            return launch_t<K, ST_, BWD_, 2, true, G_>(a, nthr, lds, grid, st);                          \
        }                                                                                                \
        if (bpq == 1) return launch_t<K, ST_, BWD_, 1, false, G_>(a, nthr, lds, grid, st);               \
        return launch_t<K, ST_, BWD_, 2, false, G_>(a, nthr, lds, grid, st);                             \
    } while (0)
    if (dtype == WTC_BF16) {
        if (bwd && shallow) WTC_RT(bf16_t, true, 3);
        if (bwd) WTC_RT(bf16_t, true, kMaxLm);
        WTC_RT(bf16_t, false, kMaxLm);
    }
    if (bwd && shallow) WTC_RT(float, true, 3);
    if (bwd) WTC_RT(float, true, kMaxLm);
    WTC_RT(float, false, kMaxLm);
#undef WTC_RT
}

// Runtime-geometry kernel for any plane the LDS pipeline holds.  Plans of
// layout mode 1 copy their planes by DMA (4-pixel rows, one block per quad,
// one plane per workgroup; fp32, or a bf16 backward of NCHW tensors);
// everything else is staged through registers.  The backward comes in two
// deep-level classes (Lm <= 3, any Lm).  NCHW and channels-last tensors.
template <int K>
hipError_t launch_rt(const FusedArgs& a, int dtype, int bwd, int bpq, int nthr, size_t lds, int grid,
                     hipStream_t st) {
    return a.nhwc ? launch_rt_l<K, true>(a, dtype, bwd, bpq, nthr, lds, grid, st)
                  : launch_rt_l<K, false>(a, dtype, bwd, bpq, nthr, lds, grid, st);
}

}  // namespace fused_detail
}  // namespace wtc

namespace wtc {
namespace fused_detail {

// Launch the fixed-geometry instantiation if the plan matches it exactly.
// A whole-plane instance (WH) matches only planes of exactly HQ x WQ pixels,
// one with a plane size (PH x PW > 0) only planes of that size.
template <int K, typename ST, bool BWD, int BPQ, bool VEC, int HQ, int WQ, int LM, int EARLY, int NPV,
          int NTHR, int BOVL, int MODE = 0, bool NH = false, bool WH = false, int PH = 0, int PW = 0>
bool try_static(const FusedArgs& a, int bpq, int nthr, size_t lds, int grid, hipStream_t st,
                hipError_t* err) {
    if (a.Hq != HQ || a.Wq != WQ || a.Lm != LM || a.lay.early_lv != EARLY || a.NP != NPV ||
        nthr != NTHR || bpq != BPQ || (a.vec != 0) != VEC || a.lay.bovl != BOVL || a.lay.mode != MODE ||
        (a.nhwc != 0) != NH || (WH && (a.H != HQ || a.W != WQ)) || (PH > 0 && (a.H != PH || a.W != PW)))
        return false;
    *err = launch_t<K, ST, BWD, BPQ, VEC,
                    CtGeom<K, HQ, WQ, LM, EARLY, NPV, NTHR, BWD, BOVL, MODE, (int)sizeof(ST), NH, WH, PH, PW>>(
        a, nthr, lds, grid, st);
    return true;
}

}  // namespace fused_detail
}  // namespace wtc
