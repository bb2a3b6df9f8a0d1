// Internal declarations shared by the host dispatcher (wtconv_api.cpp) and the
// HIP kernels (wtconv_fused.hip, wtconv_unfused.hip).  Not part of the ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/wtconv.h"

namespace wtc {

constexpr int kMaxLm = 7;   // levels evaluated on a grid larger than 1x1 (planes <= 128)
constexpr int kMaxK = 7;       // largest kernel size of the fused and the unrolled kernels
constexpr int kMaxKAny = 31;   // largest kernel size at all (runtime-size level-by-level kernels)

// LDS layout of one plane slot (all offsets and sizes in floats).
// Without band overlap: [level-1 .. level-early bands][level-0 plane | later
// arrays][tail]; arrays first written after the level-0 phase (deeper bands,
// deep conv results, x bands) may overlap the level-0 plane ("overlap").
// With band overlap from level f ("bovl" = f >= 1): [bands of levels < f][bands
// of levels >= f and the later arrays, over the level-0 plane][tail]; the early
// bands of levels >= f are then written only after the whole workgroup is done
// reading the level-0 plane, and their rings are re-zeroed per plane.
// Layout modes: 0 = later arrays may overlap the level-0 plane (when they fit
// in it); 2 = nothing overlaps it (no per-plane ring re-zeroing); 1 = direct
// loads ("dl"): nothing overlaps it, so the next plane can be copied into the
// slot by DMA while the current one is still being processed.  fp32 planes
// land in the level-0 plane itself and the backward adds a plane of x (row
// stride Wq + 4, no halo); bf16 planes land in a staging area of raw 16-bit
// pixels (H*W/2 words) and are widened into the level-0 plane per plane.
struct Layout {
    int early_lv;      // levels analysed in registers during the level-0 phase (<= 3)
    int overlap;       // later arrays overlap the level-0 plane (rings re-zeroed per plane)
    int bovl;          // first level whose bands overlap the level-0 plane (0: none)
    int slot;          // floats per plane slot
    int a0_off, a0_S, a0_rows;                 // level-0 plane with halo k/2
    int b_off[kMaxLm + 1], b_S[kMaxLm + 1];    // level-i raw bands with halo k/2
    int b_bs[kMaxLm + 1], b_rows[kMaxLm + 1];  // band stride, rows (incl. halo)
    int yd_off[kMaxLm + 1];                    // Y'_i (i >= 3), [4][Hq_i][Wq_i]
    int xb_off[kMaxLm + 1];                    // backward: bands of x (i >= 3), [4][Hq_i][Wq_i]
    int tail_off;                              // tail term rho * kappa
    int mode;                                  // 0, 1 (direct loads) or 2 (no overlap)
    int dl;                                    // mode == 1
    int xp_off, xp_S;                          // dl fp32 backward: x plane [Hq][xp_S]
    int st_off;                                // dl bf16: staging of the raw plane (H*W/2 words)
};

constexpr int lay_round_up(int v, int m) { return (v + m - 1) / m * m; }

// The one definition of the slot layout, evaluated on the host for the
// runtime-geometry kernel and at compile time for the fixed-geometry ones.
// Floats of the backward reduction scratch: per 16-lane row of the workgroup
// C_0 (k^2), C_1 and C_2 (4 k^2 each), sum g and the tail term; then the deep
// levels' output-stationary partials (levels 3..Lm, 4 k dsub roles of k).
constexpr int red_len(int nthr, int k, int Lm, int dsub) {
    return (nthr / 16) * (9 * k * k + 2) + (Lm > 2 ? Lm - 2 : 0) * 4 * k * dsub * k;
}

constexpr Layout make_layout(int k, int Hq, int Wq, int Lm, int early_req, bool bwd, int bovl, int mode = 0,
                             int esize = 4) {
    Layout L{};
    const int R = k / 2;
    L.early_lv = Lm < early_req ? Lm : early_req;
    L.mode = mode;
    const bool dl = mode == 1;
    L.dl = dl ? 1 : 0;
    if (mode != 0) bovl = 0;
    int off = 0;
    for (int i = 1; i <= Lm; ++i) {
        L.b_rows[i] = (Hq >> i) + 2 * R;
        L.b_S[i] = lay_round_up((Wq >> i) + 2 * R, 4);
        // band stride = 8 (mod 32) floats: the four subbands start in different LDS banks
        L.b_bs[i] = lay_round_up(L.b_rows[i] * L.b_S[i], 32) + 8;
    }
    if (bovl >= 1 && bovl <= Lm) {
        L.bovl = bovl;
        L.overlap = 1;
        for (int i = 1; i < bovl; ++i) {
            L.b_off[i] = off;
            off += lay_round_up(4 * L.b_bs[i], 4);
        }
        const int base = off;
        for (int i = bovl; i <= Lm; ++i) {
            L.b_off[i] = off;
            off += lay_round_up(4 * L.b_bs[i], 4);
        }
        for (int i = 3; i <= Lm; ++i) {
            L.yd_off[i] = off;
            off += lay_round_up(4 * (Hq >> i) * (Wq >> i), 4);
            if (bwd) {
                L.xb_off[i] = off;
                off += lay_round_up(4 * (Hq >> i) * (Wq >> i), 4);
            }
        }
        L.a0_off = base;
        L.a0_rows = Hq + 2 * R;
        L.a0_S = lay_round_up(Wq + 2 * R, 4);
        const int a0_size = lay_round_up(L.a0_rows * L.a0_S, 4);
        L.tail_off = off > base + a0_size ? off : base + a0_size;
        L.slot = lay_round_up(L.tail_off + 4, 4);
        return L;
    }
    for (int i = 1; i <= L.early_lv; ++i) {
        L.b_off[i] = off;
        off += lay_round_up(4 * L.b_bs[i], 4);
    }
    L.a0_rows = Hq + 2 * R;
    L.a0_S = lay_round_up(Wq + 2 * R, 4);
    const int a0_size = lay_round_up(L.a0_rows * L.a0_S, 4);
    int r2 = 0;
    int rel_b[kMaxLm + 1] = {}, rel_y[kMaxLm + 1] = {}, rel_x[kMaxLm + 1] = {};
    for (int i = L.early_lv + 1; i <= Lm; ++i) {
        rel_b[i] = r2;
        r2 += lay_round_up(4 * L.b_bs[i], 4);
    }
    for (int i = 3; i <= Lm; ++i) {
        rel_y[i] = r2;
        r2 += lay_round_up(4 * (Hq >> i) * (Wq >> i), 4);
        if (bwd) {
            rel_x[i] = r2;
            r2 += lay_round_up(4 * (Hq >> i) * (Wq >> i), 4);
        }
    }
    L.a0_off = off;
    int r2_base = off;
    // mode 2 names a layout of its own only where mode 0 would overlap
    if (mode == 2 && !(r2 > 0 && r2 <= a0_size)) L.mode = mode = 0;
    if (r2 <= a0_size && mode == 0) {
        L.overlap = r2 > 0 ? 1 : 0;
        off += a0_size;
    } else {
        L.overlap = 0;
        off += a0_size;
        r2_base = off;
        off += r2;
    }
    for (int i = L.early_lv + 1; i <= Lm; ++i) L.b_off[i] = r2_base + rel_b[i];
    for (int i = 3; i <= Lm; ++i) {
        L.yd_off[i] = r2_base + rel_y[i];
        if (bwd) L.xb_off[i] = r2_base + rel_x[i];
    }
    if (dl && esize == 2) {
        L.st_off = lay_round_up(off, 4);
        off = L.st_off + lay_round_up(Hq * Wq / 2, 4);
    }
    if (dl && bwd && esize == 4) {
        // x rows 16-byte aligned; stride = 4 (mod 8) floats keeps the 4x4 block
        // reads of two vertically adjacent lanes in different banks
        L.xp_off = lay_round_up(off, 4);
        L.xp_S = lay_round_up(Wq, 4) % 8 == 0 ? lay_round_up(Wq, 4) + 4 : lay_round_up(Wq, 4);
        off = L.xp_off + lay_round_up(Hq * L.xp_S, 4);
    }
    L.tail_off = off;
    off += 4;
    L.slot = lay_round_up(off, 4);
    return L;
}

// Arguments of the fused plane-pipeline kernel.  All offsets are in floats.
// A workgroup walks a contiguous range of planes in channel-major order, NP
// planes at a time, each plane held in an LDS "slot".
struct FusedArgs {
    const void* src;   // forward: x;  backward: g  (the tensor that is convolved)
    const void* aux;   // backward: x (correlation partner); forward: unused
    const float* w0;
    const float* s0;
    const float* b0;
    const float* wl;
    const float* sl;
    void* dst;         // forward: out;  backward: dx
    float* partials;   // backward: [grid][2][P] per-(workgroup, channel segment) sums

    int B, C, H, W;
    int L;             // levels requested
    int Lm;            // levels on grids larger than 1x1; levels Lm+1..L are 1x1 ("tail")
    int Hq, Wq;        // zero-extended plane: multiples of max(8, 2^Lm)
    int ppw;           // planes per workgroup (channel-major range, <= B)
    int NP;            // plane slots per workgroup iteration
    int qpp, nqx;      // 8x8 pixel blocks ("quad blocks") per plane, per plane row
    int vec;           // W % 4 == 0: 4-pixel vector global accesses
    int pf_on;         // prefetch the next planes into registers
    int nobase;        // skip the base conv: the LL problem of a peeled plane (its scale and bias are 0)
    int units;         // 1: one (batch chunk, channel) unit per workgroup, dealt to the XCDs in
                       //    contiguous ranges; records [chunk][channel] (finalize in chunk mode)
    int nchunk;        // units: batch chunks per channel (of ppw entries)
    int nhwc;          // x, g, out, dx are channels-last [B, H, W, C] (the kernel's kNHWC)
    Layout lay;
    int wts_off;       // folded weights (per workgroup)
    int red_off;       // reduction scratch (backward)
    int dsub;          // band-row subsets of the deep-level (>= 3) correlation roles
    int P;             // partial record length (floats)
};

// Floats of the per-row base-correlation accumulators (after the weights) of
// the backward kernel with two blocks per quad and three levels or more: it
// adds each plane's C_0 into them (one 16-lane row per slot set) instead of
// holding 25 accumulators per lane across the plane, which spilled.
constexpr int flush_len(bool bwd, int bpq, int nthr, int k, int Lm) {
    return (bwd && bpq > 1 && Lm >= 3) ? (nthr / 16) * k * k : 0;
}

// Waves per SIMD the fused kernels are compiled for (register budget 512 /
// waves): 3 forward, 2 backward or with two blocks per quad; the
// fixed-geometry kernels without wavelet levels (a plain depthwise conv) are
// small enough for 4 forward and 3 backward.
constexpr int fused_waves_per_simd(bool bwd, int bpq, bool no_levels_static) {
    return no_levels_static ? (bwd ? 3 : 4) : ((bwd || bpq > 1) ? 2 : 3);
}

// Next-plane prefetch capacity in floats per thread: the forward kernel with
// two blocks per quad (large planes) has the registers for a whole plane.
constexpr int pf_capacity(bool bwd, int bpq) { return (!bwd && bpq > 1) ? 32 : 16; }

// Partial record of one (workgroup, channel segment): [C_0 (k*k)] [levels 1..Lm: 4 bands x k*k]
// [sum g] [tail correlation]; all correlations in natural tap order.
constexpr int partial_len(int k, int Lm) { return k * k * (1 + 4 * Lm) + 2; }

struct FinalizeArgs {
    const float* partials;
    const float* w0;
    const float* s0;
    const float* wl;
    const float* sl;
    float* dw0;
    float* ds0;
    float* db0;
    float* dwl;
    float* dsl;
    int C, B, L, Lm, k, ppw, P;
    int chunks;   // > 0: records laid out [chunk][channel] (small-plane kernel)
};

// Launchers (defined in the .hip files); return a hipError_t as int.
int launch_fused(const FusedArgs& a, int k, int dtype, int bwd, int bpq, int nthr,
                 size_t lds_bytes, int grid, void* stream);
int launch_finalize(const FinalizeArgs& f, void* stream);
// Register-resident kernel for planes of at most 8 x 8 (k = 5, 1 <= L = Lm <= 2):
// one 64-lane workgroup per 16 consecutive channels and ppw batch entries
// (grid = ceil(C / 16) x ceil(B / ppw)); backward records [chunk][channel].
int launch_tiny(const FusedArgs& a, int dtype, int bwd, int grid, void* stream);
// One plane per lane for 7 x 7 planes with one level (k = 5): one wave per 64
// batch entries of a channel (grid = C * ceil(B / 64)); backward records
// [chunk][channel] as the register-resident kernel's.
int launch_lane(const FusedArgs& a, int dtype, int bwd, int grid, void* stream);
constexpr bool lane_supported(int k, int H, int W, int L, int Lm) {
    return k == 5 && H == 7 && W == 7 && L == 1 && Lm == 1;
}
constexpr bool tiny_supported(int k, int Hq, int Wq, int L, int Lm) {
    return k == 5 && Hq == 8 && Wq == 8 && L == Lm && Lm >= 1 && Lm <= 2;
}

// ---------------------------------------------------------------------------
// Unfused (level-by-level) baseline
// ---------------------------------------------------------------------------
constexpr int kMaxUnfusedL = 30;   // levels the baseline accepts (grids stay 1x1 beyond log2 size)
// Large planes of the baseline (both sides >= kUnfusedBigSide) run 64 x 64
// tiles; its weight-gradient correlations aim at kUnfusedCorrTarget workgroups
// per launch.  The peeled top level runs kTopTile x kTopTile output tiles.
constexpr int kUnfusedBigTile = 64;
constexpr int kUnfusedBigSide = 48;
constexpr int kUnfusedCorrTarget = 2048;
constexpr int kTopTile = 64;
inline bool unfused_big_planes(int h, int w) { return h >= kUnfusedBigSide && w >= kUnfusedBigSide; }

struct UnfusedPlan {
    // workspace offsets in bytes, per level 1..L (float32 tensors)
    size_t s_off[kMaxUnfusedL + 1];    // S_i   [B, C, 4, h_i, w_i]  bands of x
    size_t y_off[kMaxUnfusedL + 1];    // Y_i (forward) / dS_i (backward), same shape
    size_t z_off[kMaxUnfusedL + 1];    // Z_i (forward) / dLL_{i-1} (backward) [B, C, h_{i-1}, w_{i-1}]
    size_t dt_off[kMaxUnfusedL + 1];   // backward: analysis of g, same shape as S_i
    size_t part_off;                   // backward: correlation partial sums
    size_t total;
    int h[kMaxUnfusedL + 1], w[kMaxUnfusedL + 1];
};

// workgroups per channel of the baseline's weight-gradient correlation
int unfused_corr_blocks(int nb, int nch, int h, int w);

// Peeled planes: the top level (level 1 and the base conv, fused over 64 x 64
// tiles) and the normalised level-1 LL band feeding the sub-problem.
int top_forward(const wtc_desc* d, const void* x, const float* w0, const float* s0, const float* b0,
                const float* wl, const float* sl, const float* zext, void* out, void* stream);
int top_ll(const wtc_desc* d, const void* x, float* ll, void* stream);
// Backward of the top level: dx, and per (batch entry, tile) partial
// correlation records of the base (part0: [B ntile][C][k^2 + 1], slot k^2 = sum g)
// and of level 1 (part1: [B ntile][4C][k^2 + 1]); top_records() floats of each.
size_t top_records(const wtc_desc* d);
int top_backward(const wtc_desc* d, const void* x, const void* g, const float* w0, const float* s0, const float* wl,
                 const float* sl, const float* dll, void* dx, float* part0, float* part1, void* stream);
// Chain rule of one level from correlation partials [nblk][nch][k^2 + 1]:
// dw = scale C, ds = sum W C, db = slot k^2 (if db)
int launch_corr_finalize(const float* part, int nch, int nblk, int k, const float* wt, const float* scale, float* dw,
                         float* ds, float* db, void* stream);
int unfused_plan(const wtc_desc* d, int bwd, UnfusedPlan* p);
// stage 0: the whole pipeline; 1: only the analysis cascades (into the
// workspace); 2: everything after them, with `zext` (may be null) added to the
// LL band of the deepest level in the synthesis -- the term of deeper levels
// computed elsewhere (forward: their output Z_{L+1}; backward: dLL_L).
int unfused_forward(const wtc_desc* d, const UnfusedPlan& p, const void* x, const float* w0,
                    const float* s0, const float* b0, const float* wl, const float* sl, void* out,
                    char* ws, void* stream, int stage = 0, const float* zext = nullptr);
int unfused_backward(const wtc_desc* d, const UnfusedPlan& p, const void* x, const void* g,
                     const float* w0, const float* s0, const float* wl, const float* sl, void* dx,
                     float* dw0, float* ds0, float* db0, float* dwl, float* dsl, char* ws,
                     void* stream, int stage = 0, const float* zext = nullptr);
int launch_fill_zero(float* p, int n, void* stream);
// The base level's weight-gradient correlation partials alone, by the
// level-by-level baseline's tile kernels: part[blk][c][k^2 + 1] (slot k^2 =
// sum of g), *nblk blocks; part holds unfused_corr_blocks(B, C, H, W) blocks.
int base_corr_partials(const wtc_desc* d, const void* x, const void* g, float* part, int* nblk, void* stream);
// The same correlation of bf16 planes (k <= 7, H, W <= 64) on the matrix
// cores: part[chunk][c][k^2 + 1] over nchunk batch chunks (slot k^2 unused).
int launch_corr0_mfma(const wtc_desc* d, const void* x, const void* g, float* part, int nchunk, void* stream);
// out[c][t] = sum over nblk blocks of part[blk][c][t] (t < kk; record length kk1), fixed order
int launch_corr_sum(const float* part, int C, int nblk, int kk1, int kk, float* out, void* stream);
// Argument checks of the backward entry points (descriptor, then pointers):
// WTC_OK or the status the entry point returns, before any HIP call.
int backward_check(const wtc_desc* d, const void* x, const void* g, const float* w0, const float* s0,
                   const float* wl, const float* sl, const void* dx, const float* dw0, const float* ds0,
                   const float* db0, const float* dwl, const float* dsl);
// [batch][rows][cols] -> [batch][cols][rows], elements of esize (4 or 2) bytes
int launch_transpose(const void* src, void* dst, int batch, int rows, int cols, int esize, void* stream);

}  // namespace wtc
