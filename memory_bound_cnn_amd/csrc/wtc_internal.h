// Internal declarations shared by the host dispatcher (wtconv_api.cpp) and the
// HIP kernels (wtconv_fused.hip, wtconv_unfused.hip).  Not part of the ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/wtconv.h"

namespace wtc {

constexpr int kMaxLm = 7;   // levels evaluated on a grid larger than 1x1 (planes <= 128)
constexpr int kMaxK = 7;

// Arguments of the fused plane-pipeline kernel.  All offsets are in floats.
// One workgroup owns one channel c and a chunk of batch entries; it walks the
// chunk NP planes at a time, each plane held in an LDS "slot".
struct FusedArgs {
    const void* src;   // forward: x;  backward: g  (the tensor that is convolved)
    const void* aux;   // backward: x (correlation partner); forward: unused
    const float* w0;
    const float* s0;
    const float* b0;
    const float* wl;
    const float* sl;
    void* dst;         // forward: out;  backward: dx
    float* partials;   // backward: [nchunk][C][P] per-workgroup correlation sums

    int B, C, H, W;
    int L;             // levels requested
    int Lm;            // levels on grids larger than 1x1; levels Lm+1..L are 1x1 ("tail")
    int Hq, Wq;        // zero-extended plane: multiples of max(8, 2^Lm)
    int bpc;           // batch entries per workgroup
    int NP;            // plane slots per workgroup iteration
    int qpp, nqx;      // 8x8 pixel blocks ("quad blocks") per plane, per plane row
    int vec;           // W % 4 == 0: 4-pixel vector global accesses
    int overlap;       // level>=2 arrays overlap the level-0 array (rings re-zeroed)
    int slot_stride;

    int a0_off, a0_S, a0_rows;                 // level-0 plane with halo k/2
    int b_off[kMaxLm + 1], b_S[kMaxLm + 1];    // level-i raw bands with halo k/2
    int b_bs[kMaxLm + 1], b_rows[kMaxLm + 1];  // band stride, rows (incl. halo)
    int z_off[kMaxLm + 1];                     // Z_i (i >= 2) on the level i-1 grid
    int yd_off[kMaxLm + 1];                    // Y'_i (i >= 3), [4][Hq_i][Wq_i]
    int xl2_off;                               // backward: LL_2 of x, [Hq_2][Wq_2]
    int xb_off[kMaxLm + 1];                    // backward: bands of x (i >= 3), [4][Hq_i][Wq_i]
    int tail_off;                              // per slot: tail term rho * kappa
    int wts_off;                               // folded weights (per workgroup)
    int red_off;                               // reduction scratch (backward)
    int dsub;                                  // position subsets of the deep-level correlation
    int P;                                     // partial record length (floats)
};

// Partial record of one (chunk, channel): [C_0 (k*k)] [levels 1..Lm: 4 bands x k*k]
// [sum g] [tail correlation]; all correlations in natural tap order.
inline int partial_len(int k, int Lm) { return k * k * (1 + 4 * Lm) + 2; }

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
    int C, L, Lm, k, nchunk, P;
};

// Launchers (defined in the .hip files); return a hipError_t as int.
int launch_fused(const FusedArgs& a, int k, int dtype, int bwd, int bpq, int nthr,
                 size_t lds_bytes, int grid, void* stream);
int launch_finalize(const FinalizeArgs& f, void* stream);

// ---------------------------------------------------------------------------
// Unfused (level-by-level) baseline
// ---------------------------------------------------------------------------
struct UnfusedPlan {
    // workspace offsets in bytes
    size_t ll_off[kMaxLm + 2];   // forward: raw LL/band tensors per level [B,4C,h_i,w_i] (fp32)
    size_t y_off[kMaxLm + 2];    // Y_i (scaled conv outputs) [B,4C,h_i,w_i]
    size_t z_off[kMaxLm + 2];    // Z_i [B,C,h_{i-1},w_{i-1}]
    size_t dt_off[kMaxLm + 2];   // backward: analysis of dZ per level
    size_t ds_off[kMaxLm + 2];   // backward: dS per level
    size_t part_off;             // weight-gradient partial sums
    size_t base_off;             // forward: base conv output
    size_t total;
    int h[kMaxLm + 2], w[kMaxLm + 2];
    int nblk;                    // reduction partial blocks per channel
};

int unfused_plan(const wtc_desc* d, int bwd, UnfusedPlan* p);
int unfused_forward(const wtc_desc* d, const UnfusedPlan& p, const void* x, const float* w0,
                    const float* s0, const float* b0, const float* wl, const float* sl, void* out,
                    char* ws, void* stream);
int unfused_backward(const wtc_desc* d, const UnfusedPlan& p, const void* x, const void* g,
                     const float* w0, const float* s0, const float* wl, const float* sl, void* dx,
                     float* dw0, float* ds0, float* db0, float* dwl, float* dsl, char* ws,
                     void* stream);

}  // namespace wtc
