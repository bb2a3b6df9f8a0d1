// Host side of libwtconv: argument checks, launch planning, dispatch, and the
// analytic HBM-traffic model.  See include/wtconv.h for the contract.
#include <algorithm>
#include <cstring>

#include "wtc_internal.h"

namespace wtc {
namespace {

constexpr size_t kLdsLimit = 160 * 1024;       // gfx950 LDS per workgroup
constexpr int kComputeUnits = 256;             // MI355X

int ceil_log2(int v) {
    int l = 0;
    while ((1 << l) < v) ++l;
    return l;
}
int round_up(int v, int m) { return (v + m - 1) / m * m; }
int cdiv(int a, int b) { return (a + b - 1) / b; }

int check_desc(const wtc_desc* d) {
    if (!d) return WTC_EINVAL;
    if (d->B < 1 || d->C < 1 || d->H < 1 || d->W < 1 || d->L < 0) return WTC_EINVAL;
    if (d->k < 1 || d->k % 2 == 0) return WTC_EINVAL;
    if (d->dtype != WTC_FP32 && d->dtype != WTC_BF16) return WTC_EDTYPE;
    if (d->layout < 0 || d->layout > 2) return WTC_EDTYPE;
    if (d->layout != 0 && d->B > 65535) return WTC_ESHAPE;   // transpose grid
    return WTC_OK;
}

// NCHW twin of a descriptor (the compute paths are NCHW; layout 1 is adapted)
wtc_desc nchw_of(const wtc_desc* d) {
    wtc_desc n = *d;
    n.layout = 0;
    return n;
}

struct FusedPlan {
    FusedArgs a;
    int nthr, bpq, grid, nchunk;
    size_t lds;
    int tiny;   // 1: register-resident kernel for planes of at most 8 x 8; 2: one plane per lane (7 x 7)
    long nrec;  // backward partial records
};

int plan_fused(const wtc_desc* d, bool bwd, FusedPlan* p) {
    int st = check_desc(d);
    if (st != WTC_OK) return st;
    const int k = d->k, KK = k * k;
    if (k > kMaxK) return WTC_ESHAPE;
    FusedArgs& a = p->a;
    std::memset(&a, 0, sizeof(a));
    a.B = d->B; a.C = d->C; a.H = d->H; a.W = d->W; a.L = d->L;
    const int Lcap = ceil_log2(std::max(d->H, d->W));
    a.Lm = std::min(d->L, Lcap);
    if (a.Lm > kMaxLm) return WTC_ESHAPE;
    const int T = std::max(8, 1 << a.Lm);
    a.Hq = cdiv(d->H, T) * T;
    a.Wq = cdiv(d->W, T) * T;
    a.nqx = a.Wq / 8;
    a.qpp = (a.Hq / 8) * a.nqx;
    a.vec = (d->W % 4 == 0) ? 1 : 0;
    // channels-last tensors: the plane pipeline reads and writes them in place,
    // one (batch chunk, channel) unit per workgroup, the units of neighbouring
    // channels -- which share every cache line -- on one XCD at a time
    a.nhwc = d->layout != 0 ? 1 : 0;
    a.units = a.nhwc;
    p->tiny = 0;
    if (!a.nhwc && lane_supported(k, d->H, d->W, d->L, a.Lm)) {
        // one plane per lane, one wave per 64 batch entries of a channel
        p->tiny = 2;
        a.P = partial_len(k, a.Lm);
        a.ppw = 64;
        p->nchunk = (d->B + 63) / 64;
        p->grid = 8 * cdiv(d->C * p->nchunk, 8);   // XCD-aware unit order (8 XCDs)
        p->nrec = (long)p->nchunk * d->C;
        p->nthr = 64;
        p->bpq = 1;
        p->lds = 0;
        return WTC_OK;
    }
    const long esize = d->dtype == WTC_BF16 ? 2 : 4;
    if (!a.nhwc && tiny_supported(k, a.Hq, a.Wq, d->L, a.Lm) &&
        ((long)d->B + 16) * d->C * d->H * d->W * esize < (1L << 31)) {   // 32-bit buffer offsets
        // one wave per workgroup: 16 consecutive channels, ppw batch entries (one
        // pass per entry); one resident round of waves (registers allow 3 per
        // SIMD forward, 2 backward)
        p->tiny = 1;
        a.P = partial_len(k, a.Lm);
        const long ngrp = (d->C + 15) / 16;
        const long slots = (long)kComputeUnits * 4 * (bwd ? 2 : 3);
        const long nchunk = std::max<long>(1, std::min<long>(d->B, slots / ngrp));
        a.ppw = (int)((d->B + nchunk - 1) / nchunk);
        p->nchunk = (int)((d->B + a.ppw - 1) / a.ppw);
        p->grid = (int)(ngrp * p->nchunk);
        p->nrec = (long)p->nchunk * d->C;
        p->nthr = 64;
        p->bpq = 1;
        p->lds = 0;
        return WTC_OK;
    }
    // Launch plan: the LDS layout (levels 2 and 3 analysed in registers when
    // their bands fit; bands beside the level-0 plane, or from level 1 or 2
    // over it), planes per workgroup and threads.  Chosen to maximise the
    // lanes doing work per CU (resident workgroups are limited by LDS and by
    // registers: the kernels are compiled for 3 waves per SIMD forward, 2
    // backward or with two blocks per quad); on a tie the plan without band
    // overlap (one barrier less per plane), then overlap from level 2, then
    // the smaller workgroup.  Overlapping bands must have their zero rings
    // rewritten for every plane; in the forward pass, with half the arithmetic
    // per pixel of the backward, that mostly costs more than the occupancy it
    // buys, so the forward pass overlaps only when nothing else fits, or for
    // bf16 32x32 planes (below).
    // folded level weights (one 16-byte aligned set of round_up(k^2, 4) floats
    // per level and band), base weights, bias and scale
    const int wts_n = round_up(round_up(KK, 4) * 4 * d->L + KK + 4, 4);
    const int per_units = a.vec ? d->H * (d->W / 4) : d->H * d->W;
    struct Cand {
        Layout lay;
        int NP, nthr, bpq, wgs;
        long score;
    };
    Cand best{};
    best.score = -1;
    auto consider = [&](const Layout& lay, int NP, int nthr, int bpq) {
        const int dsub = std::max(1, nthr / (4 * k));
        const int red_n = red_len(nthr, k, a.Lm, dsub);
        const size_t lds = (size_t)std::max(NP * lay.slot + wts_n + flush_len(bwd, bpq, nthr, k, a.Lm), bwd ? red_n : 0) * 4;
        if (lds > kLdsLimit || NP * per_units >= 65536) return;   // fast in-kernel division range
        // plain depthwise conv (no levels) on a plane class with fixed-geometry
        // direct-load instances: those are compiled for more waves per SIMD
        const bool nolev = d->L == 0 && d->dtype == WTC_FP32 && lay.dl && a.Hq == 64 && (k == 5 || k == 7);
        const int wpe = fused_waves_per_simd(bwd, bpq, nolev);
        const int lds_wgs = (int)(kLdsLimit / lds);
        const int reg_wgs = std::max(1, 4 * wpe / (nthr / 64));
        const int wgs = std::max(1, std::min(lds_wgs, reg_wgs));
        const long score = (long)wgs * std::min(nthr, 4 * a.qpp * NP / bpq);
        const bool better = score > best.score ||
                            (score == best.score && best.lay.bovl == lay.bovl && nthr < best.nthr);
        if (better) best = Cand{lay, NP, nthr, bpq, wgs, score};
    };
    if (a.qpp > 256) return WTC_ESHAPE;
    // direct loads (DMA into the LDS slot, layout mode 1): planes of 4-pixel
    // rows with one block per quad (at most 128 quads), one plane per
    // workgroup.  The backward, fp32 or bf16: staged through registers it holds
    // a plane's prefetch next to its correlation accumulators and spills.  The
    // fp32 forward: 7-8 % faster than register staging on 32x32 to 56x56
    // planes; the bf16 forward measured faster staging through registers (54 us
    // against 70 us on 32x32 planes).  Tried first, so it wins ties.
    const int esz = d->dtype == WTC_BF16 ? 2 : 4;
    const bool dl_ok = a.vec && a.qpp <= 128 && (bwd || d->dtype == WTC_FP32) && !(a.nhwc && d->dtype == WTC_BF16);
    // The backward takes direct loads whenever one plane fills a wave, even where
    // the larger slot (it holds a plane of x too) leaves fewer workgroups resident
    // (32x32 fp32: 7 instead of 8 per CU).
    const bool dl_only = dl_ok && bwd && a.qpp >= 16;
    // then the layout without overlap (mode 2), which spares the per-plane ring
    // re-zeroing and wins ties against the overlapping one (32x32 bf16 forward:
    // 52 us against 54 us)
    for (const int variant : {-1, -2, 0, 2, 1}) {
        const bool dl = variant == -1;
        const int bovl = variant < 0 ? 0 : variant;
        const int mode = dl ? 1 : (variant == -2 ? 2 : 0);
        if (dl && !dl_ok) continue;
        if (!dl && dl_only && best.score >= 0) break;
        if (bovl > a.Lm) continue;
        Layout lay = make_layout(k, a.Hq, a.Wq, a.Lm, 3, bwd, bovl, mode, esz);
        if ((size_t)(lay.slot + wts_n) * 4 > kLdsLimit) lay = make_layout(k, a.Hq, a.Wq, a.Lm, 1, bwd, bovl, mode, esz);
        if (variant == -2 && lay.mode != 2) continue;   // same layout as mode 0
        // (forward overlap: only bf16 32x32 planes from level 1, whose fixed-geometry
        // instance it takes to three waves per SIMD: 58.7 -> 54.8 us on 64x192 planes;
        // 16x16 fp32 planes with overlap measured 60 -> 75 us)
        const bool fwd_ovl = d->dtype == WTC_BF16 && a.Hq == 32 && a.Wq == 32 && bovl == 1;
        if (bovl > 0 && !bwd && best.score >= 0 && !fwd_ovl) continue;
        if (a.qpp <= 64) {
            // several planes per workgroup when planes are small
            for (int np = 1; np <= (dl ? 1 : 64 / a.qpp); ++np) consider(lay, np, round_up(4 * a.qpp * np, 64), 1);
        } else if (a.qpp <= 128) {
            consider(lay, 1, 512, 1);
        } else {
            consider(lay, 1, 512, 2);
        }
    }
    if (best.score < 0) return WTC_ESHAPE;
    a.lay = best.lay;
    const int slot = a.lay.slot;
    const int NP = best.NP, nthr = best.nthr, bpq = best.bpq;
    a.NP = NP;
    {
        // prefetch when every thread's share of a plane group fits its capacity
        // (single-pixel units: counted per plane, NP * ceil(H W / threads), the
        // mapping of the fixed-geometry kernels)
        const int units = a.vec ? cdiv(NP * per_units, nthr) : NP * cdiv(per_units, nthr);
        a.pf_on = (!a.lay.dl && units * (a.vec ? 4 : 1) <= pf_capacity(bwd, bpq)) ? 1 : 0;
        // the kernel keeps unit offsets within a plane group in 32 bits
        if ((long)NP * d->C * d->H * d->W >= (1L << 31)) a.pf_on = 0;
    }
    a.dsub = std::max(1, nthr / (4 * k));
    a.wts_off = NP * slot;
    a.P = partial_len(k, a.Lm);
    // reduction scratch reuses the plane slots after the last plane
    a.red_off = 0;
    const int red_n = red_len(nthr, k, a.Lm, a.dsub);
    size_t lds_floats = (size_t)std::max(NP * slot + wts_n + flush_len(bwd, bpq, nthr, k, a.Lm), bwd ? red_n : 0);
    p->lds = lds_floats * 4;
    if (p->lds > kLdsLimit) return WTC_ESHAPE;

    // Work split over the batch: one resident "wave" of workgroups over the
    // whole chip, each walking a chunk of planes of one channel.
    const int wgs_per_cu = best.wgs;
    const long qtot = (long)d->B * d->C;
    const long slots = (long)kComputeUnits * wgs_per_cu;
    long ppw = (qtot + slots - 1) / slots;
    ppw = (ppw + NP - 1) / NP * NP;            // whole plane groups where channels allow
    ppw = std::min<long>(ppw, d->B);           // at most two channel segments per workgroup
    a.ppw = (int)std::max<long>(1, ppw);
    const int grid = (int)((qtot + a.ppw - 1) / a.ppw);
    p->nchunk = grid;
    p->grid = grid;
    p->nrec = 2L * grid;
    if (a.units) {
        // (batch chunk, channel) units of ppw planes: the chunk length (a whole
        // number of plane groups) that minimises rounds x chunk length
        long best_t = -1;
        int best_ppw = 1;
        for (int nc = 1; nc <= d->B; ++nc) {
            const int pp = std::min(d->B, round_up(cdiv(d->B, nc), NP));
            const long units = (long)d->C * cdiv(d->B, pp);
            const long t = (units + slots - 1) / slots * pp;
            if (best_t < 0 || t < best_t) {
                best_t = t;
                best_ppw = pp;
            }
        }
        a.ppw = best_ppw;
        a.nchunk = cdiv(d->B, a.ppw);
        const long units = (long)d->C * a.nchunk;
        if (8 * cdiv((int)std::min<long>(units, 1L << 28), 8) < units) return WTC_ESHAPE;
        p->nchunk = a.nchunk;
        p->grid = 8 * cdiv((int)units, 8);   // the units dealt to the 8 XCDs in contiguous ranges
        p->nrec = units;
    }
    p->nthr = nthr;
    p->bpq = bpq;
    return WTC_OK;
}

// ---------------------------------------------------------------------------
// Planes beyond the on-chip pipeline: peel one wavelet level.
// The levels >= 2 of WTConv are WTConv itself (one level fewer, no base conv)
// applied to the level-1 LL band, so such a plane runs its LL band (half the
// size in each direction) recursively through the fused entry points -- fused
// as soon as it fits -- and level 1 with the base conv fused over tiles of the
// full-resolution plane; with L = 0 (a depthwise conv too large for the
// pipeline) the level-by-level conv.  Workspace: [L = 0: that conv's
// intermediates; backward: the tile records][LL of x][Z_2 or LL of g][dLL_1]
// [zero scale and bias, unused gradients][the sub-problem's workspace]; only
// the front part when L < 2.
// ---------------------------------------------------------------------------
constexpr int kMaxPeel = 8;
size_t al256(size_t v) { return (v + 255) / 256 * 256; }

struct PeelPlan {
    wtc_desc d1, sub;   // level 1 of this plane; the LL problem (L - 1 levels, fp32)
    UnfusedPlan u;      // L = 0: the level-by-level depthwise conv
    size_t n1;          // floats of one LL tensor [B, C, h1, w1]
    size_t rec1_off;    // backward: level-1 tile records (base records at 0)
    size_t a_off, b_off, c_off, par_off, sub_off, total;
};

size_t fused_fwd_ws(const wtc_desc* d, int depth, int* st);
size_t fused_bwd_ws(const wtc_desc* d, int depth, int* st);

int peel_plan(const wtc_desc* d, bool bwd, int depth, PeelPlan* pp) {
    if (depth >= kMaxPeel) return WTC_ESHAPE;
    pp->d1 = *d;
    pp->d1.L = std::min(d->L, 1);
    int st = unfused_plan(&pp->d1, bwd ? 1 : 0, &pp->u);
    if (st != WTC_OK) return st;
    const int h1 = (d->H + 1) / 2, w1 = (d->W + 1) / 2;
    pp->n1 = (size_t)d->B * d->C * h1 * w1;
    pp->sub = wtc_desc{d->B, d->C, h1, w1, d->L - 1, d->k, WTC_FP32, 0};
    // front of the workspace: L = 0, the level-by-level conv's intermediates;
    // backward with levels, the tile kernel's correlation records (base, level 1)
    size_t base = 0;
    pp->rec1_off = 0;
    if (d->L == 0) {
        base = pp->u.total;
    } else if (bwd) {
        const size_t nrec = top_records(d);
        pp->rec1_off = al256(nrec * sizeof(float));
        base = pp->rec1_off + al256(4 * nrec * sizeof(float));
    }
    size_t off = al256(base);
    pp->a_off = off;   // forward: LL of x;  backward: LL of x
    pp->b_off = off = off + al256(pp->n1 * 4);   // forward: Z_2;  backward: LL of g
    pp->c_off = off = off + al256(pp->n1 * 4);   // backward: dLL_1
    if (bwd) off += al256(pp->n1 * 4);
    pp->par_off = off;  // zero scale and bias (2C); backward: unused base gradients (C k^2 + 2C)
    off += al256((size_t)4 * (2 * d->C + (bwd ? d->C * d->k * d->k + 2 * d->C : 0)));
    pp->sub_off = off;
    if (d->L < 2) {
        pp->total = base;
        return WTC_OK;
    }
    const size_t sw = bwd ? fused_bwd_ws(&pp->sub, depth + 1, &st) : fused_fwd_ws(&pp->sub, depth + 1, &st);
    if (st != WTC_OK) return st;
    pp->total = off + sw;
    return WTC_OK;
}

// Kernel sizes beyond the fused kernels (k > kMaxK) run the level-by-level
// kernels with the taps looped at run time: same results, same contract.
bool beyond_fused_k(const wtc_desc* d) { return d->k > kMaxK; }

size_t fused_fwd_ws(const wtc_desc* d, int depth, int* st) {
    if (beyond_fused_k(d)) {
        UnfusedPlan u;
        *st = unfused_plan(d, 0, &u);
        return *st == WTC_OK ? u.total : 0;
    }
    FusedPlan p;
    *st = plan_fused(d, false, &p);
    if (*st == WTC_OK) return 0;
    if (*st != WTC_ESHAPE) return 0;
    PeelPlan pp;
    *st = peel_plan(d, false, depth, &pp);
    return *st == WTC_OK ? pp.total : 0;
}

size_t fused_bwd_ws(const wtc_desc* d, int depth, int* st) {
    if (beyond_fused_k(d)) {
        UnfusedPlan u;
        *st = unfused_plan(d, 1, &u);
        return *st == WTC_OK ? u.total : 0;
    }
    FusedPlan p;
    *st = plan_fused(d, true, &p);
    if (*st == WTC_OK) return (size_t)p.nrec * p.a.P * sizeof(float);
    if (*st != WTC_ESHAPE) return 0;
    PeelPlan pp;
    *st = peel_plan(d, true, depth, &pp);
    return *st == WTC_OK ? pp.total : 0;
}

int unf_fwd_run(const wtc_desc* d, const void* x, const float* w0, const float* s0, const float* b0,
                const float* wl, const float* sl, void* out, char* ws, size_t wsb, void* stream);
int unf_bwd_run(const wtc_desc* d, const void* x, const void* g, const float* w0, const float* s0,
                const float* wl, const float* sl, void* dx, float* dw0, float* ds0, float* db0, float* dwl,
                float* dsl, char* ws, size_t wsb, void* stream);

int fused_fwd_run(const wtc_desc* d, const void* x, const float* w0, const float* s0, const float* b0,
                  const float* wl, const float* sl, void* out, char* ws, size_t wsb, void* stream, int depth) {
    if (beyond_fused_k(d)) return unf_fwd_run(d, x, w0, s0, b0, wl, sl, out, ws, wsb, stream);
    FusedPlan p;
    int st = plan_fused(d, false, &p);
    if (st == WTC_OK) {
        FusedArgs& a = p.a;
        a.src = x;
        a.aux = nullptr;
        a.w0 = w0; a.s0 = s0; a.b0 = b0; a.wl = wl; a.sl = sl;
        a.dst = out;
        a.partials = nullptr;
        a.nobase = depth > 0 ? 1 : 0;   // the LL problem of a peeled plane: scale and bias 0
        const int e = p.tiny == 2 ? launch_lane(a, d->dtype, 0, p.grid, stream)
                      : p.tiny    ? launch_tiny(a, d->dtype, 0, p.grid, stream)
                                  : launch_fused(a, d->k, d->dtype, 0, p.bpq, p.nthr, p.lds, p.grid, stream);
        return e == 0 ? WTC_OK : WTC_EHIP;
    }
    if (st != WTC_ESHAPE) return st;
    PeelPlan pp;
    st = peel_plan(d, false, depth, &pp);
    if (st != WTC_OK) return st;
    if (pp.total > 0 && (!ws || wsb < pp.total)) return WTC_EWORKSPACE;
    // L = 0: the plain depthwise conv
    if (d->L == 0) return unfused_forward(&pp.d1, pp.u, x, w0, s0, b0, wl, sl, out, ws, stream, 0, nullptr);
    const float* zext = nullptr;
    if (d->L >= 2) {
        float* ll = reinterpret_cast<float*>(ws + pp.a_off);
        float* z2 = reinterpret_cast<float*>(ws + pp.b_off);
        float* zero = reinterpret_cast<float*>(ws + pp.par_off);
        const size_t lvl = (size_t)4 * d->C * d->k * d->k;
        if ((st = top_ll(d, x, ll, stream)) != WTC_OK) return st;
        if (launch_fill_zero(zero, 2 * d->C, stream) != 0) return WTC_EHIP;
        // Z_2 = WTConv of LL_1 with levels 2..L; scale and bias 0 remove its base conv
        st = fused_fwd_run(&pp.sub, ll, w0, zero, zero + d->C, wl + lvl, sl + 4 * d->C, z2, ws + pp.sub_off,
                           wsb - pp.sub_off, stream, depth + 1);
        if (st != WTC_OK) return st;
        zext = z2;
    }
    // level 1 and the base conv, fused over tiles
    return top_forward(d, x, w0, s0, b0, wl, sl, zext, out, stream);
}

int fused_bwd_run(const wtc_desc* d, const void* x, const void* g, const float* w0, const float* s0,
                  const float* wl, const float* sl, void* dx, float* dw0, float* ds0, float* db0, float* dwl,
                  float* dsl, char* ws, size_t wsb, void* stream, int depth) {
    if (beyond_fused_k(d)) return unf_bwd_run(d, x, g, w0, s0, wl, sl, dx, dw0, ds0, db0, dwl, dsl, ws, wsb, stream);
    FusedPlan p;
    int st = plan_fused(d, true, &p);
    if (st == WTC_OK) {
        const size_t need = (size_t)p.nrec * p.a.P * sizeof(float);
        if (!ws || wsb < need) return WTC_EWORKSPACE;
        FusedArgs& a = p.a;
        a.src = g;
        a.aux = x;
        a.w0 = w0; a.s0 = s0; a.b0 = nullptr; a.wl = wl; a.sl = sl;
        a.dst = dx;
        a.partials = reinterpret_cast<float*>(ws);
        a.nobase = depth > 0 ? 1 : 0;
        int e = p.tiny == 2 ? launch_lane(a, d->dtype, 1, p.grid, stream)
                : p.tiny    ? launch_tiny(a, d->dtype, 1, p.grid, stream)
                            : launch_fused(a, d->k, d->dtype, 1, p.bpq, p.nthr, p.lds, p.grid, stream);
        if (e != 0) return WTC_EHIP;
        FinalizeArgs f;
        f.partials = a.partials;
        f.w0 = w0; f.s0 = s0; f.wl = wl; f.sl = sl;
        f.dw0 = dw0; f.ds0 = ds0; f.db0 = db0; f.dwl = dwl; f.dsl = dsl;
        f.C = d->C; f.B = d->B; f.L = d->L; f.Lm = a.Lm; f.k = d->k; f.ppw = a.ppw; f.P = a.P;
        f.chunks = (p.tiny || a.units) ? p.nchunk : 0;
        e = launch_finalize(f, stream);
        return e == 0 ? WTC_OK : WTC_EHIP;
    }
    if (st != WTC_ESHAPE) return st;
    PeelPlan pp;
    st = peel_plan(d, true, depth, &pp);
    if (st != WTC_OK) return st;
    if (!ws || wsb < pp.total) return WTC_EWORKSPACE;
    // L = 0: the plain depthwise conv and its correlation
    if (d->L == 0)
        return unfused_backward(&pp.d1, pp.u, x, g, w0, s0, wl, sl, dx, dw0, ds0, db0, dwl, dsl, ws, stream, 0,
                                nullptr);
    const float* zext = nullptr;
    if (d->L >= 2) {
        float* xll = reinterpret_cast<float*>(ws + pp.a_off);
        float* gll = reinterpret_cast<float*>(ws + pp.b_off);
        float* dll = reinterpret_cast<float*>(ws + pp.c_off);
        float* zero = reinterpret_cast<float*>(ws + pp.par_off);
        float* scratch = zero + 2 * d->C;   // the sub-problem's base gradients (unused)
        const int KK = d->k * d->k;
        const size_t lvl = (size_t)4 * d->C * KK;
        if ((st = top_ll(d, x, xll, stream)) != WTC_OK) return st;
        if ((st = top_ll(d, g, gll, stream)) != WTC_OK) return st;
        if (launch_fill_zero(zero, 2 * d->C, stream) != 0) return WTC_EHIP;
        // levels 2..L: the backward of WTConv(LL_1) with upstream gradient LL_1(g)
        // (the level-1 synthesis adjoint); scale 0 removes its base conv from dLL_1
        st = fused_bwd_run(&pp.sub, xll, gll, w0, zero, wl + lvl, sl + 4 * d->C, dll, scratch, scratch + d->C * KK,
                           scratch + d->C * KK + d->C, dwl + lvl, dsl + 4 * d->C, ws + pp.sub_off, wsb - pp.sub_off,
                           stream, depth + 1);
        if (st != WTC_OK) return st;
        zext = dll;
    }
    // level 1 and the base conv fused over tiles; the tiles' correlation
    // records go where the level-by-level intermediates would (unused here)
    const size_t nrec = top_records(d);
    float* part0 = reinterpret_cast<float*>(ws);
    float* part1 = reinterpret_cast<float*>(ws + pp.rec1_off);
    if ((st = top_backward(d, x, g, w0, s0, wl, sl, zext, dx, part0, part1, stream)) != WTC_OK) return st;
    const int nblk = (int)(nrec / ((size_t)d->C * (d->k * d->k + 1)));
    if ((st = launch_corr_finalize(part0, d->C, nblk, d->k, w0, s0, dw0, ds0, db0, stream)) != WTC_OK) return st;
    return launch_corr_finalize(part1, 4 * d->C, nblk, d->k, wl, sl, dwl, dsl, nullptr, stream);
}

int unf_fwd_run(const wtc_desc* d, const void* x, const float* w0, const float* s0, const float* b0,
                const float* wl, const float* sl, void* out, char* ws, size_t wsb, void* stream) {
    UnfusedPlan p;
    const int st = unfused_plan(d, 0, &p);
    if (st != WTC_OK) return st;
    if (p.total > 0 && (!ws || wsb < p.total)) return WTC_EWORKSPACE;
    return unfused_forward(d, p, x, w0, s0, b0, wl, sl, out, ws, stream);
}

int unf_bwd_run(const wtc_desc* d, const void* x, const void* g, const float* w0, const float* s0,
                const float* wl, const float* sl, void* dx, float* dw0, float* ds0, float* db0, float* dwl,
                float* dsl, char* ws, size_t wsb, void* stream) {
    UnfusedPlan p;
    const int st = unfused_plan(d, 1, &p);
    if (st != WTC_OK) return st;
    if (!ws || wsb < p.total) return WTC_EWORKSPACE;
    return unfused_backward(d, p, x, g, w0, s0, wl, sl, dx, dw0, ds0, db0, dwl, dsl, ws, stream);
}

// ---------------------------------------------------------------------------
// Channels-last (NHWC) tensors: transposed into NCHW copies at the front of
// the workspace, computed there, the result transposed back.
// ---------------------------------------------------------------------------
// Channels-last tensors read and written in place (layout 2): planes the
// on-chip pipeline holds, k <= kMaxK.  Layout 1, and layout 2 anywhere else,
// is adapted through NCHW copies.
bool nhwc_native(const wtc_desc* d, bool bwd) {
    if (d->layout != 2 || beyond_fused_k(d)) return false;
    FusedPlan p;
    return plan_fused(d, bwd, &p) == WTC_OK;
}

size_t nhwc_tensor_bytes(const wtc_desc* d) {
    return al256((size_t)d->B * d->C * d->H * d->W * (d->dtype == WTC_BF16 ? 2 : 4));
}

int nhwc_forward(const wtc_desc* d, bool unf, const void* x, const float* w0, const float* s0, const float* b0,
                 const float* wl, const float* sl, void* out, char* ws, size_t wsb, void* stream) {
    const wtc_desc n = nchw_of(d);
    const size_t T = nhwc_tensor_bytes(d);
    size_t inner = 0;
    if (unf) {
        UnfusedPlan p;
        const int st = unfused_plan(&n, 0, &p);
        if (st != WTC_OK) return st;
        inner = p.total;
    } else {
        int st = WTC_OK;
        inner = fused_fwd_ws(&n, 0, &st);
        if (st != WTC_OK) return st;
    }
    if (!ws || wsb < 2 * T + inner) return WTC_EWORKSPACE;
    const int HW = d->H * d->W, e = d->dtype == WTC_BF16 ? 2 : 4;
    char* xt = ws;
    char* ot = ws + T;
    if (launch_transpose(x, xt, d->B, HW, d->C, e, stream) != 0) return WTC_EHIP;
    const int st = unf ? unf_fwd_run(&n, xt, w0, s0, b0, wl, sl, ot, ws + 2 * T, wsb - 2 * T, stream)
                       : fused_fwd_run(&n, xt, w0, s0, b0, wl, sl, ot, ws + 2 * T, wsb - 2 * T, stream, 0);
    if (st != WTC_OK) return st;
    return launch_transpose(ot, out, d->B, d->C, HW, e, stream) == 0 ? WTC_OK : WTC_EHIP;
}

int nhwc_backward(const wtc_desc* d, bool unf, const void* x, const void* g, const float* w0, const float* s0,
                  const float* wl, const float* sl, void* dx, float* dw0, float* ds0, float* db0, float* dwl,
                  float* dsl, char* ws, size_t wsb, void* stream) {
    const wtc_desc n = nchw_of(d);
    const size_t T = nhwc_tensor_bytes(d);
    size_t inner = 0;
    if (unf) {
        UnfusedPlan p;
        const int st = unfused_plan(&n, 1, &p);
        if (st != WTC_OK) return st;
        inner = p.total;
    } else {
        int st = WTC_OK;
        inner = fused_bwd_ws(&n, 0, &st);
        if (st != WTC_OK) return st;
    }
    if (!ws || wsb < 3 * T + inner) return WTC_EWORKSPACE;
    const int HW = d->H * d->W, e = d->dtype == WTC_BF16 ? 2 : 4;
    char* xt = ws;
    char* gt = ws + T;
    char* dxt = ws + 2 * T;
    if (launch_transpose(x, xt, d->B, HW, d->C, e, stream) != 0) return WTC_EHIP;
    if (launch_transpose(g, gt, d->B, HW, d->C, e, stream) != 0) return WTC_EHIP;
    const int st = unf ? unf_bwd_run(&n, xt, gt, w0, s0, wl, sl, dxt, dw0, ds0, db0, dwl, dsl, ws + 3 * T,
                                     wsb - 3 * T, stream)
                       : fused_bwd_run(&n, xt, gt, w0, s0, wl, sl, dxt, dw0, ds0, db0, dwl, dsl, ws + 3 * T,
                                       wsb - 3 * T, stream, 0);
    if (st != WTC_OK) return st;
    return launch_transpose(dxt, dx, d->B, d->C, HW, e, stream) == 0 ? WTC_OK : WTC_EHIP;
}

double spec_level_area(const wtc_desc* d, int i) {
    int h = d->H, w = d->W;
    for (int l = 0; l < i; ++l) {
        h = (h + 1) / 2;
        w = (w + 1) / 2;
    }
    return (double)h * w;
}

double io_unfused(const wtc_desc* d, int dir) {
    const double e = d->dtype == WTC_BF16 ? 2.0 : 4.0;
    const double KK = (double)d->k * d->k;
    const double BC = (double)d->B * d->C;
    const double N = BC * d->H * d->W;
    const double params = 4.0 * (d->C * KK * (1 + 4.0 * d->L) + d->C * (2.0 + 4.0 * d->L));
    UnfusedPlan p;
    if (unfused_plan(d, dir, &p) != WTC_OK) return -1.0;
    // Level-by-level baseline: the bytes its kernels move, each tensor read or
    // written once per kernel that touches it (stencil halos hit in cache).
    // Intermediates are float32; x, g, out and dx use the storage dtype.
    const double f4 = 4.0;
    const int kk1 = d->k * d->k + 1;
    auto band = [&](int i) { return BC * spec_level_area(d, i) * f4; };   // one band of level i
    double t = 0.0;
    // analysis cascade (forward: of x; backward: of g and of x): read LL_{i-1}, write 4 bands
    const double casc_n = dir == 0 ? 1.0 : 2.0;
    for (int i = 1; i <= d->L; ++i) t += casc_n * ((i == 1 ? N * e : band(i - 1)) + 4.0 * band(i));
    // subband conv per level: read 4 bands, write 4 bands
    for (int i = 1; i <= d->L; ++i) t += 8.0 * band(i);
    // synthesis per level: read 4 bands (+ the deeper partial result), write the finer grid
    for (int i = 1; i <= d->L; ++i) t += 4.0 * band(i) + (i < d->L ? band(i) : 0.0) + band(i - 1);
    // base: read the convolved tensor and Z_1 (dLL_0), write out (dx)
    t += 2.0 * N * e + (d->L > 0 ? band(0) : 0.0);
    if (dir == 0) return t + params;
    // correlations: per level read dT_i and S_i (8 bands), base read g and x;
    // partials written and read back; parameters read twice, gradients written
    for (int i = 1; i <= d->L; ++i) {
        t += 8.0 * band(i);
        t += 2.0 * f4 * unfused_corr_blocks(d->B, 4 * d->C, p.h[i], p.w[i]) * 4.0 * d->C * kk1;
    }
    t += 2.0 * N * e + 2.0 * f4 * unfused_corr_blocks(d->B, d->C, d->H, d->W) * (double)d->C * kk1;
    return t + 3.0 * params;
}

double io_unfused(const wtc_desc* d, int dir);

double io_fused(const wtc_desc* d, int dir, int depth) {
    if (beyond_fused_k(d)) return io_unfused(d, dir);
    const double e = d->dtype == WTC_BF16 ? 2.0 : 4.0;
    const double KK = (double)d->k * d->k;
    const double BC = (double)d->B * d->C;
    const double N = BC * d->H * d->W;
    const double params = 4.0 * (d->C * KK * (1 + 4.0 * d->L) + d->C * (2.0 + 4.0 * d->L));
    FusedPlan p;
    const int st = plan_fused(d, dir == 1, &p);
    if (st == WTC_OK) {
        if (dir == 0) return 2.0 * N * e + params;
        const double partials = 4.0 * (double)p.nrec * p.a.P;
        // read x and g, write dx; params read; partials written then read; grads written
        return 3.0 * N * e + params + 2.0 * partials + params;
    }
    // peeled plane: the LL band recursively, level 1 and the base fused over tiles
    PeelPlan pp;
    if (st != WTC_ESHAPE || peel_plan(d, dir == 1, depth, &pp) != WTC_OK) return -1.0;
    if (d->L == 0) return io_unfused(&pp.d1, dir);   // the plain depthwise conv
    const double ll = 4.0 * (double)pp.n1;
    double t = 0.0;
    if (d->L >= 2) {
        // LL bands (forward: of x; backward: of x and g): read the tensor, write the band;
        // then the sub-problem, whose result (gradient) the tile kernel reads once
        t += (dir == 0 ? 1.0 : 2.0) * (N * e + ll) + io_fused(&pp.sub, dir, depth + 1) + ll;
    }
    if (dir == 0) return t + 2.0 * N * e + params;   // tiles: read x, write out
    // tiles: read g and x, write dx; per-tile correlation records (base and level 1)
    // written and read back by the two finalizes; parameters read, gradients written
    const double recs = 4.0 * 5.0 * (double)top_records(d);
    return t + 3.0 * N * e + 2.0 * recs + 2.0 * params;
}

// Base-level correlation on its own: the batch chunks of the matrix-core
// kernel (one-wave workgroups, about four per SIMD in all) and the limits of
// each path.
int corr_chunks(const wtc_desc* d) {
    const int want = std::max(1, cdiv(16 * kComputeUnits, d->C));
    const int ppc = cdiv(d->B, std::min(want, d->B));
    return cdiv(d->B, ppc);
}
int base_corr_check(const wtc_desc* d, int impl) {
    int st = check_desc(d);
    if (st != WTC_OK) return st;
    if (d->layout != 0) return WTC_EDTYPE;
    if (impl != 0 && impl != 1) return WTC_EINVAL;
    if ((long)d->B * d->C * d->H * d->W >= (1L << 31)) return WTC_ESHAPE;   // 32-bit element indices
    if (impl == 0) return d->k <= kMaxKAny ? WTC_OK : WTC_ESHAPE;
    if (d->dtype != WTC_BF16) return WTC_EDTYPE;
    if (d->k > kMaxK || d->H > 64 || d->W > 64) return WTC_ESHAPE;
    return WTC_OK;
}
size_t base_corr_floats(const wtc_desc* d, int impl) {
    const size_t rec = (size_t)d->C * (d->k * d->k + 1);
    return impl == 0 ? (size_t)unfused_corr_blocks(d->B, d->C, d->H, d->W) * rec : (size_t)corr_chunks(d) * rec;
}

}  // namespace

int backward_check(const wtc_desc* d, const void* x, const void* g, const float* w0, const float* s0,
                   const float* wl, const float* sl, const void* dx, const float* dw0, const float* ds0,
                   const float* db0, const float* dwl, const float* dsl) {
    const int st = check_desc(d);
    if (st != WTC_OK) return st;
    if (!x || !g || !w0 || !s0 || !dx || !dw0 || !ds0 || !db0) return WTC_EINVAL;
    if (d->L > 0 && (!wl || !sl || !dwl || !dsl)) return WTC_EINVAL;
    return WTC_OK;
}

}  // namespace wtc

using namespace wtc;

extern "C" {

const char* wtconv_status_string(int s) {
    switch (s) {
        case WTC_OK: return "ok";
        case WTC_EINVAL: return "invalid argument";
        case WTC_ESHAPE: return "shape outside the supported limits";
        case WTC_EDTYPE: return "unsupported dtype or layout";
        case WTC_EWORKSPACE: return "workspace missing or too small";
        case WTC_EHIP: return "HIP launch or runtime error";
        case WTC_ESCRATCH: return "needs more scratch than the fixed no-allocation buffer holds";
        default: return "unknown status";
    }
}

size_t wtconv_forward_workspace(const wtc_desc* d) {
    if (check_desc(d) != WTC_OK) return 0;
    if (nhwc_native(d, false)) return 0;
    const wtc_desc n = nchw_of(d);
    int st = WTC_OK;
    const size_t inner = fused_fwd_ws(&n, 0, &st);
    if (st != WTC_OK) return 0;
    return d->layout != 0 ? 2 * nhwc_tensor_bytes(d) + inner : inner;
}

int wtconv_forward(const wtc_desc* d, const void* x, const float* w0, const float* s0,
                   const float* b0, const float* wl, const float* sl, void* out, void* workspace,
                   size_t workspace_bytes, void* stream) {
    int st = check_desc(d);
    if (st != WTC_OK) return st;
    if (!x || !w0 || !s0 || !b0 || !out) return WTC_EINVAL;
    if (d->L > 0 && (!wl || !sl)) return WTC_EINVAL;
    if (d->layout != 0 && !nhwc_native(d, false))
        return nhwc_forward(d, false, x, w0, s0, b0, wl, sl, out, static_cast<char*>(workspace), workspace_bytes,
                            stream);
    return fused_fwd_run(d, x, w0, s0, b0, wl, sl, out, static_cast<char*>(workspace), workspace_bytes, stream, 0);
}

size_t wtconv_backward_workspace(const wtc_desc* d) {
    if (check_desc(d) != WTC_OK) return 0;
    if (nhwc_native(d, true)) {
        int st = WTC_OK;
        return fused_bwd_ws(d, 0, &st);
    }
    const wtc_desc n = nchw_of(d);
    int st = WTC_OK;
    const size_t inner = fused_bwd_ws(&n, 0, &st);
    if (st != WTC_OK) return 0;
    return d->layout != 0 ? 3 * nhwc_tensor_bytes(d) + inner : inner;
}

int wtconv_backward(const wtc_desc* d, const void* x, const void* g, const float* w0,
                    const float* s0, const float* wl, const float* sl, void* dx, float* dw0,
                    float* ds0, float* db0, float* dwl, float* dsl, void* workspace,
                    size_t workspace_bytes, void* stream) {
    const int st = backward_check(d, x, g, w0, s0, wl, sl, dx, dw0, ds0, db0, dwl, dsl);
    if (st != WTC_OK) return st;
    if (d->layout != 0 && !nhwc_native(d, true))
        return nhwc_backward(d, false, x, g, w0, s0, wl, sl, dx, dw0, ds0, db0, dwl, dsl,
                             static_cast<char*>(workspace), workspace_bytes, stream);
    return fused_bwd_run(d, x, g, w0, s0, wl, sl, dx, dw0, ds0, db0, dwl, dsl, static_cast<char*>(workspace),
                         workspace_bytes, stream, 0);
}

// ---------------------------------------------------------------------------
// Unfused baseline
// ---------------------------------------------------------------------------
size_t wtconv_forward_unfused_workspace(const wtc_desc* d) {
    if (check_desc(d) != WTC_OK) return 0;
    const wtc_desc n = nchw_of(d);
    UnfusedPlan p;
    if (unfused_plan(&n, 0, &p) != WTC_OK) return 0;
    return d->layout != 0 ? 2 * nhwc_tensor_bytes(d) + p.total : p.total;
}

int wtconv_forward_unfused(const wtc_desc* d, const void* x, const float* w0, const float* s0,
                           const float* b0, const float* wl, const float* sl, void* out,
                           void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_desc(d);
    if (st != WTC_OK) return st;
    if (!x || !w0 || !s0 || !b0 || !out) return WTC_EINVAL;
    if (d->L > 0 && (!wl || !sl)) return WTC_EINVAL;
    if (d->layout != 0)
        return nhwc_forward(d, true, x, w0, s0, b0, wl, sl, out, static_cast<char*>(workspace), workspace_bytes,
                            stream);
    return unf_fwd_run(d, x, w0, s0, b0, wl, sl, out, static_cast<char*>(workspace), workspace_bytes, stream);
}

size_t wtconv_backward_unfused_workspace(const wtc_desc* d) {
    if (check_desc(d) != WTC_OK) return 0;
    const wtc_desc n = nchw_of(d);
    UnfusedPlan p;
    if (unfused_plan(&n, 1, &p) != WTC_OK) return 0;
    return d->layout != 0 ? 3 * nhwc_tensor_bytes(d) + p.total : p.total;
}

int wtconv_backward_unfused(const wtc_desc* d, const void* x, const void* g, const float* w0,
                            const float* s0, const float* wl, const float* sl, void* dx,
                            float* dw0, float* ds0, float* db0, float* dwl, float* dsl,
                            void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_desc(d);
    if (st != WTC_OK) return st;
    if (!x || !g || !w0 || !s0 || !dx || !dw0 || !ds0 || !db0) return WTC_EINVAL;
    if (d->L > 0 && (!wl || !sl || !dwl || !dsl)) return WTC_EINVAL;
    if (d->layout != 0)
        return nhwc_backward(d, true, x, g, w0, s0, wl, sl, dx, dw0, ds0, db0, dwl, dsl,
                             static_cast<char*>(workspace), workspace_bytes, stream);
    return unf_bwd_run(d, x, g, w0, s0, wl, sl, dx, dw0, ds0, db0, dwl, dsl, static_cast<char*>(workspace),
                       workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
// Base-level correlation (VALU tiles or matrix cores)
// ---------------------------------------------------------------------------
size_t wtconv_base_correlation_workspace(const wtc_desc* d, int impl) {
    if (base_corr_check(d, impl) != WTC_OK) return 0;
    return base_corr_floats(d, impl) * sizeof(float);
}

int wtconv_base_correlation(const wtc_desc* d, const void* x, const void* g, float* c0, int impl, void* workspace,
                            size_t workspace_bytes, void* stream) {
    int st = base_corr_check(d, impl);
    if (st != WTC_OK) return st;
    if (!x || !g || !c0) return WTC_EINVAL;
    const size_t need = base_corr_floats(d, impl) * sizeof(float);
    if (!workspace || workspace_bytes < need) return WTC_EWORKSPACE;
    float* part = static_cast<float*>(workspace);
    const int kk = d->k * d->k;
    int nblk = 0;
    if (impl == 0) {
        st = base_corr_partials(d, x, g, part, &nblk, stream);
    } else {
        nblk = corr_chunks(d);
        st = launch_corr0_mfma(d, x, g, part, nblk, stream);
    }
    if (st != WTC_OK) return st;
    return launch_corr_sum(part, d->C, nblk, kk + 1, kk, c0, stream);
}

// ---------------------------------------------------------------------------
// I/O model and flop count
// ---------------------------------------------------------------------------
double wtconv_flops(const wtc_desc* d, int dir) {
    if (check_desc(d) != WTC_OK || (dir != 0 && dir != 1)) return -1.0;
    const double KK = (double)d->k * d->k;
    const double BC = (double)d->B * d->C;
    const double N = BC * d->H * d->W;
    // forward: base conv (FMA) + bias/combine; per level: 4 subband convs (FMA),
    // 8 add/sub analysis butterfly and 8 add/sub synthesis butterfly per position
    double f = 2.0 * KK * N + 2.0 * N;
    for (int i = 1; i <= d->L; ++i) f += BC * spec_level_area(d, i) * (2.0 * 4.0 * KK + 16.0);
    if (dir == 0) return f;
    // backward: dX is the same pipeline without the bias; the correlations repeat
    // every FMA once more; x needs its own analysis cascade; sum of g
    double b = f - N;
    b += 2.0 * KK * N + N;
    for (int i = 1; i <= d->L; ++i) b += BC * spec_level_area(d, i) * (2.0 * 4.0 * KK + 8.0);
    return b;
}

double wtconv_io_model_bytes(const wtc_desc* d, int impl, int dir) {
    if (check_desc(d) != WTC_OK || (dir != 0 && dir != 1) || (impl != 0 && impl != 1)) return -1.0;
    if (impl == 0 && nhwc_native(d, dir == 1)) return io_fused(d, dir, 0);   // read and written in place
    const wtc_desc n = nchw_of(d);
    const double t = impl == 0 ? io_fused(&n, dir, 0) : io_unfused(&n, dir);
    if (t < 0 || d->layout == 0) return t;
    // channels-last: x (and g) transposed in, out (dx) transposed back, each read and written
    const double N = (double)d->B * d->C * d->H * d->W * (d->dtype == WTC_BF16 ? 2.0 : 4.0);
    return t + (dir == 0 ? 4.0 : 6.0) * N;
}

}  // extern "C"
