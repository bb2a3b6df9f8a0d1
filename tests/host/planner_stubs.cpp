// Host stand-ins for libwtconv's kernel launchers, for the sanitizer build of
// the dispatcher and planner (wtconv_api.cpp, wtconv_plan.cpp) on a machine
// without a GPU.  Each stub checks the launch shape it is given and touches
// every byte the real kernels read or write through the pointers it gets:
// under AddressSanitizer a tensor, workspace region or record array that the
// planner sized too small is reported at once.
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "wtc_internal.h"

namespace wtc {
namespace {

volatile unsigned char g_sink;

void need(bool ok, const char* what) {
    if (!ok) {
        std::fprintf(stderr, "launch check failed: %s\n", what);
        std::abort();
    }
}
void rd(const void* p, size_t n) {
    if (!p || n == 0) return;
    const unsigned char* c = static_cast<const unsigned char*>(p);
    unsigned char s = 0;
    for (size_t i = 0; i < n; ++i) s ^= c[i];
    g_sink = s;
}
void wr(void* p, size_t n) {
    if (p && n) std::memset(p, 0, n);
}
size_t act_bytes(const FusedArgs& a, int dtype) {
    return (size_t)a.B * a.C * a.H * a.W * (dtype == WTC_BF16 ? 2 : 4);
}
void params(const FusedArgs& a, int K, bool bwd) {
    rd(a.w0, sizeof(float) * a.C * K * K);
    rd(a.s0, sizeof(float) * a.C);
    if (!bwd && !a.nobase) rd(a.b0, sizeof(float) * a.C);
    rd(a.wl, sizeof(float) * (size_t)a.L * 4 * a.C * K * K);
    rd(a.sl, sizeof(float) * (size_t)a.L * 4 * a.C);
}

}  // namespace

int launch_fused(const FusedArgs& a, int k, int dtype, int bwd, int bpq, int nthr, size_t lds_bytes, int grid,
                 void*) {
    need(k >= 1 && k <= kMaxK && k % 2 == 1, "kernel size");
    need(nthr >= 64 && nthr <= 1024 && nthr % 64 == 0, "threads");
    need(bpq == 1 || bpq == 2, "blocks per quad");
    need(lds_bytes <= 160 * 1024, "LDS");
    need(grid >= 1 && (long)grid * a.ppw >= (long)a.B * a.C, "grid covers every plane");
    need(!a.units || (grid % 8 == 0 && (long)a.nchunk * a.ppw >= a.B && grid >= a.C * a.nchunk), "unit grid");
    need(a.NP >= 1 && a.Lm <= kMaxLm && a.Hq % 8 == 0 && a.Wq % 8 == 0, "plane geometry");
    need((size_t)(a.NP * a.lay.slot) * 4 <= lds_bytes, "plane slots fit");
    rd(a.src, act_bytes(a, dtype));
    if (bwd) rd(a.aux, act_bytes(a, dtype));
    params(a, k, bwd);
    wr(a.dst, act_bytes(a, dtype));
    if (bwd) wr(a.partials, sizeof(float) * (a.units ? (size_t)a.C * a.nchunk : 2 * (size_t)grid) * a.P);
    return 0;
}

int launch_finalize(const FinalizeArgs& f, void*) {
    const int KK = f.k * f.k;
    size_t recs;
    if (f.chunks > 0) {
        recs = (size_t)f.chunks * f.C;
    } else {
        const long last_wg = ((long)f.C * f.B - 1) / f.ppw;
        recs = 2 * (size_t)(last_wg + 1);
    }
    rd(f.partials, sizeof(float) * recs * f.P);
    rd(f.w0, sizeof(float) * f.C * KK);
    rd(f.s0, sizeof(float) * f.C);
    rd(f.wl, sizeof(float) * (size_t)f.L * 4 * f.C * KK);
    rd(f.sl, sizeof(float) * (size_t)f.L * 4 * f.C);
    wr(f.dw0, sizeof(float) * f.C * KK);
    wr(f.ds0, sizeof(float) * f.C);
    wr(f.db0, sizeof(float) * f.C);
    wr(f.dwl, sizeof(float) * (size_t)f.L * 4 * f.C * KK);
    wr(f.dsl, sizeof(float) * (size_t)f.L * 4 * f.C);
    return 0;
}

int launch_tiny(const FusedArgs& a, int dtype, int bwd, int grid, void*) {
    const int ngrp = (a.C + 15) / 16;
    need(grid % ngrp == 0, "tiny grid");
    const int nchunk = grid / ngrp;
    need((long)nchunk * a.ppw >= a.B, "tiny chunks cover the batch");
    rd(a.src, act_bytes(a, dtype));
    if (bwd) rd(a.aux, act_bytes(a, dtype));
    params(a, 5, bwd);
    wr(a.dst, act_bytes(a, dtype));
    if (bwd) wr(a.partials, sizeof(float) * (size_t)nchunk * a.C * a.P);
    return 0;
}

int launch_lane(const FusedArgs& a, int dtype, int bwd, int grid, void*) {
    const int nchunk = (a.B + 63) / 64;
    need(grid % 8 == 0 && grid >= a.C * nchunk && grid < a.C * nchunk + 8, "lane grid");
    rd(a.src, act_bytes(a, dtype));
    if (bwd) rd(a.aux, act_bytes(a, dtype));
    params(a, 5, bwd);
    wr(a.dst, act_bytes(a, dtype));
    if (bwd) wr(a.partials, sizeof(float) * (size_t)nchunk * a.C * a.P);
    return 0;
}

int top_forward(const wtc_desc* d, const void* x, const float* w0, const float* s0, const float* b0,
                const float* wl, const float* sl, const float* zext, void* out, void*) {
    const size_t n = (size_t)d->B * d->C * d->H * d->W * (d->dtype == WTC_BF16 ? 2 : 4);
    const size_t n1 = (size_t)d->B * d->C * ((d->H + 1) / 2) * ((d->W + 1) / 2);
    const int KK = d->k * d->k;
    rd(x, n);
    rd(zext, sizeof(float) * n1);
    rd(w0, sizeof(float) * d->C * KK);
    rd(s0, sizeof(float) * d->C);
    rd(b0, sizeof(float) * d->C);
    rd(wl, sizeof(float) * 4 * d->C * KK);
    rd(sl, sizeof(float) * 4 * d->C);
    wr(out, n);
    return WTC_OK;
}

int top_backward(const wtc_desc* d, const void* x, const void* g, const float* w0, const float* s0, const float* wl,
                 const float* sl, const float* dll, void* dx, float* part0, float* part1, void*) {
    const size_t n = (size_t)d->B * d->C * d->H * d->W * (d->dtype == WTC_BF16 ? 2 : 4);
    const size_t n1 = (size_t)d->B * d->C * ((d->H + 1) / 2) * ((d->W + 1) / 2);
    const int KK = d->k * d->k;
    rd(x, n);
    rd(g, n);
    rd(dll, sizeof(float) * n1);
    rd(w0, sizeof(float) * d->C * KK);
    rd(s0, sizeof(float) * d->C);
    rd(wl, sizeof(float) * 4 * d->C * KK);
    rd(sl, sizeof(float) * 4 * d->C);
    wr(dx, n);
    wr(part0, sizeof(float) * top_records(d));
    wr(part1, sizeof(float) * 4 * top_records(d));
    return WTC_OK;
}

int top_ll(const wtc_desc* d, const void* x, float* ll, void*) {
    rd(x, (size_t)d->B * d->C * d->H * d->W * (d->dtype == WTC_BF16 ? 2 : 4));
    wr(ll, sizeof(float) * (size_t)d->B * d->C * ((d->H + 1) / 2) * ((d->W + 1) / 2));
    return WTC_OK;
}

int launch_corr_finalize(const float* part, int nch, int nblk, int k, const float* wt, const float* scale, float* dw,
                         float* ds, float* db, void*) {
    const int KK = k * k;
    rd(part, sizeof(float) * (size_t)nblk * nch * (KK + 1));
    rd(wt, sizeof(float) * (size_t)nch * KK);
    rd(scale, sizeof(float) * nch);
    wr(dw, sizeof(float) * (size_t)nch * KK);
    wr(ds, sizeof(float) * nch);
    wr(db, sizeof(float) * nch);
    return WTC_OK;
}

int unfused_forward(const wtc_desc* d, const UnfusedPlan& p, const void* x, const float* w0, const float* s0,
                    const float* b0, const float* wl, const float* sl, void* out, char* ws, void*, int stage,
                    const float* zext) {
    const size_t n = (size_t)d->B * d->C * d->H * d->W * (d->dtype == WTC_BF16 ? 2 : 4);
    const int KK = d->k * d->k;
    rd(x, n);
    rd(w0, sizeof(float) * d->C * KK);
    rd(s0, sizeof(float) * d->C);
    rd(b0, sizeof(float) * d->C);
    rd(wl, sizeof(float) * (size_t)d->L * 4 * d->C * KK);
    rd(sl, sizeof(float) * (size_t)d->L * 4 * d->C);
    if (zext && d->L > 0) rd(zext, sizeof(float) * (size_t)d->B * d->C * p.h[d->L] * p.w[d->L]);
    wr(ws, p.total);
    if (stage != 1) wr(out, n);
    return WTC_OK;
}

int unfused_backward(const wtc_desc* d, const UnfusedPlan& p, const void* x, const void* g, const float* w0,
                     const float* s0, const float* wl, const float* sl, void* dx, float* dw0, float* ds0,
                     float* db0, float* dwl, float* dsl, char* ws, void*, int stage, const float* zext) {
    const size_t n = (size_t)d->B * d->C * d->H * d->W * (d->dtype == WTC_BF16 ? 2 : 4);
    const int KK = d->k * d->k;
    rd(x, n);
    rd(g, n);
    rd(w0, sizeof(float) * d->C * KK);
    rd(s0, sizeof(float) * d->C);
    rd(wl, sizeof(float) * (size_t)d->L * 4 * d->C * KK);
    rd(sl, sizeof(float) * (size_t)d->L * 4 * d->C);
    if (zext && d->L > 0) rd(zext, sizeof(float) * (size_t)d->B * d->C * p.h[d->L] * p.w[d->L]);
    wr(ws, p.total);
    if (stage == 1) return WTC_OK;
    wr(dx, n);
    wr(dw0, sizeof(float) * d->C * KK);
    wr(ds0, sizeof(float) * d->C);
    wr(db0, sizeof(float) * d->C);
    wr(dwl, sizeof(float) * (size_t)d->L * 4 * d->C * KK);
    wr(dsl, sizeof(float) * (size_t)d->L * 4 * d->C);
    return WTC_OK;
}

int base_corr_partials(const wtc_desc* d, const void* x, const void* g, float* part, int* nblk, void*) {
    const size_t n = (size_t)d->B * d->C * d->H * d->W * (d->dtype == WTC_BF16 ? 2 : 4);
    rd(x, n);
    rd(g, n);
    *nblk = unfused_corr_blocks(d->B, d->C, d->H, d->W);
    wr(part, sizeof(float) * (size_t)*nblk * d->C * (d->k * d->k + 1));
    return WTC_OK;
}

int launch_corr0_mfma(const wtc_desc* d, const void* x, const void* g, float* part, int nchunk, void*) {
    need(d->dtype == WTC_BF16 && d->k <= kMaxK && d->H <= 64 && d->W <= 64 && nchunk >= 1, "matrix-core correlation");
    const size_t n = (size_t)d->B * d->C * d->H * d->W * 2;
    rd(x, n);
    rd(g, n);
    wr(part, sizeof(float) * (size_t)nchunk * d->C * (d->k * d->k + 1));
    return WTC_OK;
}

int launch_corr_sum(const float* part, int C, int nblk, int kk1, int kk, float* out, void*) {
    rd(part, sizeof(float) * (size_t)nblk * C * kk1);
    wr(out, sizeof(float) * (size_t)C * kk);
    return WTC_OK;
}

int launch_fill_zero(float* p, int n, void*) {
    wr(p, sizeof(float) * (size_t)(n > 0 ? n : 0));
    return 0;
}

int launch_transpose(const void* src, void* dst, int batch, int rows, int cols, int esize, void*) {
    const size_t n = (size_t)batch * rows * cols * esize;
    rd(src, n);
    wr(dst, n);
    return 0;
}

}  // namespace wtc
