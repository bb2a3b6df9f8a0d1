// Shape sweep of libwtconv's host side (argument checks, launch planning,
// level peeling, workspace layout, channels-last adapter, I/O and flop
// models) for the sanitizer build: every entry point that can run without a
// GPU is called with buffers of exactly the sizes the library asks for, the
// kernel launchers being the stand-ins of planner_stubs.cpp.  Exits non-zero
// (or is stopped by the sanitizers) on the first inconsistency.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "wtconv.h"

namespace {

struct Buf {
    void* p = nullptr;
    explicit Buf(size_t n) { p = n ? std::malloc(n) : nullptr; if (p) std::memset(p, 0, n); }
    ~Buf() { std::free(p); }
    float* f() const { return static_cast<float*>(p); }
};

int fails = 0;
void expect(bool ok, const char* what, const wtc_desc& d) {
    if (ok) return;
    ++fails;
    std::fprintf(stderr, "FAIL %s: B=%d C=%d H=%d W=%d L=%d k=%d dtype=%d layout=%d\n", what, d.B, d.C, d.H, d.W, d.L,
                 d.k, d.dtype, d.layout);
}

// one shape through every host-reachable entry point; returns 1 if it ran
int one(const wtc_desc& d) {
    const size_t e = d.dtype == WTC_BF16 ? 2 : 4;
    const size_t n = (size_t)d.B * d.C * d.H * d.W * e;
    const int KK = d.k * d.k;
    Buf x(n), g(n), out(n), dx(n);
    Buf w0(sizeof(float) * d.C * KK), s0(sizeof(float) * d.C), b0(sizeof(float) * d.C);
    Buf wl(sizeof(float) * (size_t)d.L * 4 * d.C * KK), sl(sizeof(float) * (size_t)d.L * 4 * d.C);
    Buf dw0(sizeof(float) * d.C * KK), ds0(sizeof(float) * d.C), db0(sizeof(float) * d.C);
    Buf dwl(sizeof(float) * (size_t)d.L * 4 * d.C * KK), dsl(sizeof(float) * (size_t)d.L * 4 * d.C);
    const float* wlp = d.L ? wl.f() : nullptr;
    const float* slp = d.L ? sl.f() : nullptr;
    float* dwlp = d.L ? dwl.f() : nullptr;
    float* dslp = d.L ? dsl.f() : nullptr;
    int ran = 0;
    for (int impl = 0; impl < 2; ++impl) {
        const size_t wf = impl ? wtconv_forward_unfused_workspace(&d) : wtconv_forward_workspace(&d);
        const size_t wb = impl ? wtconv_backward_unfused_workspace(&d) : wtconv_backward_workspace(&d);
        Buf wsf(wf), wsb(wb);
        int st = impl ? wtconv_forward_unfused(&d, x.p, w0.f(), s0.f(), b0.f(), wlp, slp, out.p, wsf.p, wf, nullptr)
                      : wtconv_forward(&d, x.p, w0.f(), s0.f(), b0.f(), wlp, slp, out.p, wsf.p, wf, nullptr);
        expect(st == WTC_OK || st == WTC_ESHAPE, "forward status", d);
        if (st == WTC_OK) {
            ++ran;
            if (wf > 0) {   // one byte short of the queried size is refused
                st = impl ? wtconv_forward_unfused(&d, x.p, w0.f(), s0.f(), b0.f(), wlp, slp, out.p, wsf.p, wf - 1,
                                                   nullptr)
                          : wtconv_forward(&d, x.p, w0.f(), s0.f(), b0.f(), wlp, slp, out.p, wsf.p, wf - 1, nullptr);
                expect(st == WTC_EWORKSPACE, "forward short workspace", d);
            }
            const double m = wtconv_io_model_bytes(&d, impl, 0);
            expect(m >= (double)(2 * n), "forward I/O model", d);
        }
        st = impl ? wtconv_backward_unfused(&d, x.p, g.p, w0.f(), s0.f(), wlp, slp, dx.p, dw0.f(), ds0.f(), db0.f(),
                                            dwlp, dslp, wsb.p, wb, nullptr)
                  : wtconv_backward(&d, x.p, g.p, w0.f(), s0.f(), wlp, slp, dx.p, dw0.f(), ds0.f(), db0.f(), dwlp,
                                    dslp, wsb.p, wb, nullptr);
        expect(st == WTC_OK || st == WTC_ESHAPE, "backward status", d);
        if (st == WTC_OK) {
            ++ran;
            expect(wb > 0, "backward needs a workspace", d);
            st = impl ? wtconv_backward_unfused(&d, x.p, g.p, w0.f(), s0.f(), wlp, slp, dx.p, dw0.f(), ds0.f(),
                                                db0.f(), dwlp, dslp, wsb.p, wb - 1, nullptr)
                      : wtconv_backward(&d, x.p, g.p, w0.f(), s0.f(), wlp, slp, dx.p, dw0.f(), ds0.f(), db0.f(),
                                        dwlp, dslp, wsb.p, wb - 1, nullptr);
            expect(st == WTC_EWORKSPACE, "backward short workspace", d);
            const double m = wtconv_io_model_bytes(&d, impl, 1);
            expect(m >= (double)(3 * n), "backward I/O model", d);
        }
    }
    expect(wtconv_flops(&d, 0) > 0 && wtconv_flops(&d, 1) > wtconv_flops(&d, 0), "flops", d);
    // the base-level correlation alone, both implementations where they apply
    for (int impl = 0; impl < 2; ++impl) {
        const size_t wc = wtconv_base_correlation_workspace(&d, impl);
        Buf wsc(wc), c0(sizeof(float) * d.C * KK);
        const int st = wtconv_base_correlation(&d, x.p, g.p, c0.f(), impl, wsc.p, wc, nullptr);
        expect(st == WTC_OK || st == WTC_ESHAPE || st == WTC_EDTYPE, "base correlation status", d);
        if (st == WTC_OK) {
            ++ran;
            expect(wtconv_base_correlation(&d, x.p, g.p, c0.f(), impl, wsc.p, wc - 1, nullptr) == WTC_EWORKSPACE,
                   "base correlation short workspace", d);
        }
    }
    return ran;
}

}  // namespace

int main(int argc, char** argv) {
    const int ncase = argc > 1 ? std::atoi(argv[1]) : 400;
    std::mt19937 rng(12345);
    auto pick = [&](std::initializer_list<int> v) { return *(v.begin() + rng() % v.size()); };
    std::vector<wtc_desc> cases = {
        // the benchmark shapes with a small batch and channel count
        {2, 3, 32, 32, 2, 5, 0, 0},   {2, 3, 64, 64, 3, 5, 0, 0},   {2, 3, 32, 32, 3, 5, 1, 0},
        {2, 3, 128, 128, 1, 5, 0, 0}, {2, 3, 128, 128, 5, 5, 0, 0}, {3, 17, 14, 14, 2, 5, 0, 0},
        {70, 3, 7, 7, 1, 5, 0, 0},    {2, 3, 224, 224, 3, 5, 0, 0}, {1, 2, 300, 260, 4, 3, 0, 0},
        {1, 2, 257, 129, 9, 5, 0, 0}, {2, 2, 260, 130, 0, 7, 0, 0}, {2, 5, 64, 64, 3, 5, 0, 1},
        {1, 1, 1, 1, 3, 5, 0, 0},     {2, 4, 8, 8, 2, 5, 1, 0},     {1, 2, 600, 40, 2, 5, 0, 0},
        {2, 3, 33, 20, 2, 31, 0, 0},  {1, 2, 200, 150, 3, 9, 1, 1},
    };
    for (int i = 0; i < ncase; ++i) {
        wtc_desc d;
        d.B = pick({1, 2, 3, 5});
        d.C = pick({1, 2, 3, 16, 17});
        d.H = pick({1, 2, 3, 7, 8, 13, 14, 16, 31, 32, 40, 64, 100, 127, 128, 129, 150, 224});
        d.W = pick({1, 2, 5, 7, 8, 14, 17, 32, 33, 36, 64, 72, 100, 128, 130, 200});
        d.L = pick({0, 1, 2, 3, 4, 5, 6, 9});
        d.k = pick({1, 3, 5, 7, 9, 11});
        d.dtype = pick({0, 1});
        d.layout = (rng() % 8 == 0) ? 1 : 0;
        cases.push_back(d);
    }
    long ran = 0;
    for (const auto& d : cases) ran += one(d);
    // rejected descriptors
    wtc_desc bad = {2, 3, 16, 16, 2, 4, 0, 0};
    expect(wtconv_forward_workspace(&bad) == 0 && wtconv_io_model_bytes(&bad, 0, 0) < 0, "even k rejected", bad);
    std::printf("cases=%zu calls_ok=%ld fails=%d\n", cases.size(), ran, fails);
    return fails ? 1 : 0;
}
