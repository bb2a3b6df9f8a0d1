// Host-side planning shared by the dispatcher and the kernel launchers: the
// level-by-level baseline's workspace layout and correlation split, and the
// record count of the peeled top level.  Plain C++ (no device code), so the
// CPU tests can build it, with the dispatcher, under the host sanitizers.
#include <algorithm>

#include "wtc_internal.h"

namespace wtc {
namespace {

size_t align256_host(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

int unfused_corr_blocks(int nb, int nch, int h, int w) {
    // large planes: units are (batch entry, tile) pairs
    const int units = unfused_big_planes(h, w) ? nb * ((h + kUnfusedBigTile - 1) / kUnfusedBigTile) *
                                                     ((w + kUnfusedBigTile - 1) / kUnfusedBigTile)
                                               : nb;
    return std::max(1, std::min(units, (kUnfusedCorrTarget + nch - 1) / nch));
}

size_t top_records(const wtc_desc* d) {
    const size_t ntile = (size_t)((d->W + kTopTile - 1) / kTopTile) * ((d->H + kTopTile - 1) / kTopTile);
    return (size_t)d->B * ntile * d->C * (d->k * d->k + 1);
}

// Workspace (float32 tensors, 256-byte aligned).  Per level i:
//   S_i  [B, C, 4, h_i, w_i]       bands of x
//   Y_i  same shape                forward: scaled conv output;  backward: dS_i
//   Z_i  [B, C, h_{i-1}, w_{i-1}]  forward: partial synthesis;  backward: dLL_{i-1}
//   dT_i same shape as S_i         backward only: analysis of g
// then the correlation partials (backward).
int unfused_plan(const wtc_desc* d, int bwd, UnfusedPlan* p) {
    if (d->k > kMaxKAny) return WTC_ESHAPE;
    if (d->L > kMaxUnfusedL) return WTC_ESHAPE;
    const uint64_t BC = (uint64_t)d->B * d->C;
    // 32-bit element indexing of every tensor (the level-1 bands are the largest)
    const uint64_t h1 = (d->H + 1) / 2, w1 = (d->W + 1) / 2;
    if (BC * d->H * d->W >= (1ull << 31) || BC * 4 * h1 * w1 >= (1ull << 31)) return WTC_ESHAPE;
    p->h[0] = d->H;
    p->w[0] = d->W;
    size_t off = 0;
    for (int i = 1; i <= d->L; ++i) {
        p->h[i] = (p->h[i - 1] + 1) / 2;
        p->w[i] = (p->w[i - 1] + 1) / 2;
        const size_t n4 = BC * 4 * p->h[i] * p->w[i] * sizeof(float);
        const size_t nz = BC * p->h[i - 1] * p->w[i - 1] * sizeof(float);
        p->s_off[i] = off;
        off += align256_host(n4);
        p->y_off[i] = off;
        off += align256_host(n4);
        p->z_off[i] = off;
        off += align256_host(nz);
        if (bwd) {
            p->dt_off[i] = off;
            off += align256_host(n4);
        }
    }
    p->part_off = off;
    if (bwd) {
        const int kk1 = d->k * d->k + 1;
        size_t np = (size_t)unfused_corr_blocks(d->B, d->C, d->H, d->W) * d->C * kk1;
        for (int i = 1; i <= d->L; ++i)
            np = std::max(np, (size_t)unfused_corr_blocks(d->B, 4 * d->C, p->h[i], p->w[i]) * 4 * d->C * kk1);
        off += align256_host(np * sizeof(float));
    }
    p->total = off;
    return WTC_OK;
}

}  // namespace wtc
