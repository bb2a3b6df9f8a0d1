// The base level's weight-gradient correlation on its own,
//   C0[c][ky][kx] = sum_{b,p} g[b,c,p] x[b,c,p + (ky - k/2, kx - k/2)]   (x zero outside),
// as a matrix product on the gfx950 matrix cores for bfloat16 planes, and the
// fixed-order sum of correlation partials.
//
// Matrix form, J rows of g per product: for g rows y .. y + J - 1 and the 32
// pixel columns x0 .. x0 + 31 (the reduction index q),
//   A[(dx, j)][q] = g[y + j][x0 + q + dx - k/2]              (k J rows)
//   B[q][n]       = x[y + k/2 + J - 1 - n][x0 + q]           (k + J - 1 columns)
//   D[(dx, j)][n] = sum over the segment of g[p] x[p + (ky - k/2, kx - k/2)]
//                   with ky = 2 (k/2) + J - 1 - n - j, kx = 2 (k/2) - dx,
// so one v_mfma_f32_16x16x32_bf16 covers J pixel rows and every tap; each tap
// is the sum of the J entries (dx, j) that map to it.  J = 16, 5, 3, 2 for
// k = 1, 3, 5, 7 (k J <= 16, k + J - 1 <= 16).  bf16 products are exact in the
// fp32 accumulator, so this is the same sum as the vector-unit path up to the
// order of the additions.
#include <hip/hip_runtime.h>

#include "wtc_internal.h"

namespace wtc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int K>
struct CorrShape {
    static constexpr int R = K / 2;
    static constexpr int J = K == 1 ? 16 : K == 3 ? 5 : K == 5 ? 3 : 2;   // g rows per product
    static constexpr int M = K * J;                                      // rows of A in use
    static constexpr int N = K + J - 1;                                  // columns of B in use
    static_assert(M <= 16 && N <= 16, "one 16 x 16 product");
};

// LDS layout of one staged plane pair (16-bit elements), rows padded to whole
// products (Hp = J * ceil(H / J)) and columns to whole 32-pixel segments:
//   gs[r][8 + cc] = g[r][cc]          Hp rows of SG = Wp + 16  (8 zero columns each side and more)
//   xs[r][cc]     = x[r - k/2][cc]    Hp + 2 (k/2) rows of SX = Wp + 8
// Everything outside the plane stays zero from the workgroup's start.
struct CorrLds {
    int Wp, Hp, SG, SX, HX;
    __host__ __device__ CorrLds(int H, int W, int J, int R)
        : Wp((W + 31) & ~31), Hp((H + J - 1) / J * J), SG(Wp + 16), SX(Wp + 8), HX(Hp + 2 * R) {}
    __host__ __device__ int elems() const { return Hp * SG + HX * SX; }
};

// One 64-lane workgroup = one (batch chunk, channel) unit; it walks the
// chunk's planes one at a time, accumulating D in four registers per lane.
// VEC: W % 8 == 0 and 16-byte aligned tensors (16-byte staging loads).
template <int K, bool VEC>
__global__ void __launch_bounds__(64) k_corr0_mfma(const uint16_t* __restrict__ g, const uint16_t* __restrict__ x,
                                                   int B, int C, int H, int W, int ppc, float* __restrict__ part) {
    using S = CorrShape<K>;
    constexpr int R = S::R, J = S::J, KK = K * K;
    extern __shared__ __align__(16) uint16_t l16[];
    __shared__ float red[256];
    const int lane = threadIdx.x;
    const int c = blockIdx.x % C, chunk = blockIdx.x / C;
    const int b0 = chunk * ppc, b1 = min(B, b0 + ppc);
    const CorrLds lay(H, W, J, R);
    uint16_t* gs = l16;
    uint16_t* xs = l16 + lay.Hp * lay.SG;
    {
        uint32_t* z = reinterpret_cast<uint32_t*>(l16);
        for (int e = lane; e < lay.elems() / 2; e += 64) z[e] = 0u;
    }
    // this lane's A row (dx, j) and B column n; lanes past the used rows /
    // columns repeat the last one (valid LDS, results never read)
    const int m = lane & 15, kg = lane >> 4;
    const int mc = m < S::M ? m : S::M - 1, nc = m < S::N ? m : S::N - 1;
    const int dx = mc / J, j = mc - dx * J;
    const int aoff = j * lay.SG + 8 + 8 * kg + dx - R;   // + y SG + x0; parity fixed per lane
    const int aeven = aoff & ~1;
    const uint32_t sh = (uint32_t)(aoff & 1) * 16u;
    const int boff = (2 * R + J - 1 - nc) * lay.SX + 8 * kg;   // + y SX + x0; 16-byte aligned
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const size_t HW = (size_t)H * W;
    for (int b = b0; b < b1; ++b) {
        const uint16_t* gp = g + ((size_t)b * C + c) * HW;
        const uint16_t* xp = x + ((size_t)b * C + c) * HW;
        __syncthreads();   // zeroing done / the previous plane consumed
        if constexpr (VEC) {
            const int W8 = W >> 3, n8 = H * W8;
            for (int e = lane; e < n8; e += 64) {
                const int y = e / W8, cx = e - y * W8;
                const u32x4 gv = *reinterpret_cast<const u32x4*>(gp + 8 * (size_t)e);
                const u32x4 xv = *reinterpret_cast<const u32x4*>(xp + 8 * (size_t)e);
                *reinterpret_cast<u32x4*>(gs + y * lay.SG + 8 + 8 * cx) = gv;
                *reinterpret_cast<u32x4*>(xs + (y + R) * lay.SX + 8 * cx) = xv;
            }
        } else {
            for (int e = lane; e < H * W; e += 64) {
                const int y = e / W, cx = e - y * W;
                gs[y * lay.SG + 8 + cx] = gp[e];
                xs[(y + R) * lay.SX + cx] = xp[e];
            }
        }
        __syncthreads();
        for (int y = 0; y < lay.Hp; y += J) {
            const uint16_t* ga = gs + y * lay.SG + aeven;
            const uint16_t* xb = xs + y * lay.SX + boff;
            for (int x0 = 0; x0 < lay.Wp; x0 += 32) {
                const uint32_t* a32 = reinterpret_cast<const uint32_t*>(ga + x0);   // 4-byte aligned
                const uint32_t d0 = a32[0], d1 = a32[1], d2 = a32[2], d3 = a32[3], d4 = a32[4];
                u32x4 av;
                av.x = __builtin_amdgcn_alignbit(d1, d0, sh);
                av.y = __builtin_amdgcn_alignbit(d2, d1, sh);
                av.z = __builtin_amdgcn_alignbit(d3, d2, sh);
                av.w = __builtin_amdgcn_alignbit(d4, d3, sh);
                const u32x4 bv = *reinterpret_cast<const u32x4*>(xb + x0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                             __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
            }
        }
    }
    // D[4 kg + r][n] -> red; tap (ky, kx) = sum over j of D[(2R - kx, j)][2R + J - 1 - ky - j]
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(4 * kg + r) * 16 + m] = acc[r];
    __syncthreads();
    if (lane <= KK) {
        float v = 0.f;
        if (lane < KK) {
            const int ky = lane / K, kx = lane - ky * K, ddx = 2 * R - kx;
#pragma unroll
            for (int jj = 0; jj < J; ++jj) v += red[(ddx * J + jj) * 16 + (2 * R + J - 1 - ky - jj)];
        }
        part[((size_t)chunk * C + c) * (KK + 1) + lane] = v;   // slot KK (sum of g) is not computed here
    }
}

// out[c][t] = sum over blocks of part[blk][c][t], t < kk (fixed order)
__global__ void __launch_bounds__(64) k_corr_sum(const float* __restrict__ part, int C, int nblk, int kk1, int kk,
                                                 float* __restrict__ out) {
    const int c = blockIdx.x;
    for (int t = threadIdx.x; t < kk; t += 64) {
        float v = 0.f;
        for (int b = 0; b < nblk; ++b) v += part[((size_t)b * C + c) * kk1 + t];
        out[(size_t)c * kk + t] = v;
    }
}

template <int K>
int corr0_mfma_t(const wtc_desc* d, const void* x, const void* g, float* part, int nchunk, hipStream_t st) {
    const int ppc = (d->B + nchunk - 1) / nchunk;
    const CorrLds lay(d->H, d->W, CorrShape<K>::J, K / 2);
    const size_t lds = (size_t)lay.elems() * sizeof(uint16_t);   // <= 21 KB for planes up to 64 x 64
    const bool vec = d->W % 8 == 0 && ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(g)) & 15) == 0;
    const dim3 grid((unsigned)(nchunk * d->C)), block(64);
    const uint16_t* gp = static_cast<const uint16_t*>(g);
    const uint16_t* xp = static_cast<const uint16_t*>(x);
    if (vec)
        hipLaunchKernelGGL((k_corr0_mfma<K, true>), grid, block, lds, st, gp, xp, d->B, d->C, d->H, d->W, ppc, part);
    else
        hipLaunchKernelGGL((k_corr0_mfma<K, false>), grid, block, lds, st, gp, xp, d->B, d->C, d->H, d->W, ppc, part);
    return hipGetLastError() == hipSuccess ? WTC_OK : WTC_EHIP;
}

}  // namespace

int launch_corr0_mfma(const wtc_desc* d, const void* x, const void* g, float* part, int nchunk, void* stream) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    switch (d->k) {
        case 1: return corr0_mfma_t<1>(d, x, g, part, nchunk, st);
        case 3: return corr0_mfma_t<3>(d, x, g, part, nchunk, st);
        case 5: return corr0_mfma_t<5>(d, x, g, part, nchunk, st);
        case 7: return corr0_mfma_t<7>(d, x, g, part, nchunk, st);
        default: return WTC_ESHAPE;
    }
}

int launch_corr_sum(const float* part, int C, int nblk, int kk1, int kk, float* out, void* stream) {
    hipLaunchKernelGGL(k_corr_sum, dim3((unsigned)C), dim3(64), 0, reinterpret_cast<hipStream_t>(stream), part, C,
                       nblk, kk1, kk, out);
    return hipGetLastError() == hipSuccess ? WTC_OK : WTC_EHIP;
}

}  // namespace wtc
