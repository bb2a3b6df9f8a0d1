// Layout adapter for channels-last (NHWC) tensors: a batched transpose through
// LDS, [batch][rows][cols] -> [batch][cols][rows].  NHWC -> NCHW is rows = H*W,
// cols = C; NCHW -> NHWC is rows = C, cols = H*W.  Both sides are read and
// written in whole 64-element row segments (coalesced); the LDS tile is padded
// by one element per row so the transposed reads hit distinct banks.
#include <hip/hip_runtime.h>

#include "wtc_internal.h"

namespace wtc {
namespace {

constexpr int kTile = 64;

template <typename T>
__global__ void __launch_bounds__(256) k_transpose(const T* __restrict__ src, T* __restrict__ dst, int rows,
                                                   int cols) {
    __shared__ T tile[kTile][kTile + 1];
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    const int r0 = blockIdx.y * kTile, c0 = blockIdx.x * kTile;
    const size_t base = (size_t)blockIdx.z * rows * cols;
#pragma unroll
    for (int i = 0; i < kTile / 4; ++i) {
        const int r = r0 + ty + 4 * i, c = c0 + tx;
        if (r < rows && c < cols) tile[ty + 4 * i][tx] = src[base + (size_t)r * cols + c];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kTile / 4; ++i) {
        const int c = c0 + ty + 4 * i, r = r0 + tx;
        if (c < cols && r < rows) dst[base + (size_t)c * rows + r] = tile[tx][ty + 4 * i];
    }
}

// Same transpose with 16-byte accesses on both sides, for tensors whose rows
// and columns are multiples of VW = 16 / sizeof(T) elements and 16-byte
// aligned: a 64 x 64 tile is read as 64 / VW vectors per row (4 VW rows per
// pass) and written the same way along the other dimension.  Fewer, wider
// memory requests: one per 16 bytes instead of one per element.
template <typename T>
__global__ void __launch_bounds__(256) k_transpose_v(const T* __restrict__ src, T* __restrict__ dst, int rows,
                                                     int cols) {
    constexpr int VW = 16 / sizeof(T), TPR = kTile / VW, RPP = 256 / TPR;
    typedef uint32_t vec_t __attribute__((ext_vector_type(4)));
    __shared__ T tile[kTile][kTile + 1];
    const int vx = threadIdx.x % TPR, ry = threadIdx.x / TPR;
    const int r0 = blockIdx.y * kTile, c0 = blockIdx.x * kTile;
    const size_t base = (size_t)blockIdx.z * rows * cols;
#pragma unroll
    for (int i = 0; i < kTile / RPP; ++i) {
        const int r = r0 + ry + RPP * i, c = c0 + VW * vx;
        if (r < rows && c < cols) {
            union { vec_t v; T e[VW]; } u;
            u.v = *reinterpret_cast<const vec_t*>(src + base + (size_t)r * cols + c);
#pragma unroll
            for (int j = 0; j < VW; ++j) tile[ry + RPP * i][VW * vx + j] = u.e[j];
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kTile / RPP; ++i) {
        const int c = c0 + ry + RPP * i, r = r0 + VW * vx;
        if (c < cols && r < rows) {
            union { vec_t v; T e[VW]; } u;
#pragma unroll
            for (int j = 0; j < VW; ++j) u.e[j] = tile[VW * vx + j][ry + RPP * i];
            *reinterpret_cast<vec_t*>(dst + base + (size_t)c * rows + r) = u.v;
        }
    }
}

}  // namespace

int launch_transpose(const void* src, void* dst, int batch, int rows, int cols, int esize, void* stream) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const dim3 grid((cols + kTile - 1) / kTile, (rows + kTile - 1) / kTile, batch);
    if (grid.y > 65535 || grid.z > 65535) return (int)hipErrorInvalidValue;
    const int vw = 16 / esize;
    const bool vec = rows % vw == 0 && cols % vw == 0 &&
                     ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0;
    if (esize == 4) {
        if (vec)
            hipLaunchKernelGGL(k_transpose_v<uint32_t>, grid, dim3(256), 0, st, static_cast<const uint32_t*>(src),
                               static_cast<uint32_t*>(dst), rows, cols);
        else
            hipLaunchKernelGGL(k_transpose<uint32_t>, grid, dim3(256), 0, st, static_cast<const uint32_t*>(src),
                               static_cast<uint32_t*>(dst), rows, cols);
    } else {
        if (vec)
            hipLaunchKernelGGL(k_transpose_v<uint16_t>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(src),
                               static_cast<uint16_t*>(dst), rows, cols);
        else
            hipLaunchKernelGGL(k_transpose<uint16_t>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(src),
                               static_cast<uint16_t*>(dst), rows, cols);
    }
    return (int)hipGetLastError();
}

}  // namespace wtc
