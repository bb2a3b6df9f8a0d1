/*
 * wtconv.h -- C ABI of libwtconv, the MI355X (gfx950) WTConv operator.
 *
 * WTConv ("Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware
 * Reformulation", arXiv 2608.10805, Abstract) is a multi-level 2-D Haar
 * wavelet convolution:
 *
 *   LL_0 = x;  for i = 1..L:  (S_i^0..S_i^3) = orthonormal 2x2 Haar analysis of
 *              LL_{i-1} (zero-padded right/bottom to even size), LL_i = S_i^0
 *   Y_i   = s_i * dwconv_k(S_i, W_i)       (4C subband-channels 4c+u, zero pad k/2)
 *   Z_{L+1} = 0,  Z_i = inverse Haar(Y_i^0 + Z_{i+1}, Y_i^1, Y_i^2, Y_i^3),
 *                 cropped to the size of LL_{i-1}
 *   out   = s0 * dwconv_k(x, W0) + b0 + Z_1
 *
 * Subband u = 2*u_y + u_x: u_x = 1 is high-pass along W, u_y = 1 along H.
 * dwconv is cross-correlation: (W * X)[p] = sum_d W[d + k/2] X[p + d].
 *
 * The library computes the operator with the three reformulations that
 * abstract names: the Haar analysis is recomputed on chip, the synthesis
 * cascade is evaluated as one closed-form pass indexed by output-coordinate
 * bits, and the scales are folded into the convolution weights.  The
 * "_unfused" entry points run the same operator level by level, one kernel
 * per step, with every intermediate in device memory (the baseline the
 * abstract compares against).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees or synchronises on these paths; calls
 *     are asynchronous on `stream` (a hipStream_t; NULL = default stream).
 *   - x, out, g (= d loss / d out) and dx are [B, C, H, W], NCHW contiguous
 *     (layout 0) or channels-last [B, H, W, C] contiguous (layouts 1 and 2),
 *     stored as float32 (dtype WTC_FP32) or bfloat16 bits (WTC_BF16; out and
 *     dx are rounded to nearest even).  All arithmetic is float32.
 *     Layout 1 (channels-last, fastest): the tensors are transposed into NCHW
 *     copies at the front of the workspace, computed there and transposed
 *     back (two extra tensors of workspace forward, three backward; four and
 *     six extra tensor passes of traffic).
 *     Layout 2 (channels-last, in place): the fused kernels read and write
 *     the tensors where they are -- no copies, no extra workspace, HBM
 *     traffic as for NCHW -- for every plane the on-chip pipeline holds (about
 *     128 x 128 at k = 5, k <= 7); slower than layout 1, because each pixel of
 *     a channel is a separate cache-line request.  Beyond those planes layout
 *     2 is adapted like layout 1.  The level-by-level entry points adapt both.
 *   - Parameters and their gradients are float32:
 *       w0 [C, k, k] (PyTorch depthwise [C,1,k,k] order), s0 [C], b0 [C],
 *       wl [L, 4C, k, k] with flat index ((l*C + c)*4 + u)*k*k + ky*k + kx,
 *       sl [L, 4C]       with flat index  (l*C + c)*4 + u.
 *     wl and sl may be NULL when L == 0.
 *   - Outputs are overwritten, never accumulated.
 *   - Arguments are checked before any HIP call; a failed check returns a
 *     negative wtc_status and touches nothing.  A failed kernel launch
 *     returns WTC_EHIP.  No C++ exception crosses this interface.
 *   - Calls with the same workspace must not overlap in time.
 */
#ifndef WTCONV_H
#define WTCONV_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    WTC_OK = 0,
    WTC_EINVAL = -1,     /* null pointer, k even or < 1, L < 0, B/C/H/W < 1, bad impl/dir */
    WTC_ESHAPE = -2,     /* k > 31, or a tensor of 2^31 elements or more */
    WTC_EDTYPE = -3,     /* dtype or layout not supported (layout > 2) */
    WTC_EWORKSPACE = -4, /* workspace NULL or smaller than the queried size */
    WTC_EHIP = -5,       /* a HIP launch or runtime call failed */
    WTC_ESCRATCH = -6    /* wtconv_backward_noalloc: the call needs more than
                            WTCONV_NOALLOC_SCRATCH_BYTES of scratch */
} wtc_status;

typedef enum { WTC_FP32 = 0, WTC_BF16 = 1 } wtc_dtype;

typedef struct {
    int B, C, H, W; /* batch, channels, height, width (all >= 1)              */
    int L;          /* wavelet levels (>= 0)                                  */
    int k;          /* kernel size: odd, 1..31 (fused kernels for k <= 7)     */
    int dtype;      /* wtc_dtype: storage type of x / out / g / dx           */
    int layout;     /* 0 = NCHW, 1 = channels-last, 2 = channels-last in place */
} wtc_desc;

/* Bytes of device workspace wtconv_forward needs (0: none).  It is 0 for every
 * plane the on-chip pipeline holds (up to about 128 x 128 with k = 5); larger
 * planes peel one wavelet level (below) and need float32 tensors of their
 * LL band and deeper result (L = 0: the level-by-level depthwise conv's
 * intermediates).  0 is also returned for a
 * descriptor that the forward pass rejects. */
size_t wtconv_forward_workspace(const wtc_desc* d);

/* Forward pass: out = WTConv(x).  `workspace` may be NULL when the queried
 * size is 0.
 * Kernel sizes 9..31 have no fused kernels (their k^2 weights and correlation
 * accumulators per lane exceed the register file): such calls run the
 * level-by-level kernels below with the taps looped at run time, and the
 * workspace queries and the I/O model count that path.  Same results, same
 * contract.
 * Planes beyond the on-chip pipeline: the levels >= 2 of the operator are the
 * operator itself (one level fewer, no base conv) applied to the level-1 LL
 * band, so the LL band (half the size per side) runs recursively through this
 * path -- on chip as soon as it fits -- and level 1 and the base conv run
 * fused over 64 x 64 tiles of the full-resolution plane (L = 0: the
 * level-by-level depthwise conv).  Same results, same contract. */
int wtconv_forward(const wtc_desc* d, const void* x,
                   const float* w0, const float* s0, const float* b0,
                   const float* wl, const float* sl,
                   void* out, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace wtconv_backward needs (per-workgroup partial
 * sums of the weight-gradient correlations; for planes beyond the on-chip
 * pipeline the per-tile correlation records of the peeled level and the
 * tensors of the LL problem). */
size_t wtconv_backward_workspace(const wtc_desc* d);

/* Backward pass: given g = d loss / d out, writes
 *   dx  [B,C,H,W]   (same storage dtype as x)
 *   dw0 [C,k,k], ds0 [C], db0 [C], dwl [L,4C,k,k], dsl [L,4C]  (float32;
 *   dwl/dsl may be NULL when L == 0).
 * Weight gradients are with respect to the unscaled weights W0 and W_i.
 * The reduction over batch and space is deterministic (fixed order). */
int wtconv_backward(const wtc_desc* d, const void* x, const void* g,
                    const float* w0, const float* s0,
                    const float* wl, const float* sl,
                    void* dx, float* dw0, float* ds0, float* db0,
                    float* dwl, float* dsl,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Backward pass that allocates nothing and takes no workspace, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments, results
 * and checks as wtconv_backward without the workspace pair; the scratch that
 * wtconv_backward takes from the workspace (the weight-gradient partial
 * records) is a fixed array of WTCONV_NOALLOC_SCRATCH_BYTES in device memory,
 * one per GPU, held from the first call on that GPU until the process ends.
 * Runs on the device current at the call (the one of `stream` and the
 * tensors).  A call whose wtconv_backward_workspace(d) exceeds the array
 * returns WTC_ESCRATCH before any HIP call: planes beyond the on-chip
 * pipeline (above about 128 x 128 at k = 5) and channels-last tensors through
 * NCHW copies (layout 1) need far more; layout 2 fits.  Nothing in the array has to start at zero (every record is
 * written before it is read), but all calls on one GPU share it: calls that
 * overlap in time on one GPU (two streams, or two threads) race and must be
 * serialised by the caller.  The first call on a device also looks up the
 * array's device address (hipGetSymbolAddress), which is not an allocation. */
#define WTCONV_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int wtconv_backward_noalloc(const wtc_desc* d, const void* x, const void* g,
                            const float* w0, const float* s0,
                            const float* wl, const float* sl,
                            void* dx, float* dw0, float* ds0, float* db0,
                            float* dwl, float* dsl, void* stream);

/* The base level's weight-gradient correlation on its own,
 *   c0[c][ky][kx] = sum_{b,p} g[b,c,p] * x[b,c,p + (ky - k/2, kx - k/2)]   (x zero outside),
 * so that dW0 = s0 * c0 (the correlation the backward pass reduces for the base
 * depthwise convolution of the operator; "Fast and Memory-Efficient Wavelet
 * Convolutions via I/O-Aware Reformulation", arXiv 2608.10805, Abstract).  Two
 * implementations of the same sum, for comparing the vector units with the
 * matrix cores (the windowed batched-matmul formulation of a depthwise
 * convolution: "WBMM: Windowed Batch Matrix Multiplication ..." review,
 * core claim):
 *   impl 0: the level-by-level baseline's register-blocked correlation tiles
 *           on the vector units (any dtype, k <= 31);
 *   impl 1: the gfx950 matrix cores, one 16 x 16 x 32 bf16 product per
 *           32-pixel segment of J rows (J = 16, 5, 3, 2 for k = 1, 3, 5, 7)
 *           accumulating every tap (dtype WTC_BF16 -- exact products --,
 *           k <= 7, H and W <= 64).
 * NCHW only (layout 0).  x, g device tensors as in wtconv_backward; c0
 * [C, k, k] float32, overwritten; the workspace (partial sums) is queried per
 * impl.  Deterministic.  WTC_EDTYPE / WTC_ESHAPE outside a path's limits,
 * WTC_EINVAL for another impl. */
size_t wtconv_base_correlation_workspace(const wtc_desc* d, int impl);
int wtconv_base_correlation(const wtc_desc* d, const void* x, const void* g, float* c0, int impl,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Level-by-level baseline: one kernel per step, every intermediate (bands,
 * convolved bands, partial syntheses) a float32 tensor in the workspace.
 * Same arguments and results as above.  It accepts any plane size but
 * returns WTC_ESHAPE for k > 31, L > 30, or tensors of 2^31 elements or more
 * (32-bit indexing).  Its weight-gradient reduction is also deterministic.
 * The forward workspace is 0 bytes when L == 0. */
size_t wtconv_forward_unfused_workspace(const wtc_desc* d);
int wtconv_forward_unfused(const wtc_desc* d, const void* x,
                           const float* w0, const float* s0, const float* b0,
                           const float* wl, const float* sl,
                           void* out, void* workspace, size_t workspace_bytes, void* stream);
size_t wtconv_backward_unfused_workspace(const wtc_desc* d);
int wtconv_backward_unfused(const wtc_desc* d, const void* x, const void* g,
                            const float* w0, const float* s0,
                            const float* wl, const float* sl,
                            void* dx, float* dw0, float* ds0, float* db0,
                            float* dwl, float* dsl,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Analytic model of device-memory (HBM) traffic in bytes for one call:
 * impl 0 = fused, 1 = unfused; dir 0 = forward, 1 = backward.  The pages
 * build an I/O model of WTConv to show where its time goes ("Fast and
 * Memory-Efficient Wavelet Convolutions via I/O-Aware Reformulation", arXiv
 * 2608.10805, Abstract); their equations are not given, so this model is the
 * library's own: every tensor counted once per kernel that reads or writes it
 * (fused forward 2 N e, backward 3 N e, plus parameters and partial records;
 * the level-by-level path adds every band and partial synthesis).
 * Returns a negative value for an invalid descriptor or impl/dir. */
double wtconv_io_model_bytes(const wtc_desc* d, int impl, int dir);

/* Algorithmic floating-point operations of one call (an FMA counts 2),
 * dir 0 = forward, 1 = backward; negative for an invalid descriptor.  Counted
 * from the operator's definition (same Abstract): the base k x k depthwise
 * convolution, per level the four subband k x k convolutions and the 2 x 2
 * analysis and synthesis butterflies; the backward repeats the convolutions
 * for dx and once more for the weight-gradient correlations, plus the analysis
 * of x. */
double wtconv_flops(const wtc_desc* d, int dir);

/* Static description of a status code (library convention, no passage). */
const char* wtconv_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* WTCONV_H */
