// Numeric helpers shared by every kernel file and compiled on the host by the
// CPU tests: float32 -> bfloat16 rounding, and integer division by a
// loop-invariant divisor through a float reciprocal.
#pragma once

#include <stdint.h>
#include <string.h>

#if defined(__HIPCC__)
#define WTC_HD __host__ __device__ __forceinline__
#else
#define WTC_HD inline
#endif

namespace wtc {

WTC_HD uint32_t f32_bits(float v) {
    uint32_t u;
    memcpy(&u, &v, sizeof(u));
    return u;
}

// float32 -> bfloat16 bits, round to nearest, ties to even; values beyond the
// largest bfloat16 round to infinity.  A NaN stays a NaN (sign and top payload
// bits kept, quiet bit set): the rounding add would otherwise carry a NaN's
// payload into the exponent (giving infinity) or wrap it to zero.
WTC_HD uint16_t bf16_rne(float v) {
    const uint32_t u = f32_bits(v);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Integer division e / d for 0 <= e < 2^16 and a loop-invariant 1 <= d < 2^16
// with e < d or d <= 32768, by a float reciprocal biased up by 2^-17: three
// full-rate VALU operations instead of the ~15-operation integer division.
// Exact over that whole range, also with the reciprocal one ulp off either
// way (checked exhaustively by the CPU tests on this very code).
struct FastDiv {
    int d;
    float r;
};
WTC_HD FastDiv make_div(int d) {
    FastDiv f;
    f.d = d;
    f.r = (1.0f / (float)d) * 1.0000076f;   // 1 + 2^-17
    return f;
}
WTC_HD int fdiv(int e, const FastDiv& f) { return (int)((float)e * f.r); }

}  // namespace wtc
