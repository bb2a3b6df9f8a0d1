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
// On the device gfx950 converts with the same rounding in one instruction
// (v_cvt_pk_bf16_f32, two values at a time); its NaN results are quiet NaNs
// too, whose payload may differ from the host's.
WTC_HD uint16_t bf16_rne(float v) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_bit_cast(uint16_t, (__bf16)v);
#else
    const uint32_t u = f32_bits(v);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
#endif
}

// Two float32 -> two bfloat16 with bf16_rne's rounding, a in the low half.
WTC_HD uint32_t bf16x2_rne(float a, float b) {
#if defined(__HIP_DEVICE_COMPILE__)
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
#else
    return (uint32_t)bf16_rne(a) | ((uint32_t)bf16_rne(b) << 16);
#endif
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
// A divisor the compiler knows (fixed plane geometry) that is a power of two
// becomes a shift.
WTC_HD int fdiv(int e, const FastDiv& f) {
#if defined(__HIP_DEVICE_COMPILE__)
    if (__builtin_constant_p(f.d) && f.d > 0 && (f.d & (f.d - 1)) == 0) return e >> __builtin_ctz(f.d);
#endif
    return (int)((float)e * f.r);
}

}  // namespace wtc
