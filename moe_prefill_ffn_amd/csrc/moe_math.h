// fp32 exponential of the SwiGLU and the router weights, compiled for the device
// (the kernels) and for the host (the library's host self-check entry point), so
// one source gives the same bits on both.
#pragma once

#include <stdint.h>

#include "moe_layout.h"

namespace moe {

// Cody-Waite reduction (Cody & Waite, "Software Manual for the Elementary
// Functions", 1980) with ln2 split into fp32 hi/lo parts, a degree-7 Taylor
// polynomial (coefficients 1/j! rounded to fp32) in Horner form, and the scale
// 2^n applied as two exact power-of-two factors.  Each step is a single IEEE
// fp32 operation, so the result is reproducible bit for bit.
MOE_HD static inline float pow2_exact(int n)  // n in [-126, 127]
{
    return __builtin_bit_cast(float, (uint32_t)(n + 127) << 23);
}

MOE_HD static inline float exp_cw(float x)
{
    if (x != x) return x;
    if (x > 89.0f) return __builtin_bit_cast(float, 0x7f800000u);
    if (x < -104.0f) return 0.0f;
    const float n = __builtin_rintf(x * 0x1.715476p+0f);     // x * log2(e)
    float r = __builtin_fmaf(-n, 0x1.62e430p-1f, x);          // - n * ln2_hi
    r = __builtin_fmaf(-n, -0x1.05c610p-29f, r);              // - n * ln2_lo
    float p = 0x1.a01a02p-13f;                                // 1/7!
    p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);                // 1/6!
    p = __builtin_fmaf(p, r, 0x1.111112p-7f);                 // 1/5!
    p = __builtin_fmaf(p, r, 0x1.555556p-5f);                 // 1/4!
    p = __builtin_fmaf(p, r, 0x1.555556p-3f);                 // 1/3!
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    const int ni = (int)n;
    const int n1 = ni / 2;
    const int n2 = ni - n1;
    return (p * pow2_exact(n1)) * pow2_exact(n2);
}

}  // namespace moe
