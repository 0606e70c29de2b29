// NVFP4 pieces shared by the quantiser and the expert kernels (not part of
// the ABI).  NVFP4 release card, precision table: routed experts W4A4, FP4
// (E2M1) values in groups of 16 with FP8 (E4M3) block scales and FP32 global
// scales; the rounding rules below are this library's reading.
#pragma once

#include "common.h"

namespace moe {

// Value of an OCP E4M3 code (finite codes only): exponent field 0 is
// subnormal, m * 2^-9; otherwise (8 + m) * 2^(e - 10).
__device__ __forceinline__ float e4m3_val(uint32_t c) {
    const int ex = (c >> 3) & 15, m = c & 7;
    const float v = ex == 0 ? (float)m * 0.001953125f : ldexpf((float)(8 + m), ex - 10);
    return (c & 0x80) ? -v : v;
}

// Nearest E4M3 code of f >= 0, ties to even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_rne(float f) {
    if (!(f > 0.0f)) return 0;
    if (f >= 448.0f) return 0x7E;
    const uint32_t b = __float_as_uint(f);
    const int E = (int)(b >> 23) - 127;
    if (E >= -6) {  // normal in E4M3: keep 3 of the 23 mantissa bits
        const uint32_t m = b & 0x7FFFFFu;
        uint32_t keep = m >> 20;
        const uint32_t rem = m & 0xFFFFFu;
        keep += (rem > 0x80000u) || (rem == 0x80000u && (keep & 1u));
        int ex = E + 7;
        if (keep == 8) { keep = 0; ++ex; }
        if (ex > 15 || (ex == 15 && keep == 7)) return 0x7E;
        return ((uint32_t)ex << 3) | keep;
    }
    // subnormal: multiples of 2^-9 (scaling by 512 is exact; rint ties to even)
    const uint32_t k = (uint32_t)__builtin_rintf(f * 512.0f);
    return k >= 8 ? 0x08u : k;
}

// Nearest E2M1 code of v (grid 0, 0.5, 1, 1.5, 2, 3, 4, 6), ties to the code
// with mantissa bit 0, magnitudes above 6 saturating; zero is +0.
__device__ __forceinline__ uint32_t e2m1_rne(float v) {
    const float a = fabsf(v);
    const uint32_t c = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                     : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
    return (c != 0 && v < 0.0f) ? (c | 8u) : c;
}

__device__ __forceinline__ float e2m1_val(uint32_t c) {
    const uint32_t m = c & 7;
    const float a = m < 2 ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)(m & 1), (int)(m >> 1) - 1);
    return (c & 8) ? -a : a;
}

// Block scale of a group with largest magnitude amax under activation global
// scale ga: the E4M3 rounding of amax / (6 ga), as its value.
__device__ __forceinline__ float nvfp4_group_scale(float amax, float ga) {
    return e4m3_val(e4m3_rne(__fdiv_rn(amax, 6.0f * ga)));
}

// The value of e2m1_rne(a) for a >= 0, computed directly: on [0, 1) the grid
// is the multiples of 0.5 (rint ties to even, so 0.25 -> 0 and 0.75 -> 1);
// from 1 up it is the floats with one mantissa bit, reached by rounding the
// fp32 to one mantissa bit (ties to even) in its bit pattern, then
// saturated at 6 (+inf too).  Equal to e2m1_val(e2m1_rne(a)) for every
// non-negative float: checked exhaustively on the host, 2^31 - 2^23 + 1
// values.
__device__ __forceinline__ float e2m1_round(float a) {
    if (a < 1.0f) return __builtin_rintf(2.0f * a) * 0.5f;
    uint32_t b = __float_as_uint(a);
    b += 0x1FFFFFu + ((b >> 22) & 1u);
    return fminf(__uint_as_float(b & 0xFFC00000u), 6.0f);
}

// v quantised with block scale s (s > 0) under ga: e2m1(code) * s, exact
// (a zero code is +0, as e2m1_val gives it).
__device__ __forceinline__ float nvfp4_qv(float v, float s, float ga) {
    if (s == 0.0f) return 0.0f;
    const float q = __fdiv_rn(v, s * ga);
    const float r = e2m1_round(fabsf(q));
    return r == 0.0f ? 0.0f : __builtin_copysignf(r, q) * s;
}

}  // namespace moe
