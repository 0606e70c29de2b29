// Exhaustive host check of the direct E2M1 rounding that the NVFP4 quantiser
// uses (nvfp4.h, e2m1_round) against the threshold definition (e2m1_rne and
// e2m1_val there: nearest grid value, ties to the code with mantissa bit 0,
// saturating at 6), written out again here in plain C.
// Every non-negative float is checked; the exit status is the verdict.
#include <stdio.h>
#include <stdint.h>
#include <string.h>
#include <math.h>
static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float def_q(float a) {  // the library's definition (code, then value)
    const uint32_t c = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                     : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
    const uint32_t m = c & 7;
    return m < 2 ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)(m & 1), (int)(m >> 1) - 1);
}
static float new_q(float a) {
    if (a < 1.0f) return rintf(2.0f * a) * 0.5f;
    uint32_t b = f2u(a);
    b += 0x1FFFFFu + ((b >> 22) & 1u);
    b &= 0xFFC00000u;
    return fminf(u2f(b), 6.0f);
}
int main(void) {
    long bad = 0, n = 0;
    for (uint64_t u = 0; u <= 0x7FFFFFFFull; ++u) {
        const float a = u2f((uint32_t)u);
        if (isnan(a)) continue;
        ++n;
        const float x = def_q(a), y = new_q(a);
        if (f2u(x) != f2u(y)) { if (bad < 10) printf("a=%.9g def %g new %g\n", a, x, y); ++bad; }
    }
    printf("checked %ld non-negative floats, %ld mismatches\n", n, bad);
    return bad != 0;
}
