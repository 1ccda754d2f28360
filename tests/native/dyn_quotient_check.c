/* Exhaustive check of the code quotient of the fused per-token quantization
 * (qgemm_w8a8_*_dynamic; test infrastructure, host only).
 *
 * For every positive finite bf16 row abs-max `amax` whose scale
 * s = amax / q_max (IEEE fp32) is at least 2^-100, and every bf16 value a with
 * 0 <= a <= amax (negative values mirror them: every step is odd in a), the
 * code of the IEEE quotient a / s must equal the code of
 *     r = 1 / s, q0 = a * r, e = fma(-q0, s, a), q = fma(e, r, q0).
 * Codes: e4m3 (q_max 448) round-to-nearest-even on the e4m3 grid after a clamp
 * to +-448; int8 (q_max 127) round half to even, clamped to +-127.  Built
 * without floating-point contraction.  Prints the pair count and the number
 * of differing codes; exits 1 if any differ. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bf16(uint32_t bits) {
    const uint32_t u = bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* nearest e4m3 value (ties to even), |x| clamped to 448 */
static double e4m3_code(float q) {
    const double x = fabs((double)q), sgn = q < 0 ? -1.0 : 1.0;
    if (x >= 448.0) return sgn * 448.0;
    int e;
    frexp(x, &e);                          /* x in [2^(e-1), 2^e) */
    int ex = e - 1;
    if (ex < -6) ex = -6;                  /* subnormal spacing 2^-9 */
    const double step = ldexp(1.0, ex - 3);
    double r = nearbyint(x / step) * step; /* ties to even: default rounding mode */
    if (r > 448.0) r = 448.0;
    return sgn * r;
}

static double int8_code(float q) {
    double r = nearbyint((double)q);
    if (r > 127.0) r = 127.0;
    if (r < -127.0) r = -127.0;
    return r;
}

int main(int argc, char **argv) {
    const int fp8 = argc > 1 && argv[1][0] == 'f';
    const float qmax = fp8 ? 448.0f : 127.0f;
    long long pairs = 0, bad = 0;
    for (uint32_t mb = 1; mb < 0x7f80u; ++mb) {
        const float amax = bf16(mb);
        const volatile float s = amax / qmax;
        if (!(s >= 0x1p-100f)) continue;
        const volatile float r = 1.0f / s;
        for (uint32_t ab = 0; ab <= mb; ++ab) {
            const float a = bf16(ab);
            const volatile float q_ieee = a / s;
            const volatile float q0 = a * r;
            const volatile float e = fmaf(-q0, s, a);
            const volatile float q = fmaf(e, r, q0);
            ++pairs;
            if (q != q_ieee) {
                const double c0 = fp8 ? e4m3_code(q_ieee) : int8_code(q_ieee);
                const double c1 = fp8 ? e4m3_code(q) : int8_code(q);
                if (c0 != c1) {
                    if (bad < 5) printf("differ: amax=%a a=%a s=%a %g vs %g\n", amax, a, s, c0, c1);
                    ++bad;
                }
            }
        }
    }
    printf("%s: %lld pairs, %lld differing codes\n", fp8 ? "e4m3" : "int8", pairs, bad);
    return bad != 0;
}
