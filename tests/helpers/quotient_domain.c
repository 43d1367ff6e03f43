/*
 * Exhaustive check, on the host, of the division shortcut the FP8 expand
 * kernel uses for q = x / scale:
 *     inv = RN(1/scale); q0 = RN(x*inv); rn = fma(q0, scale, -x); q = fma(-rn, inv, q0)
 * (Markstein's correction step, with the residual negated so that x = -0
 * keeps its sign).  The domain is every pair the kernel can
 * see: amax = a bf16 magnitude >= 1e-4 or the clamp value 1e-4f,
 * scale = RN(amax/448), and x = every bf16 value with |x| <= amax, both
 * signs (-0 included).  For each pair the
 * shortcut must equal the IEEE quotient RN(x/scale) bit for bit, except where
 * both lie below 2^-10 -- half the smallest E4M3 subnormal, so both encode to
 * the same signed zero.  (Differences occur only for x tiny against a huge
 * block maximum, where x*inv or the residual underflows: quotients near the
 * bottom of the fp32 range.)
 *
 * Built by the test with -O2 -ffp-contract=off -mfma so that fmaf is one
 * fused instruction; prints "pairs normal_mismatches tiny_mismatches".
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float g_max_tiny_mismatch = 0.0f;  /* largest |quotient| among tiny mismatches */

static float f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static long long check_amax(float amax, long long* pairs, long long* tiny)
{
    const float scale = amax / 448.0f;
    const float inv = 1.0f / scale;
    const float kTiny = 0x1p-10f;
    long long bad = 0, n = 0;
    for (uint32_t h = 0; h < 0x10000u; ++h) {
        const float x = f32(h << 16);
        if (!(fabsf(x) <= amax)) continue;
        const float q0 = x * inv;
        const float rn = fmaf(q0, scale, -x);
        /* -rn by its sign bit, as the kernel's negation modifier: a compiler
           may not turn -fma(a, b, c) into fma(-a, b, -c), which differs for
           a zero result */
        const float q = fmaf(f32(bits(rn) ^ 0x80000000u), inv, q0);
        const float ref = x / scale;
        if (bits(q) != bits(ref)) {
            if (fabsf(q) < kTiny && fabsf(ref) < kTiny && signbit(q) == signbit(ref)) {
                ++*tiny;
                if (fabsf(ref) > g_max_tiny_mismatch) g_max_tiny_mismatch = fabsf(ref);
            } else {
                if (bad < 5) printf("mismatch amax=%a x=%a q=%a ref=%a\n", amax, x, q, ref);
                ++bad;
            }
        }
        ++n;
    }
    *pairs += n;
    return bad;
}

int main(void)
{
    long long pairs = 0, bad = 0, tiny = 0;  /* the max-tiny tracker is not
                                                 thread-safe; it is a report only */
    bad += check_amax(1e-4f, &pairs, &tiny);
    long long p_local = 0, b_local = 0, t_local = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : p_local, b_local, t_local)
    for (uint32_t h = 0; h < 0x7F80u; ++h) {
        const float a = f32(h << 16);
        if (a < 1e-4f) continue;
        long long p = 0, ti = 0;
        b_local += check_amax(a, &p, &ti);
        p_local += p;
        t_local += ti;
    }
    pairs += p_local;
    bad += b_local;
    tiny += t_local;
    printf("largest quotient where the shortcut differs: %a\n", g_max_tiny_mismatch);
    printf("%lld %lld %lld\n", pairs, bad, tiny);
    return 0;
}
