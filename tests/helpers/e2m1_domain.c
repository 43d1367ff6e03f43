/*
 * Exhaustive check, on the host, of the FP4 E2M1 encoder the tk_quant FP4
 * kernel uses: clamp |v| to 6, shift [0, 1) by +1.0, round the fp32 bits to
 * one mantissa bit by integer arithmetic (add 2^21 - 1 plus the kept bit, drop
 * 22 bits), and read the code off exponent and kept bit.  The domain is every
 * value the kernel can encode: v = x * 2^k, x any finite bf16 value (the
 * input), 2^k the block's power-of-two reciprocal scale, k in [-40, 40] (the
 * clamp amax >= 1e-4 bounds k above by 16; the bf16 range bounds the rest).
 * Each code must equal the nearest E2M1 value with ties to the even code,
 * saturating at 6, sign kept -- found here by plain search over the 8
 * magnitudes.  Prints "values mismatches".
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static uint32_t bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

static uint32_t kernel_code(float v)
{
    const float a = fminf(fabsf(v), 6.0f);
    const int sub = a < 1.0f;
    uint32_t b = bits(sub ? a + 1.0f : a);
    b += 0x1FFFFFu + ((b >> 22) & 1u);
    const uint32_t c = (b >> 22) - (sub ? 254u : 252u);
    return c | ((bits(v) >> 28) & 8u);
}

static const double kMag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

static uint32_t nearest_code(float v)
{
    const uint32_t s = signbit(v) ? 8u : 0u;
    const double a = fabs((double)v);
    if (a >= 6.0) return s | 7u;
    int best = 0;
    for (int c = 1; c < 8; ++c) {
        const double dc = fabs(a - kMag[c]), db = fabs(a - kMag[best]);
        if (dc < db || (dc == db && (c & 1) == 0)) best = c;
    }
    return s | (uint32_t)best;
}

int main(void)
{
    long long n = 0, bad = 0;
    for (uint32_t h = 0; h < 0x10000u; ++h) {
        const float x = f32(h << 16);
        if (!isfinite(x)) continue;
        for (int k = -40; k <= 40; ++k) {
            const float v = ldexpf(x, k);
            if (!isfinite(v)) continue;
            ++n;
            if (kernel_code(v) != nearest_code(v)) {
                if (bad < 5) printf("mismatch v=%a kernel=%u nearest=%u\n", v, kernel_code(v), nearest_code(v));
                ++bad;
            }
        }
    }
    printf("%lld %lld\n", n, bad);
    return 0;
}
