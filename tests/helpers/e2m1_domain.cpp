/*
 * Exhaustive check, on the host, of the FP4 E2M1 encoding the tk_quant FP4
 * kernel uses: the compile-time table of moe_routing_amd/csrc/e2m1_table.h,
 * indexed by the quotient's clamped bf16 magnitude, sign in bit 3.  This file
 * includes that header, so it runs the kernel's own table and lookup.  The
 * domain is every value the kernel can encode: v = x * 2^k, x any finite bf16
 * value (the input), 2^k the block's power-of-two reciprocal scale, k in
 * [-40, 40] (the clamp amax >= 1e-4 bounds k above by 16; the bf16 range
 * bounds the rest).  Each code must equal the nearest E2M1 value with ties to
 * the even code, saturating at 6, sign kept -- found here by plain search over
 * the 8 magnitudes in double precision.  Prints "values mismatches".
 */
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "e2m1_table.h"

static uint32_t bits(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }
static float f32(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }

static const double kMag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

static uint32_t nearest_code(float v)
{
    const uint32_t s = std::signbit(v) ? 8u : 0u;
    const double a = std::fabs(static_cast<double>(v));
    if (a >= 6.0) return s | 7u;
    int best = 0;
    for (int c = 1; c < 8; ++c) {
        const double dc = std::fabs(a - kMag[c]), db = std::fabs(a - kMag[best]);
        if (dc < db || (dc == db && (c & 1) == 0)) best = c;
    }
    return s | static_cast<uint32_t>(best);
}

int main()
{
    static const tk::E2m1Table table = tk::make_e2m1_table();
    long long n = 0, bad = 0;
    for (uint32_t h = 0; h < 0x10000u; ++h) {
        const float x = f32(h << 16);
        if (!std::isfinite(x)) continue;
        for (int k = -40; k <= 40; ++k) {
            const float v = std::ldexp(x, k);
            if (!std::isfinite(v)) continue;
            ++n;
            const uint32_t got = tk::e2m1_lookup(bits(v), table.code);
            if (got != nearest_code(v)) {
                if (bad < 5) std::printf("mismatch v=%a kernel=%u nearest=%u\n", v, got, nearest_code(v));
                ++bad;
            }
        }
    }
    std::printf("%lld %lld\n", n, bad);
    return 0;
}
