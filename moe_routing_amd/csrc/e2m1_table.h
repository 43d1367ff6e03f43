// FP4 E2M1 encoding by table (plain C++17: the FP4 kernel and a host proof of
// it include the same code).
//
// E2M1 magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes 0..7); a value is
// encoded to the nearest one, ties to the even code, saturating at 6, with
// the sign in bit 3.  The FP4 kernel encodes quotients q = x * 2^j of bf16
// inputs x by an exact power of two, so q carries at most 8 significant bits
// and its code depends only on the top 16 bits of its fp32 pattern.  Below
// 0.25 every magnitude encodes to 0 and from 6 up to 7, so a table over the
// bf16 magnitudes [0.25, 8) -- 640 entries -- holds every code; magnitudes
// outside are clamped onto its ends (0.25 -> 0, just below 8 -> 7).  The
// table is built at compile time with integer arithmetic only: a magnitude
// in the band is an integer number of 2^-9 steps, and so are the E2M1 values
// and their midpoints.
#pragma once

#include <cstdint>

namespace tk {

constexpr uint32_t kE2m1Lo = 0x3E80u;   // bf16 0.25
constexpr uint32_t kE2m1Hi = 0x4100u;   // bf16 8.0
constexpr uint32_t kE2m1N = kE2m1Hi - kE2m1Lo;

// E2M1 code (0..7) of the bf16 magnitude bits m, kE2m1Lo <= m < kE2m1Hi
constexpr uint32_t e2m1_code_of_bf16(uint32_t m)
{
    const uint32_t mant = (m & 0x7Fu) | 0x80u;                 // 8 significant bits
    const int e = static_cast<int>(m >> 7) - 127;              // -2 .. 2 in the band
    const int64_t v = static_cast<int64_t>(mant) << (e + 2);   // value in 2^-9 steps
    constexpr int64_t grid[8] = {0, 256, 512, 768, 1024, 1536, 2048, 3072};
    uint32_t best = 0;
    for (uint32_t c = 1; c < 8; ++c) {
        const int64_t dc = v > grid[c] ? v - grid[c] : grid[c] - v;
        const int64_t db = v > grid[best] ? v - grid[best] : grid[best] - v;
        if (dc < db || (dc == db && (c & 1u) == 0)) best = c;
    }
    return best;
}

struct E2m1Table {
    uint8_t code[kE2m1N];
};

constexpr E2m1Table make_e2m1_table()
{
    E2m1Table t{};
    for (uint32_t i = 0; i < kE2m1N; ++i) t.code[i] = static_cast<uint8_t>(e2m1_code_of_bf16(kE2m1Lo + i));
    return t;
}

// Code of the fp32 value with bit pattern `bits` (a quotient as above): the
// clamped table entry, sign in bit 3.
constexpr uint32_t e2m1_lookup(uint32_t bits, const uint8_t* table)
{
    const uint32_t m = (bits >> 16) & 0x7FFFu;
    const uint32_t c = m < kE2m1Lo ? kE2m1Lo : (m > kE2m1Hi - 1 ? kE2m1Hi - 1 : m);
    return table[c - kE2m1Lo] | ((bits >> 28) & 8u);
}

}  // namespace tk
