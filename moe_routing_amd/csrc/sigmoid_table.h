// The pinned fp32 sigmoid on bf16 arguments, as a table.
//
// A SwiGLU gate g is bf16 (the expert GEMM's output), so sigmoid(g) takes one
// of 65536 values.  Over bf16 the pinned sigmoid is constant outside a band of
// magnitudes m = bits & 0x7FFF: exactly 1/2 for m < kSigLo (|g| < 2^-24),
// exactly 1 for positive and exactly 0 for negative g with m >= kSigHi
// (|g| >= 96).  The table holds, for i = 0 .. kSigN + 1 and sign s,
//   entry[2 i + s] = sigmoid(g) for magnitude m = kSigLo - 1 + i,
// with i = 0 standing for every m < kSigLo and i = kSigN + 1 for every
// m >= kSigHi (infinities and NaNs included).  A kernel forms
// i = med3(m, kSigLo - 1, kSigHi) - (kSigLo - 1) and reads one LDS word in
// place of some thirty instructions of exp and division.  The build computes
// the table on the host with the same pinned steps (IEEE fp32, no
// contraction) and fails if a band edge does not hold.
#pragma once

namespace tk {
constexpr unsigned kSigLo = 0x3380u;                 // 2^-24
constexpr unsigned kSigHi = 0x42C0u;                 // 96
constexpr unsigned kSigN = kSigHi - kSigLo;          // magnitudes inside the band
constexpr unsigned kSigEntries = 2u * (kSigN + 2u);  // 7812 floats, 31248 bytes
}  // namespace tk
