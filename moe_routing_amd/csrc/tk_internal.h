// Internal helpers shared by the HIP sources of libtk (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <tuple>
#include <utility>

#include "tk.h"

#define TK_EXPORT extern "C" __attribute__((visibility("default")))

namespace tk {

// ---------------------------------------------------------------- host side
// Record a failure for tk_last_error() and return `status`.
tk_status fail(tk_status status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the error text and return TK_OK.
tk_status ok();
// Turn a HIP launch result into a status.
tk_status launched(hipError_t e, const char* what);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Launch kernel `k` with arguments converted to its exact parameter types;
// returns the launch status directly (no sticky-error lookups).
template <typename... KA, typename... PA>
hipError_t launch(void (*k)(KA...), dim3 grid, dim3 block, size_t lds_bytes, hipStream_t s,
                  PA&&... pa)
{
    std::tuple<KA...> args(std::forward<PA>(pa)...);
    void* argv[sizeof...(KA) ? sizeof...(KA) : 1];
    std::apply([&](auto&... a) {
        int i = 0;
        ((argv[i++] = static_cast<void*>(&a)), ...);
    }, args);
    return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, argv, lds_bytes, s);
}

// Waves of 64 lanes; the kernels here use 256-lane workgroups (4 waves).
constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;

// ------------------------------------------------------------- device side
// Wave-uniform copy of a value (the first active lane's), kept in an SGPR.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// 16 bytes as a native vector (the form the nontemporal builtins take).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte global load / store with the nontemporal (streaming) hint, for data
// touched exactly once; compiles to global_load/store_dwordx4 ... nt.
__device__ __forceinline__ u32x4 load_stream(const void* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void store_stream(void* p, u32x4 v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// bf16 pair packed in a 32-bit word -> two fp32 values (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Cross-lane moves inside a row of 16 lanes (DPP), full exec assumed.
// kQuadXor1 / kQuadXor2: quad_perm [1,0,3,2] / [2,3,0,1]; kHalfMirror: lane
// i <-> 7-i within 8 lanes; kMirror: lane i <-> 15-i within 16 lanes.
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140;
// Across rows (GFX9 DPP): lane 15 of each row to the whole next row, and lane
// 31 to rows 2 and 3; which rows are written is the instruction's row mask.
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Maximum over each aligned run of 8 lanes, returned to every lane of the run.
__device__ __forceinline__ float max_run8(float v)
{
    v = fmaxf(v, dpp_f32<kQuadXor1>(v));
    v = fmaxf(v, dpp_f32<kQuadXor2>(v));
    return fmaxf(v, dpp_f32<kHalfMirror>(v));
}

// Maximum over each aligned run of `width` lanes (a power of two <= 64),
// returned to every lane of the run.
__device__ __forceinline__ uint32_t max_run_u32(uint32_t v, int width)
{
    if (width >= 2) v = max(v, dpp_u32<kQuadXor1>(v));
    if (width >= 4) v = max(v, dpp_u32<kQuadXor2>(v));
    if (width >= 8) v = max(v, dpp_u32<kHalfMirror>(v));
    if (width >= 16) v = max(v, dpp_u32<kMirror>(v));
    if (width >= 32) {
        const uint32_t r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
        const uint32_t r2 = __builtin_amdgcn_readlane(v, 47), r3 = __builtin_amdgcn_readlane(v, 63);
        const uint32_t lo = max(r0, r1), hi = max(r2, r3);
        v = (width == 64) ? max(lo, hi) : ((threadIdx.x & 32) ? hi : lo);
    }
    return v;
}

// Maximum over the whole wave as a wave-uniform (SGPR) value.
__device__ __forceinline__ uint32_t max_wave_u32(uint32_t v)
{
    v = max(v, dpp_u32<kQuadXor1>(v));
    v = max(v, dpp_u32<kQuadXor2>(v));
    v = max(v, dpp_u32<kHalfMirror>(v));
    v = max(v, dpp_u32<kMirror>(v));
    // every lane of a row now holds the row's maximum.  row_bcast:15 brings
    // lane 15 of rows 0 and 2 into rows 1 and 3, row_bcast:31 lane 31 into
    // rows 2 and 3 (rows outside the row mask keep their value, as max with
    // 0 leaves it), so lane 63 holds the maximum of all four rows
    v = max(v, static_cast<uint32_t>(
                   __builtin_amdgcn_update_dpp(0, static_cast<int>(v), kRowBcast15, 0xA, 0xF, false)));
    v = max(v, static_cast<uint32_t>(
                   __builtin_amdgcn_update_dpp(0, static_cast<int>(v), kRowBcast31, 0xC, 0xF, false)));
    return __builtin_amdgcn_readlane(v, 63);
}

// Sum / maximum over the whole wave, returned wave-uniform.  DPP row steps
// then the four row results in a fixed order: every lane of a row holds the
// same partial after each step (the pairs add in either order to the same
// value), so the result does not depend on the lane and is deterministic.
__device__ __forceinline__ float sum_wave_f32(float v)
{
    v += dpp_f32<kQuadXor1>(v);
    v += dpp_f32<kQuadXor2>(v);
    v += dpp_f32<kHalfMirror>(v);
    v += dpp_f32<kMirror>(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 47));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
    return (r0 + r1) + (r2 + r3);
}
__device__ __forceinline__ float max_wave_f32(float v)
{
    v = fmaxf(v, dpp_f32<kQuadXor1>(v));
    v = fmaxf(v, dpp_f32<kQuadXor2>(v));
    v = fmaxf(v, dpp_f32<kHalfMirror>(v));
    v = fmaxf(v, dpp_f32<kMirror>(v));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 47));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Two fp32 -> two bf16 (round to nearest even, hardware convert) packed.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const __bf16 a = static_cast<__bf16>(lo);
    const __bf16 b = static_cast<__bf16>(hi);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

// ------------------------------------------------ shared fp32 arithmetic
// Pinned fp32 e^y: Cody & Waite reduction by ln 2 split in two words (the
// high word has 16 significant bits, so n*LN2_HI is exact for |n| <= 128),
// then the degree-7 Taylor polynomial of e^r in Horner form with fused
// multiply-adds.  Every step is one IEEE fp32 operation (the library is built
// with -ffp-contract=off), so the result is the same on any IEEE machine
// that follows these steps; y is cut to [-86, 88] so p * 2^n stays normal.
// (Host and device: the build evaluates it on the host for the bf16 sigmoid
// table the SwiGLU kernels read.)
constexpr float kLog2e = 0x1.715476p+0f;    // RN(log2 e)
constexpr float kLn2Hi = 0x1.62e4p-1f;      // ln 2 truncated to 16 bits
constexpr float kLn2Lo = 0x1.7f7d1cp-20f;   // RN(ln 2 - kLn2Hi)
constexpr float kC2 = 0x1p-1f, kC3 = 0x1.555556p-3f, kC4 = 0x1.555556p-5f,
                kC5 = 0x1.111112p-7f, kC6 = 0x1.6c16c2p-10f, kC7 = 0x1.a01a02p-13f;  // RN(1/i!)

__host__ __device__ __forceinline__ float pinned_exp(float y)
{
    if (y > 88.0f) return __builtin_inff();
    if (y < -86.0f) return 0.0f;
    const float n = __builtin_rintf(y * kLog2e);
    float r = __builtin_fmaf(-n, kLn2Hi, y);
    r = __builtin_fmaf(-n, kLn2Lo, r);
    float p = kC7;
    p = __builtin_fmaf(p, r, kC6);
    p = __builtin_fmaf(p, r, kC5);
    p = __builtin_fmaf(p, r, kC4);
    p = __builtin_fmaf(p, r, kC3);
    p = __builtin_fmaf(p, r, kC2);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    return __builtin_ldexpf(p, static_cast<int>(n));
}

__host__ __device__ __forceinline__ float pinned_sigmoid(float x) { return 1.0f / (1.0f + pinned_exp(-x)); }

// -------------------------------------------------- 1x128 E4M3 codec
// x / scale for scale > 0 by Markstein's correction on the correctly rounded
// reciprocal inv = RN(1/scale): q0 = RN(x*inv); r = x - q0*scale (exact);
// q = RN(q0 + r*inv) is the correctly rounded quotient (P. Markstein, IBM J.
// Res. Dev. 34(1), 1990; Muller et al., Handbook of Floating-Point
// Arithmetic).  Quotients that underflow encode to a signed E4M3 zero either
// way.  The residual is formed negated, rn = fma(q0, scale, -x) = -r (RN is
// symmetric), and applied as fma(-rn, inv, q0): three instructions with the
// negations as operand modifiers.  For x = -0 that keeps the sign (q0 = -0,
// rn = +0, and -0 + -0 = -0), where fma(r, inv, q0) with r = +0 would give
// +0 and need the sign put back.
__device__ __forceinline__ float fp8_quotient(float x, float scale, float inv)
{
    const float q0 = x * inv;
    const float rn = __builtin_fmaf(q0, scale, -x);
    return __builtin_fmaf(-rn, inv, q0);
}

// Four quotients -> four E4M3 codes (gfx950 hardware convert: OCP E4M3FN,
// round to nearest even).  amax / RN(amax/448) can exceed 448 by one fp32
// ulp; such values round to 448 like every value below 464.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return static_cast<uint32_t>(w);
}


}  // namespace tk
