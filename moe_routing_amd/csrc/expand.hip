// tk_expand_quant: expand tokens into expert-contiguous rows, optionally with
// fused per-token 1x128 FP8 E4M3 quantisation (the fused expand of TileKernels'
// moe/ module and the per-token FP8 of its quant/ module, "刚刚！DeepSeek开源高性能
// GPU算子库TileKernels", items moe/ and quant/; FP8 dispatch at the DeepSeek-V3
// shape, "剛剛，DeepSeek開始頻繁更新：Tile Kernels、DeepEP V2", section 性能表現).
// Also tk_expert_standin, the dequantise-and-scale harness kernel.
//
// Token-major: one workgroup of 4 waves per token.  Wave w walks the row's
// 1024-column chunks w, w+4, ...; each lane reads 16 bf16 (two 16-byte
// loads), so every 8-lane group holds one 128-column quantisation block and
// the block amax is a 3-step DPP butterfly inside the group.  The token is
// read once, quantised once, and its 16 code bytes per lane are stored to
// each of its k rows (one 1 KiB contiguous segment per row per wave), so HBM
// traffic is T*H*2 read + R*H written, not R*H*2 read; a token none of whose
// routes has a row (no local expert, or rows beyond the capacity) is not read
// at all.  The expanded rows are written once and not read again by this
// pipeline, so they go out through nontemporal stores.  The token is read
// with ordinary loads, which allocate it in the memory-side cache (MALL,
// 256 MB): a following pass over the same hidden states finds them there,
// where a nontemporal read would not.  All scale writes of a row come from
// one workgroup, so no 4-byte scale shares a cache line with another
// workgroup's.

// Quotient x/scale: Markstein's correction on the reciprocal,
//   inv = RN(1/scale); q0 = RN(x*inv); rn = fma(q0, scale, -x); q = fma(-rn, inv, q0)
// (P. Markstein, IBM J. Res. Dev. 34(1), 1990; the residual is negated so
// that x = -0 keeps its sign).  It equals the IEEE quotient RN(x/scale) for every (x, scale)
// this kernel can see, except where both lie below 2^-10 and so encode to the
// same signed zero; tests/test_quotient_domain.py enumerates that domain.
// FP8 encoding: gfx950's v_cvt_pk_fp8_f32 (OCP E4M3FN, round to nearest even).
#include "tk_internal.h"

namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kChunkFp8 = 1024;   // columns per wave step, FP8 mode (16 per lane)
constexpr int kChunkBf16 = 512;   // columns per wave step, bf16 mode (8 per lane)
constexpr int kExpandWaves = 4;   // waves per workgroup (one token per workgroup; a token
                                  // with no row costs the dispatcher 4 waves, not 8)

// Rows of token t: rows[j] for j < k, -1 where the route is skipped.
template <int KMAX>
__device__ __forceinline__ void token_rows(const int32_t* __restrict__ pos, int t, int k,
                                           int64_t cap, int64_t (&rows)[KMAX])
{
    const int32_t* p = pos + static_cast<size_t>(t) * k;
    int32_t r[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) r[j] = (j < k) ? p[j] : -1;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) rows[j] = (r[j] >= 0 && r[j] < cap) ? r[j] : -1;
}

// Whether any of the token's rows is written (the same for every thread of
// the workgroup, so an early return is uniform).
template <int KMAX>
__device__ __forceinline__ bool any_row(const int64_t (&rows)[KMAX])
{
    bool any = false;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) any = any || rows[j] >= 0;
    return any;
}

// One token per workgroup; K > 0 is a compile-time k, K == 0 a runtime k.
template <int K>
__global__ __launch_bounds__(tk::kWave * kExpandWaves) void expand_fp8_kernel(
    const uint16_t* __restrict__ x, int T, int H, int k_rt, const int32_t* __restrict__ pos,
    uint8_t* __restrict__ out, float* __restrict__ scales, int64_t cap)
{
    constexpr int KMAX = K > 0 ? K : TK_MAX_TOPK;
    const int k = K > 0 ? K : k_rt;
    const int lane = threadIdx.x & (tk::kWave - 1);
    const int wave = tk::uniform(threadIdx.x / tk::kWave);
    const int t = blockIdx.x;
    if (t >= T) return;
    const int nb = H / 128;
    int64_t rows[KMAX];
    token_rows<KMAX>(pos, t, k, cap, rows);
    if (!any_row<KMAX>(rows)) return;   // no destination (e.g. no local route): x is not read
    const uint16_t* xt = x + static_cast<size_t>(t) * H;
    for (int col = wave * kChunkFp8 + lane * 16; col - lane * 16 < H; col += kExpandWaves * kChunkFp8) {
        // H % 128 == 0: an 8-lane group (128 columns) is wholly inside or outside the row
        const bool active = col < H;
        tk::u32x4 a = tk::u32x4{0u, 0u, 0u, 0u}, b = a;
        if (active) {
            a = tk::load16(xt + col);
            b = tk::load16(xt + col + 8);
        }
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        float v[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[2 * i] = tk::bf16_lo(w[i]);
            v[2 * i + 1] = tk::bf16_hi(w[i]);
        }
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
        amax = fmaxf(tk::max_run8(amax), 1e-4f);   // one 128-column block per 8 lanes
        const float scale = amax / 448.0f;
        const float inv = 1.0f / scale;
        tk::u32x4 q;
        q.x = tk::pack_fp8x4(tk::fp8_quotient(v[0], scale, inv), tk::fp8_quotient(v[1], scale, inv),
                         tk::fp8_quotient(v[2], scale, inv), tk::fp8_quotient(v[3], scale, inv));
        q.y = tk::pack_fp8x4(tk::fp8_quotient(v[4], scale, inv), tk::fp8_quotient(v[5], scale, inv),
                         tk::fp8_quotient(v[6], scale, inv), tk::fp8_quotient(v[7], scale, inv));
        q.z = tk::pack_fp8x4(tk::fp8_quotient(v[8], scale, inv), tk::fp8_quotient(v[9], scale, inv),
                         tk::fp8_quotient(v[10], scale, inv), tk::fp8_quotient(v[11], scale, inv));
        q.w = tk::pack_fp8x4(tk::fp8_quotient(v[12], scale, inv), tk::fp8_quotient(v[13], scale, inv),
                         tk::fp8_quotient(v[14], scale, inv), tk::fp8_quotient(v[15], scale, inv));
        if (active) {
#pragma unroll
            for (int j = 0; j < KMAX; ++j) {
                if (rows[j] < 0) continue;
                tk::store_stream(out + static_cast<size_t>(rows[j]) * H + col, q);
                if ((lane & 7) == 0) scales[static_cast<size_t>(rows[j]) * nb + col / 128] = scale;
            }
        }
    }
}

template <int K>
__global__ __launch_bounds__(tk::kWave * kExpandWaves) void expand_bf16_kernel(
    const uint16_t* __restrict__ x, int T, int H, int k_rt, const int32_t* __restrict__ pos,
    uint16_t* __restrict__ out, int64_t cap)
{
    constexpr int KMAX = K > 0 ? K : TK_MAX_TOPK;
    const int k = K > 0 ? K : k_rt;
    const int lane = threadIdx.x & (tk::kWave - 1);
    const int wave = tk::uniform(threadIdx.x / tk::kWave);
    const int t = blockIdx.x;
    if (t >= T) return;
    int64_t rows[KMAX];
    token_rows<KMAX>(pos, t, k, cap, rows);
    if (!any_row<KMAX>(rows)) return;
    const uint16_t* xt = x + static_cast<size_t>(t) * H;
    for (int col = wave * kChunkBf16 + lane * 8; col < H; col += kExpandWaves * kChunkBf16) {
        const tk::u32x4 a = tk::load16(xt + col);
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (rows[j] >= 0) tk::store_stream(out + static_cast<size_t>(rows[j]) * H + col, a);
    }
}

__global__ __launch_bounds__(tk::kBlock) void standin_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ scales,
    const int32_t* __restrict__ n_rows, int64_t cap, int H, float mult,
    uint16_t* __restrict__ y, int chunks)
{
    const int lane = threadIdx.x & (tk::kWave - 1);
    const int nb = H / 128;
    int64_t rows = *n_rows;
    rows = rows < 0 ? 0 : (rows > cap ? cap : rows);
    const int64_t n_units = rows * chunks;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * tk::kWavesPerBlock;
    for (int64_t u = static_cast<int64_t>(blockIdx.x) * tk::kWavesPerBlock +
                     tk::uniform(threadIdx.x / tk::kWave);
         u < n_units; u += stride) {
        const int64_t r = u / chunks;
        const int c0 = static_cast<int>(u - r * chunks) * kChunkFp8 + lane * 8;
        const uint8_t* xr = xq + static_cast<size_t>(r) * H;
        const float* sr = scales + static_cast<size_t>(r) * nb;
        uint16_t* yr = y + static_cast<size_t>(r) * H;
        // lane l takes 8 columns at l*8 and 8 more at 512 + l*8: every load
        // and store instruction covers one contiguous run (512 B of codes,
        // 1 KiB of bf16), so streaming stores leave as whole lines.  y is
        // read once, by the combine: plain stores would leave it dirty in the
        // memory-side cache and the combine's own writes would pay for its
        // write-back.
        // both halves' loads go out before any arithmetic; a lane past the
        // row's end (H % 128 == 0: 16-lane groups are wholly in or out) reads
        // column 0 and stores nothing
        int col[2];
        bool in[2];
        u32x2 q[2];
        float sc[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            col[half] = c0 + half * (kChunkFp8 / 2);
            in[half] = col[half] < H;
            const int cl = in[half] ? col[half] : 0;
            q[half] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(xr + cl));
            sc[half] = sr[cl / 128];
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const uint32_t w[2] = {q[half].x, q[half].y};
            uint32_t o[4];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int wi = static_cast<int>(w[i]);
                const float d0 = __builtin_amdgcn_cvt_f32_fp8(wi, 0);
                const float d1 = __builtin_amdgcn_cvt_f32_fp8(wi, 1);
                const float d2 = __builtin_amdgcn_cvt_f32_fp8(wi, 2);
                const float d3 = __builtin_amdgcn_cvt_f32_fp8(wi, 3);
                o[2 * i] = tk::pack_bf16x2((d0 * sc[half]) * mult, (d1 * sc[half]) * mult);
                o[2 * i + 1] = tk::pack_bf16x2((d2 * sc[half]) * mult, (d3 * sc[half]) * mult);
            }
            if (in[half]) tk::store_stream(yr + col[half], tk::u32x4{o[0], o[1], o[2], o[3]});
        }
    }
}

// Workgroups for a grid-stride loop over n_units waves of work.
unsigned grid_for(int64_t n_units)
{
    const int64_t blocks = (n_units + tk::kWavesPerBlock - 1) / tk::kWavesPerBlock;
    constexpr int64_t kMaxBlocks = 1 << 16;
    return static_cast<unsigned>(blocks < kMaxBlocks ? (blocks < 1 ? 1 : blocks) : kMaxBlocks);
}

}  // namespace

TK_EXPORT tk_status tk_expand_quant(const void* x_bf16, int32_t T, int32_t H, int32_t k,
                                    const int32_t* pos, int32_t mode, void* out, float* scales,
                                    int64_t rows_capacity, hipStream_t stream)
{
    using tk::fail;
    if (T < 0) return fail(TK_ERR_ARG, "tk_expand_quant: T=%d < 0", T);
    if (k < 1) return fail(TK_ERR_ARG, "tk_expand_quant: k=%d < 1", k);
    if (k > TK_MAX_TOPK)
        return fail(TK_ERR_UNSUPPORTED, "tk_expand_quant: k=%d > %d", k, TK_MAX_TOPK);
    if (rows_capacity < 0) return fail(TK_ERR_ARG, "tk_expand_quant: rows_capacity < 0");
    if (mode != TK_EXPAND_BF16 && mode != TK_EXPAND_FP8_E4M3_1X128)
        return fail(TK_ERR_ARG, "tk_expand_quant: unknown mode %d", mode);
    if (H <= 0 || H % 8 != 0)
        return fail(TK_ERR_ARG, "tk_expand_quant: H=%d must be a positive multiple of 8", H);
    if (mode == TK_EXPAND_FP8_E4M3_1X128 && H % 128 != 0)
        return fail(TK_ERR_ARG, "tk_expand_quant: FP8 1x128 mode needs H %% 128 == 0 (H=%d)", H);
    if (mode == TK_EXPAND_FP8_E4M3_1X128 && scales == nullptr && rows_capacity > 0)
        return fail(TK_ERR_ARG, "tk_expand_quant: FP8 mode needs scales");
    if (T == 0 || rows_capacity == 0) return tk::ok();
    if (x_bf16 == nullptr || pos == nullptr || out == nullptr)
        return fail(TK_ERR_ARG, "tk_expand_quant: NULL tensor pointer");
    if (!tk::aligned16(x_bf16) || !tk::aligned16(out) || !tk::aligned4(pos) ||
        (scales && !tk::aligned4(scales)))
        return fail(TK_ERR_ARG, "tk_expand_quant: x/out must be 16-byte aligned, pos/scales 4-byte");

    const auto* x = static_cast<const uint16_t*>(x_bf16);
    const dim3 grid(static_cast<unsigned>(T)), block(tk::kWave * kExpandWaves);
    hipError_t e;
    if (mode == TK_EXPAND_FP8_E4M3_1X128) {
        auto* q = static_cast<uint8_t*>(out);
        switch (k) {
        case 1: e = tk::launch(expand_fp8_kernel<1>, grid, block, 0, stream, x, T, H, k, pos, q, scales, rows_capacity); break;
        case 2: e = tk::launch(expand_fp8_kernel<2>, grid, block, 0, stream, x, T, H, k, pos, q, scales, rows_capacity); break;
        case 4: e = tk::launch(expand_fp8_kernel<4>, grid, block, 0, stream, x, T, H, k, pos, q, scales, rows_capacity); break;
        case 6: e = tk::launch(expand_fp8_kernel<6>, grid, block, 0, stream, x, T, H, k, pos, q, scales, rows_capacity); break;
        case 8: e = tk::launch(expand_fp8_kernel<8>, grid, block, 0, stream, x, T, H, k, pos, q, scales, rows_capacity); break;
        default: e = tk::launch(expand_fp8_kernel<0>, grid, block, 0, stream, x, T, H, k, pos, q, scales, rows_capacity); break;
        }
    } else {
        auto* o = static_cast<uint16_t*>(out);
        switch (k) {
        case 1: e = tk::launch(expand_bf16_kernel<1>, grid, block, 0, stream, x, T, H, k, pos, o, rows_capacity); break;
        case 2: e = tk::launch(expand_bf16_kernel<2>, grid, block, 0, stream, x, T, H, k, pos, o, rows_capacity); break;
        case 4: e = tk::launch(expand_bf16_kernel<4>, grid, block, 0, stream, x, T, H, k, pos, o, rows_capacity); break;
        case 8: e = tk::launch(expand_bf16_kernel<8>, grid, block, 0, stream, x, T, H, k, pos, o, rows_capacity); break;
        default: e = tk::launch(expand_bf16_kernel<0>, grid, block, 0, stream, x, T, H, k, pos, o, rows_capacity); break;
        }
    }
    return tk::launched(e, "tk_expand_quant");
}

TK_EXPORT tk_status tk_expert_standin(const uint8_t* xq, const float* scales,
                                      const int32_t* n_rows, int64_t rows_capacity, int32_t H,
                                      float mult, void* y_bf16, hipStream_t stream)
{
    using tk::fail;
    if (rows_capacity < 0) return fail(TK_ERR_ARG, "tk_expert_standin: rows_capacity < 0");
    if (H <= 0 || H % 128 != 0)
        return fail(TK_ERR_ARG, "tk_expert_standin: H=%d must be a positive multiple of 128", H);
    if (rows_capacity == 0) return tk::ok();
    if (xq == nullptr || scales == nullptr || n_rows == nullptr || y_bf16 == nullptr)
        return fail(TK_ERR_ARG, "tk_expert_standin: NULL pointer");
    if (!tk::aligned16(xq) || !tk::aligned16(y_bf16) || !tk::aligned4(scales) ||
        !tk::aligned4(n_rows))
        return fail(TK_ERR_ARG, "tk_expert_standin: xq/y must be 16-byte aligned");
    const int chunks = (H + kChunkFp8 - 1) / kChunkFp8;
    const hipError_t e = tk::launch(standin_kernel, dim3(grid_for(rows_capacity * chunks)),
                                    dim3(tk::kBlock), 0, stream, xq, scales, n_rows, rows_capacity,
                                    H, mult, static_cast<uint16_t*>(y_bf16), chunks);
    return tk::launched(e, "tk_expert_standin");
}
