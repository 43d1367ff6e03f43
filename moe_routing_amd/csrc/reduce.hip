// tk_reduce: weighted combine of expert outputs back to tokens (the fused reduce
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
//
// tk_reduce_dense, the same combine for dense routings (every slot, or
// nearly, has a row): one 1024-thread workgroup takes up to 16 consecutive
// tokens; each of its 16 waves combines up to 14 of their units -- the same
// units and arithmetic as above, so the results are bit-identical -- keeps
// the outputs in registers, and stores them only after a workgroup barrier,
// so the workgroup's output rows (224 KiB at H = 7168) leave as one burst
// after all of its reads.  With the writes grouped into bursts the HBM bus
// turns between reads and writes less often: 174-177 -> 169-170 us at
// T=8192, H=7168, k=8, while the same schedule with each unit stored as soon
// as it is combined takes 201 us.  One such workgroup fits on a CU at a time,
// so they run in rounds of one per CU, with the tokens spread evenly over the
// rounds (fewer than 16 per workgroup when T is not a multiple of 16 x CUs):
// with 16 each, T=4500 left its second round a quarter full (122 -> 98 us at
// H=7168, k=8).  Where a round moves at least 480 MiB (H=7168, k=8: 504 MiB
// on 256 CUs) each round is a launch of its own, so that all workgroups work
// on one window of consecutive tokens at a time: 728 -> 703 us at T=32768
// and 1705 -> 1588 us at T=76800, the same within noise up to T=16384; with
// smaller rounds the launch boundaries cost more than the windows give (4 to
// 49 launches of 9-453 MB: up to 40 % slower).  Rows shorter than four
// 512-column units take tk_reduce's kernel (H=256: 124 against 90 us,
// H=1024: 192 against 185; from H=2048 on the staged form is as fast or
// faster).  A device-wide barrier between each launch's reads and its
// stores added nothing.  When most slots are masked (one GPU's
// expert-parallel share: two thirds of the tokens have no local route) the
// big workgroups lose to the many short waves of tk_reduce (222 against 128
// us at T=32768, H=7168, k=8), and the call cannot see the routing, so the
// caller chooses.
#include "tk_internal.h"

#include <atomic>

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

constexpr int kStThreads = 1024;                       // 16 waves per workgroup (dense form)
constexpr int kStWaves = kStThreads / tk::kWave;
constexpr int kStUnits = 14;                           // units per wave at most
constexpr int kStMaxTokens = 16;                       // tokens per workgroup at most
constexpr int kStMinChunks = 4;                        // staged form from H > 1536 on
constexpr int64_t kStRoundBytes = int64_t(480) << 20;  // one launch per round from here on
constexpr int kMaxDevices = 64;

template <int K>
__global__ __launch_bounds__(kStThreads) void reduce_staged_kernel(
    const uint16_t* __restrict__ y, int64_t rows_in, const int32_t* __restrict__ pos,
    const float* __restrict__ w, int T, int H, int chunks, int tpw, int g0, uint16_t* __restrict__ out)
{
    const int lane = threadIdx.x & (tk::kWave - 1);
    const int wave = tk::uniform(threadIdx.x / tk::kWave);
    const int64_t t_first = (static_cast<int64_t>(g0) + blockIdx.x) * tpw;
    const int64_t left = T - t_first;
    const int nt = left <= 0 ? 0 : (left > tpw ? tpw : static_cast<int>(left));
    const int t0 = nt > 0 ? static_cast<int>(t_first) : 0;
    const int units = nt * chunks;   // <= kStWaves * kStUnits (the host's choice of tpw)
    tk::u32x4 res[kStUnits];
#pragma unroll
    for (int i = 0; i < kStUnits; ++i) {
        res[i] = tk::u32x4{0u, 0u, 0u, 0u};
        const int u = wave + kStWaves * i;
        if (u >= units) continue;   // wave-uniform
        const int tl = u / chunks;
        const int t = t0 + tl;
        const int col = (u - tl * chunks) * kChunk + lane * 8;
        const int32_t* p = pos + static_cast<size_t>(t) * K;
        const float* wt = w + static_cast<size_t>(t) * K;
        int32_t r32[K];
        float wj[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            r32[j] = p[j];
            wj[j] = wt[j];
        }
        bool ok[K];
#pragma unroll
        for (int j = 0; j < K; ++j) ok[j] = r32[j] >= 0 && r32[j] < rows_in && col < H;
        tk::u32x4 d[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            d[j] = tk::u32x4{0u, 0u, 0u, 0u};
            if (ok[j]) d[j] = tk::load_stream(y + static_cast<size_t>(r32[j]) * H + col);
        }
        float acc[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = 0.f;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            if (!ok[j]) continue;
            const uint32_t v[4] = {d[j].x, d[j].y, d[j].z, d[j].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] = __builtin_fmaf(wj[j], tk::bf16_lo(v[q]), acc[2 * q]);
                acc[2 * q + 1] = __builtin_fmaf(wj[j], tk::bf16_hi(v[q]), acc[2 * q + 1]);
            }
        }
        res[i].x = tk::pack_bf16x2(acc[0], acc[1]);
        res[i].y = tk::pack_bf16x2(acc[2], acc[3]);
        res[i].z = tk::pack_bf16x2(acc[4], acc[5]);
        res[i].w = tk::pack_bf16x2(acc[6], acc[7]);
    }
    __syncthreads();   // every read of the workgroup before any of its stores
    // rows t0 .. t0 + nt - 1 are contiguous in out; unit u is its 1 KiB at
    // t * H + chunk * 512, so neighbouring waves store neighbouring pieces
#pragma unroll
    for (int i = 0; i < kStUnits; ++i) {
        const int u = wave + kStWaves * i;
        if (u >= units) continue;
        const int tl = u / chunks;
        const int col = (u - tl * chunks) * kChunk + lane * 8;
        if (col < H) tk::store_stream(out + static_cast<size_t>(t0 + tl) * H + col, res[i]);
    }
}

// Tokens per workgroup for the staged form: as many as the waves' unit slots
// hold (16 waves x 14), at most 16; 0 if one token's row alone has more units.
int staged_tokens(int chunks)
{
    const int tpw = kStWaves * kStUnits / chunks;
    return tpw < 1 ? 0 : (tpw > kStMaxTokens ? kStMaxTokens : tpw);
}

// Compute units of the current device (cached per device); 0 if unknown.
int device_cus(int dev)
{
    static std::atomic<int> cus[kMaxDevices];
    if (dev < 0 || dev >= kMaxDevices) return 0;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0 && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
        cus[dev].store(n, std::memory_order_relaxed);
    return n > 0 ? n : 0;
}

// The staged form when it applies: rows of at least kStMinChunks units (with
// shorter rows a workgroup holds little work, and the many small workgroups
// of the one-wave-per-unit kernel hide latency better) and at least one full
// workgroup of tokens per CU (with fewer the chip idles).  Only one of these
// workgroups fits on a CU at a time, so they run in rounds of one per CU; the
// tokens are spread evenly over the rounds (tpw = ceil(T / (rounds * CUs)) <=
// the cap), so that the last round is as full as the others.  When a full
// round moves at least kStRoundBytes, each round is a launch of its own: every
// workgroup of a launch works on one window of consecutive tokens, whose
// rows (expert-contiguous, in token order within each expert) lie in short
// runs, and the next window starts only after the previous one is written.
template <int K>
bool launch_staged(const uint16_t* y, int64_t rows, const int32_t* pos, const float* w, int T,
                   int H, uint16_t* out, hipStream_t stream, hipError_t* e)
{
    const int chunks = (H + kChunk - 1) / kChunk;
    const int cap = staged_tokens(chunks);
    int dev = -1;
    if (cap == 0 || chunks < kStMinChunks || hipGetDevice(&dev) != hipSuccess) return false;
    const int64_t cus = device_cus(dev);
    if (cus == 0 || static_cast<int64_t>(T) < cus * cap) return false;
    const int64_t rounds = ((static_cast<int64_t>(T) + cap - 1) / cap + cus - 1) / cus;
    const int tpw = static_cast<int>((static_cast<int64_t>(T) + rounds * cus - 1) / (rounds * cus));
    const int64_t groups = (static_cast<int64_t>(T) + tpw - 1) / tpw;   // <= rounds * cus
    const int64_t token_bytes = (static_cast<int64_t>(K) * 2 + 2) * H + static_cast<int64_t>(K) * 8;
    const int64_t per_launch = cus * cap * token_bytes >= kStRoundBytes ? cus : groups;
    for (int64_t g0 = 0; g0 < groups; g0 += per_launch) {
        const int64_t n = groups - g0 < per_launch ? groups - g0 : per_launch;
        *e = tk::launch(reduce_staged_kernel<K>, dim3(static_cast<unsigned>(n)), dim3(kStThreads),
                        0, stream, y, rows, pos, w, T, H, chunks, tpw, static_cast<int>(g0), out);
        if (*e != hipSuccess) break;
    }
    return true;
}

// Both entry points: argument checks, then the staged form (dense, when it
// applies) or the one-wave-per-unit kernel.
tk_status reduce_call(const void* y_bf16, int64_t rows, const int32_t* pos, const float* topk_w,
                      int32_t T, int32_t k, int32_t H, void* out_bf16, hipStream_t stream,
                      bool dense)
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
    if (dense) {
        bool staged = false;
        switch (k) {
        case 1: staged = launch_staged<1>(y, rows, pos, topk_w, T, H, out, stream, &e); break;
        case 2: staged = launch_staged<2>(y, rows, pos, topk_w, T, H, out, stream, &e); break;
        case 4: staged = launch_staged<4>(y, rows, pos, topk_w, T, H, out, stream, &e); break;
        case 6: staged = launch_staged<6>(y, rows, pos, topk_w, T, H, out, stream, &e); break;
        case 8: staged = launch_staged<8>(y, rows, pos, topk_w, T, H, out, stream, &e); break;
        default: break;
        }
        if (staged) return tk::launched(e, "tk_reduce_dense");
    }
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

}  // namespace

TK_EXPORT tk_status tk_reduce(const void* y_bf16, int64_t rows, const int32_t* pos,
                              const float* topk_w, int32_t T, int32_t k, int32_t H,
                              void* out_bf16, hipStream_t stream)
{
    return reduce_call(y_bf16, rows, pos, topk_w, T, k, H, out_bf16, stream, false);
}

TK_EXPORT tk_status tk_reduce_dense(const void* y_bf16, int64_t rows, const int32_t* pos,
                                    const float* topk_w, int32_t T, int32_t k, int32_t H,
                                    void* out_bf16, hipStream_t stream)
{
    return reduce_call(y_bf16, rows, pos, topk_w, T, k, H, out_bf16, stream, true);
}
