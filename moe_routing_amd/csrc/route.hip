// tk_route: top-k expert gating and scoring, one token per 64-lane wave.
//
// Semantics: the moe/ gating ops of TileKernels ("刚刚！DeepSeek开源高性能GPU算子库
// TileKernels", item moe/) with the order and tie rule of the gating listing
// ("DeepSeek 的 GPU 内核帝国…", section 第三层：TileKernels, subsection
// "MoE TopK 门控": k rounds of max + min-index argmax, the winner masked
// before the next round), and DeepSeek-V3's group-limited sigmoid gating.
//
// Layout on the wave: lane l holds experts [l*EPL, l*EPL + EPL), so a row of
// E <= 64*EPL logits is one coalesced load.  A selection key is mapped to an
// order-preserving uint32 (0 = "not eligible"); one round of the argmax is a
// lane-local scan over EPL keys, a 6-step butterfly max, and a ballot whose
// lowest set lane is the lowest expert index holding the maximum (experts are
// laid out in lane order).  Groups of E/n_groups experts are aligned runs of
// lanes, so group scores use butterflies confined to the run.
#include "tk_internal.h"

namespace {

// Pinned fp32 e^y: Cody & Waite reduction by ln 2 split in two words (the
// high word has 16 significant bits, so n*LN2_HI is exact for |n| <= 128),
// then the degree-7 Taylor polynomial of e^r in Horner form with fused
// multiply-adds.  Every step is one IEEE fp32 operation (the file is built
// with -ffp-contract=off), so the result is the same on any IEEE machine
// that follows these steps; y is cut to [-86, 88] so p * 2^n stays normal.
constexpr float kLog2e = 0x1.715476p+0f;    // RN(log2 e)
constexpr float kLn2Hi = 0x1.62e4p-1f;      // ln 2 truncated to 16 bits
constexpr float kLn2Lo = 0x1.7f7d1cp-20f;   // RN(ln 2 - kLn2Hi)
constexpr float kC2 = 0x1p-1f, kC3 = 0x1.555556p-3f, kC4 = 0x1.555556p-5f,
                kC5 = 0x1.111112p-7f, kC6 = 0x1.6c16c2p-10f, kC7 = 0x1.a01a02p-13f;  // RN(1/i!)

__device__ __forceinline__ float pinned_exp(float y)
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

__device__ __forceinline__ float pinned_sigmoid(float x) { return 1.0f / (1.0f + pinned_exp(-x)); }

// Order-preserving map fp32 -> uint32 with -0 folded onto +0; every real key
// (including -inf) maps above 0, which marks "not eligible".
__device__ __forceinline__ uint32_t order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) == 0) u = 0;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t o)
{
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

__device__ __forceinline__ int readlane_i(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }
__device__ __forceinline__ float readlane_f(float v, int lane)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

struct RouteArgs {
    const float* logits;
    const float* bias;
    int32_t* topk_idx;
    float* topk_w;
    int T, E, k;
    int score, n_groups, topk_groups, group_topn, renormalize;
    int lanes_per_group;
    float route_scale;
};

template <int EPL>
__global__ __launch_bounds__(tk::kBlock) void route_kernel(RouteArgs a)
{
    const int lane = threadIdx.x & (tk::kWave - 1);
    const int t = blockIdx.x * tk::kWavesPerBlock + tk::uniform(threadIdx.x / tk::kWave);
    if (t >= a.T) return;
    const bool sigmoid = a.score == TK_SCORE_SIGMOID;
    const float* row = a.logits + static_cast<size_t>(t) * a.E;
    const int e0 = lane * EPL;

    float x[EPL];
    if constexpr (EPL % 4 == 0) {
        if ((a.E & 3) == 0) {
#pragma unroll
            for (int i = 0; i < EPL; i += 4) {
                float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                if (e0 + i < a.E) v = *reinterpret_cast<const float4*>(row + e0 + i);
                x[i] = v.x; x[i + 1] = v.y; x[i + 2] = v.z; x[i + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < EPL; ++i) x[i] = (e0 + i < a.E) ? row[e0 + i] : 0.f;
        }
    } else {
#pragma unroll
        for (int i = 0; i < EPL; ++i) x[i] = (e0 + i < a.E) ? row[e0 + i] : 0.f;
    }

    // score (what the weights use) and selection key per expert
    float s[EPL];
    uint32_t key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = e0 + i;
        float kf;
        if (sigmoid) {
            s[i] = pinned_sigmoid(x[i]);
            kf = (a.bias != nullptr && e < a.E) ? s[i] + a.bias[e] : s[i];
        } else {
            s[i] = x[i];
            kf = x[i];
        }
        key[i] = (e < a.E) ? order_key(kf) : 0u;
    }

    // group limit: score each run of lanes, keep the topk_groups best runs
    if (a.n_groups > 1) {
        const int lpg = a.lanes_per_group;
        const int seg_base = lane & ~(lpg - 1);
        const uint64_t seg_mask = (lpg == 64) ? ~0ull : (((1ull << lpg) - 1ull) << seg_base);
        uint32_t gk[EPL];
#pragma unroll
        for (int i = 0; i < EPL; ++i) gk[i] = key[i];
        float gsum = 0.f;
        for (int r = 0; r < a.group_topn; ++r) {
            uint32_t b = 0;
            int bi = 0;
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (gk[i] > b) { b = gk[i]; bi = i; }
            const uint32_t m = tk::max_run_u32(b, lpg);
            const uint64_t won = __ballot(b == m) & seg_mask;
            const int wl = __ffsll(static_cast<long long>(won)) - 1;
            if (lane == wl) {
#pragma unroll
                for (int i = 0; i < EPL; ++i)
                    if (i == bi) gk[i] = 0;
            }
            const float v = key_value(m);
            gsum = (r == 0) ? v : gsum + v;
        }
        const int g = lane / lpg;
        int rank = 0;
        for (int gp = 0; gp < a.n_groups; ++gp) {
            const float o = readlane_f(gsum, gp * lpg);
            rank += (o > gsum || (o == gsum && gp < g)) ? 1 : 0;
        }
        if (rank >= a.topk_groups) {
#pragma unroll
            for (int i = 0; i < EPL; ++i) key[i] = 0;
        }
    }

    // softmax over all experts (only when not renormalising)
    float xmax = 0.f, zall = 0.f;
    if (!sigmoid && !a.renormalize) {
        float m = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (e0 + i < a.E) m = fmaxf(m, x[i]);
        for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        xmax = m;
        float z = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (e0 + i < a.E) z += expf(x[i] - xmax);
        for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off);
        zall = z;
    }

    // k rounds of argmax; lane j keeps the winner of round j
    float my_v = 0.f, x0 = 0.f, zsum = 0.f;
    int my_e = 0;
    for (int j = 0; j < a.k; ++j) {
        uint32_t b = 0;
        int bi = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (key[i] > b) { b = key[i]; bi = i; }
        const uint32_t m = tk::max_wave_u32(b);
        const uint64_t won = __ballot(b == m);
        const int wl = tk::uniform(__ffsll(static_cast<long long>(won)) - 1);
        float sv = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (i == bi) sv = s[i];
        const float v = readlane_f(sv, wl);
        const int e = wl * EPL + readlane_i(bi, wl);
        if (lane == wl) {
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (i == bi) key[i] = 0;
        }
        if (lane == j) { my_v = v; my_e = e; }
        if (sigmoid) {
            zsum = (j == 0) ? v : zsum + v;
        } else {
            if (j == 0) x0 = v;
            const float ev = expf(v - x0);
            zsum = (j == 0) ? ev : zsum + ev;
        }
    }

    if (lane < a.k) {
        float w;
        if (sigmoid)
            w = a.renormalize ? (my_v / zsum) * a.route_scale : my_v * a.route_scale;
        else if (a.renormalize)
            w = (expf(my_v - x0) / zsum) * a.route_scale;
        else
            w = (expf(my_v - xmax) / zall) * a.route_scale;
        const size_t o = static_cast<size_t>(t) * a.k + lane;
        a.topk_idx[o] = my_e;
        a.topk_w[o] = w;
    }
}

// Experts per lane: the power of two that fits E into one wave.
int experts_per_lane(int E)
{
    int epl = 1;
    while (epl * tk::kWave < E) epl *= 2;
    return epl;
}

}  // namespace

TK_EXPORT tk_status tk_route(const float* logits, const float* bias, int32_t T, int32_t E,
                             int32_t k, const tk_route_opts* opts, int32_t* topk_idx,
                             float* topk_w, hipStream_t stream)
{
    using tk::fail;
    if (opts == nullptr) return fail(TK_ERR_ARG, "tk_route: opts is NULL");
    if (T < 0) return fail(TK_ERR_ARG, "tk_route: T=%d < 0", T);
    if (E < 1) return fail(TK_ERR_ARG, "tk_route: E=%d < 1", E);
    if (E > TK_MAX_EXPERTS)
        return fail(TK_ERR_UNSUPPORTED, "tk_route: E=%d > %d", E, TK_MAX_EXPERTS);
    if (k < 1 || k > E) return fail(TK_ERR_ARG, "tk_route: k=%d not in [1, E=%d]", k, E);
    if (k > TK_MAX_TOPK) return fail(TK_ERR_UNSUPPORTED, "tk_route: k=%d > %d", k, TK_MAX_TOPK);
    if (opts->score != TK_SCORE_SOFTMAX && opts->score != TK_SCORE_SIGMOID)
        return fail(TK_ERR_ARG, "tk_route: unknown score %d", opts->score);
    if (bias != nullptr && opts->score != TK_SCORE_SIGMOID)
        return fail(TK_ERR_ARG, "tk_route: bias is only defined for sigmoid scores");
    if (opts->n_groups < 1 || E % opts->n_groups != 0)
        return fail(TK_ERR_ARG, "tk_route: n_groups=%d must divide E=%d", opts->n_groups, E);
    const int epl = experts_per_lane(E);
    int lpg = 0;
    if (opts->n_groups > 1) {
        const int gs = E / opts->n_groups;
        if (opts->topk_groups < 1 || opts->topk_groups > opts->n_groups)
            return fail(TK_ERR_ARG, "tk_route: topk_groups=%d not in [1, n_groups=%d]",
                        opts->topk_groups, opts->n_groups);
        if (opts->group_topn < 1 || opts->group_topn > gs)
            return fail(TK_ERR_ARG, "tk_route: group_topn=%d not in [1, group size %d]",
                        opts->group_topn, gs);
        if (opts->topk_groups * gs < k)
            return fail(TK_ERR_ARG, "tk_route: %d groups of %d experts hold fewer than k=%d",
                        opts->topk_groups, gs, k);
        if (gs % epl != 0 || ((gs / epl) & (gs / epl - 1)) != 0)
            return fail(TK_ERR_UNSUPPORTED,
                        "tk_route: group size %d is not a power-of-two run of lanes "
                        "(%d experts per lane)", gs, epl);
        lpg = gs / epl;
    }
    if (T == 0) return tk::ok();
    if (logits == nullptr || topk_idx == nullptr || topk_w == nullptr)
        return fail(TK_ERR_ARG, "tk_route: NULL tensor pointer");
    if (!tk::aligned4(logits) || !tk::aligned4(topk_idx) || !tk::aligned4(topk_w) ||
        (bias && !tk::aligned4(bias)))
        return fail(TK_ERR_ARG, "tk_route: fp32/int32 tensors must be 4-byte aligned");
    if (epl >= 4 && E % 4 == 0 && !tk::aligned16(logits))
        return fail(TK_ERR_ARG, "tk_route: logits must be 16-byte aligned when E %% 4 == 0");

    RouteArgs a{logits, bias, topk_idx, topk_w, T, E, k,
                opts->score, opts->n_groups, opts->topk_groups, opts->group_topn,
                opts->renormalize ? 1 : 0, lpg, opts->route_scale};
    const dim3 grid((T + tk::kWavesPerBlock - 1) / tk::kWavesPerBlock), block(tk::kBlock);
    hipError_t e;
    switch (epl) {
    case 1: e = tk::launch(route_kernel<1>, grid, block, 0, stream, a); break;
    case 2: e = tk::launch(route_kernel<2>, grid, block, 0, stream, a); break;
    case 4: e = tk::launch(route_kernel<4>, grid, block, 0, stream, a); break;
    case 8: e = tk::launch(route_kernel<8>, grid, block, 0, stream, a); break;
    default: e = tk::launch(route_kernel<16>, grid, block, 0, stream, a); break;
    }
    return tk::launched(e, "tk_route");
}
