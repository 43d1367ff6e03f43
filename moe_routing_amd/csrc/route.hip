// tk_route: top-k expert gating and scoring, one token per 64-lane wave (two
// per wave, one per 32-lane half, for many tokens with 128 < E <= 256).
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
// lanes, so group scores use butterflies confined to the run.  The
// two-tokens-per-wave form lays each token over half a wave in the same way.
#include "tk_internal.h"

namespace {

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
            s[i] = tk::pinned_sigmoid(x[i]);
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

// ------------------------------------------------------------ fast kernel
// The same selection, specialised at compile time for EPL <= 4 experts per
// lane, a fixed k and one score function, with renormalised weights and
// group_topn <= 2.  Differences in how it gets there (not in what it
// computes):
//  - each lane sorts its EPL keys once, descending, as 64-bit composites
//    (key << 32 | EPL-1-i), so equal keys keep the lower expert first; a
//    round of the top-k is then one wave max over the lanes' heads, a ballot
//    whose lowest lane holds the lowest expert with that key, and a pop of
//    the winning lane's list;
//  - a group's top-2 keys come from a butterfly over its lanes that merges
//    (largest, second largest) pairs;
//  - groups are ranked with one lane transpose and a ballot count when a
//    group spans at least as many lanes as there are groups;
//  - lane j fetches slot j's score from the lane holding it (ds_bpermute)
//    for the weights.
struct FastArgs {
    const float* logits;
    const float* bias;
    int32_t* topk_idx;
    float* topk_w;
    int T, E;
    int n_groups, topk_groups, group_topn, lanes_per_group;
    float route_scale;
};

// (largest, second largest) of the union of two such pairs
__device__ __forceinline__ void merge_top2(uint32_t& a1, uint32_t& a2, uint32_t b1, uint32_t b2)
{
    const uint32_t lo = min(a1, b1);
    a1 = max(a1, b1);
    a2 = max(lo, max(a2, b2));
}

template <int CTRL>
__device__ __forceinline__ void merge_top2_dpp(uint32_t& m1, uint32_t& m2)
{
    merge_top2(m1, m2, tk::dpp_u32<CTRL>(m1), tk::dpp_u32<CTRL>(m2));
}

__device__ __forceinline__ void merge_top2_xor(uint32_t& m1, uint32_t& m2, int off)
{
    merge_top2(m1, m2, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m1), off)),
               static_cast<uint32_t>(__shfl_xor(static_cast<int>(m2), off)));
}

__device__ __forceinline__ void cas_desc(uint64_t& a, uint64_t& b)
{
    const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
    a = hi;
    b = lo;
}

template <int EPL, int K, bool SIGMOID>
__global__ __launch_bounds__(tk::kBlock) void route_fast_kernel(FastArgs a)
{
    static_assert(EPL == 1 || EPL == 2 || EPL == 4, "fast route handles 1, 2 or 4 experts per lane");
    const int lane = threadIdx.x & (tk::kWave - 1);
    const int t = blockIdx.x * tk::kWavesPerBlock + tk::uniform(threadIdx.x / tk::kWave);
    if (t >= a.T) return;
    const float* row = a.logits + static_cast<size_t>(t) * a.E;
    const int e0 = lane * EPL;
    const bool has_bias = a.bias != nullptr;

    float x[EPL], b[EPL];
    if (EPL == 4 && (a.E & 3) == 0) {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f), w = v;
        if (e0 < a.E) {
            v = *reinterpret_cast<const float4*>(row + e0);
            if (has_bias) w = *reinterpret_cast<const float4*>(a.bias + e0);
        }
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
        b[0] = w.x; b[1] = w.y; b[2] = w.z; b[3] = w.w;
    } else {
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const bool in = e0 + i < a.E;
            x[i] = in ? row[e0 + i] : 0.f;
            b[i] = (in && has_bias) ? a.bias[e0 + i] : 0.f;
        }
    }

    // scores (what the weights use) and selection keys (order-preserving
    // uint32, 0 = not eligible)
    float sc[EPL];
    uint32_t key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        float kf;
        if constexpr (SIGMOID) {
            sc[i] = tk::pinned_sigmoid(x[i]);
            kf = has_bias ? sc[i] + b[i] : sc[i];
        } else {
            sc[i] = x[i];
            kf = x[i];
        }
        key[i] = (e0 + i < a.E) ? order_key(kf) : 0u;
    }

    // group limit
    if (a.n_groups > 1) {
        uint32_t m1 = 0, m2 = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            m2 = max(m2, min(m1, key[i]));
            m1 = max(m1, key[i]);
        }
        const int lpg = a.lanes_per_group;
        if (lpg >= 2) merge_top2_dpp<tk::kQuadXor1>(m1, m2);
        if (lpg >= 4) merge_top2_dpp<tk::kQuadXor2>(m1, m2);
        if (lpg >= 8) merge_top2_dpp<tk::kHalfMirror>(m1, m2);
        if (lpg >= 16) merge_top2_dpp<tk::kMirror>(m1, m2);
        if (lpg >= 32) merge_top2_xor(m1, m2, 16);
        if (lpg >= 64) merge_top2_xor(m1, m2, 32);
        const float gs = (a.group_topn == 2) ? key_value(m1) + key_value(m2) : key_value(m1);
        const uint32_t og = order_key(gs);
        const int g = lane / lpg;
        int rank = 0;
        if (lpg >= a.n_groups) {
            // lane i of group g compares group g with group i; a ballot over
            // the group's lanes counts the groups that beat g
            const int i = lane & (lpg - 1);
            const bool real = i < a.n_groups;
            const uint32_t oi = static_cast<uint32_t>(__shfl(static_cast<int>(og), (real ? i : 0) * lpg));
            const bool beats = real && (oi > og || (oi == og && i < g));
            const uint64_t bal = __ballot(beats);
            const uint64_t seg = (lpg == 64) ? ~0ull : (((1ull << lpg) - 1ull) << (g * lpg));
            rank = __popcll(bal & seg);
        } else {
            for (int gp = 0; gp < a.n_groups; ++gp) {
                const uint32_t o = static_cast<uint32_t>(readlane_i(static_cast<int>(og), gp * lpg));
                rank += (o > og || (o == og && gp < g)) ? 1 : 0;
            }
        }
        if (rank >= a.topk_groups) {
#pragma unroll
            for (int i = 0; i < EPL; ++i) key[i] = 0;
        }
    }

    // per-lane list, sorted descending; ties keep the lower expert first.
    // Sorted as 64-bit (key << 32 | EPL-1-i) composites, then split into the
    // keys and a packed list of 2-bit local indices, head in the low bits.
    uint32_t lk[EPL];
    uint32_t li_packed = 0;
    {
        uint64_t c[EPL];
#pragma unroll
        for (int i = 0; i < EPL; ++i) c[i] = (static_cast<uint64_t>(key[i]) << 32) | (EPL - 1 - i);
        if constexpr (EPL == 2) {
            cas_desc(c[0], c[1]);
        } else if constexpr (EPL == 4) {
            cas_desc(c[0], c[1]); cas_desc(c[2], c[3]);
            cas_desc(c[0], c[2]); cas_desc(c[1], c[3]);
            cas_desc(c[1], c[2]);
        }
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            lk[i] = static_cast<uint32_t>(c[i] >> 32);
            li_packed |= (EPL - 1 - static_cast<uint32_t>(c[i] & 3u)) << (2 * i);
        }
    }

    int my_e = 0;
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const uint32_t m = tk::max_wave_u32(lk[0]);
        const uint64_t won = __ballot(lk[0] == m);
        const int wl = tk::uniform(__ffsll(static_cast<long long>(won)) - 1);
        const int e = wl * EPL + readlane_i(static_cast<int>(li_packed & 3u), wl);
        if (lane == j) my_e = e;
        if (lane == wl) {
#pragma unroll
            for (int i = 0; i + 1 < EPL; ++i) lk[i] = lk[i + 1];
            lk[EPL - 1] = 0;
            li_packed >>= 2;
        }
    }

    // weights over the chosen experts, sums in slot order; lane j fetches
    // the score of its expert from the lane that holds it
    const int src_lane = my_e / EPL, src_i = my_e % EPL;
    float sv = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const float v = __shfl(sc[i], src_lane);
        if (i == src_i) sv = v;
    }
    float z = 0.f, v0 = 0.f;
    if constexpr (SIGMOID) {
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const float v = readlane_f(sv, j);
            z = (j == 0) ? v : z + v;
        }
    } else {
        v0 = readlane_f(sv, 0);
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const float ev = expf(readlane_f(sv, j) - v0);
            z = (j == 0) ? ev : z + ev;
        }
    }
    if (lane < K) {
        const float num = SIGMOID ? sv : expf(sv - v0);
        const size_t o = static_cast<size_t>(t) * K + lane;
        a.topk_idx[o] = my_e;
        a.topk_w[o] = (num / z) * a.route_scale;
    }
}

// ------------------------------------------------------- two tokens per wave
// For many tokens (the grid then holds more waves than the SIMDs can run at
// once and the kernel is bound by VALU issue): the fast kernel's selection
// for 128 < E <= 256 (E a multiple of 8) with two tokens per wave -- lanes
// [0, 32) hold one token, lanes [32, 64) the next, eight experts per lane.
// The cross-lane work (group top-2 butterflies, the group ranking, the k
// rounds of max + ballot) then serves two tokens per instruction; the
// lane-local work (scores, the sort of eight keys) costs the same per token.
// A round's maximum over a half is four DPP steps within 16-lane rows and one
// row exchange (v_permlane16_swap swaps rows 0 and 1, 2 and 3), which leaves
// each half's maximum in all of its lanes.  With fewer tokens the longer
// per-wave instruction stream is not hidden and the one-token kernel is
// faster, so the host takes this form from kHalfMinTokens on.
constexpr int kHalfMinTokens = 12288;

__device__ __forceinline__ uint32_t max_half_u32(uint32_t v)
{
    v = max(v, tk::dpp_u32<tk::kQuadXor1>(v));
    v = max(v, tk::dpp_u32<tk::kQuadXor2>(v));
    v = max(v, tk::dpp_u32<tk::kHalfMirror>(v));
    v = max(v, tk::dpp_u32<tk::kMirror>(v));
    const auto sw = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return max(static_cast<uint32_t>(sw[0]), static_cast<uint32_t>(sw[1]));
}

template <int K, bool SIGMOID>
__global__ __launch_bounds__(tk::kBlock) void route_half_kernel(FastArgs a)
{
    constexpr int EPL = 8;
    const int lane = threadIdx.x & (tk::kWave - 1);
    const int half = lane >> 5, hl = lane & 31;
    const int t0 = 2 * (blockIdx.x * tk::kWavesPerBlock + tk::uniform(threadIdx.x / tk::kWave));
    if (t0 >= a.T) return;
    const int t = t0 + half;
    const bool live = t < a.T;                 // the last wave's second token may not exist
    const float* row = a.logits + static_cast<size_t>(live ? t : t0) * a.E;
    const int e0 = hl * EPL;
    const bool has_bias = a.bias != nullptr;

    float x[EPL], b[EPL];
    {
        float4 v0 = make_float4(0.f, 0.f, 0.f, 0.f), v1 = v0, w0 = v0, w1 = v0;
        if (e0 < a.E) {
            v0 = *reinterpret_cast<const float4*>(row + e0);
            v1 = *reinterpret_cast<const float4*>(row + e0 + 4);
            if (has_bias) {
                w0 = *reinterpret_cast<const float4*>(a.bias + e0);
                w1 = *reinterpret_cast<const float4*>(a.bias + e0 + 4);
            }
        }
        x[0] = v0.x; x[1] = v0.y; x[2] = v0.z; x[3] = v0.w;
        x[4] = v1.x; x[5] = v1.y; x[6] = v1.z; x[7] = v1.w;
        b[0] = w0.x; b[1] = w0.y; b[2] = w0.z; b[3] = w0.w;
        b[4] = w1.x; b[5] = w1.y; b[6] = w1.z; b[7] = w1.w;
    }
    const bool mine = live && e0 < a.E;
    float sc[EPL];
    uint32_t key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        float kf;
        if constexpr (SIGMOID) {
            sc[i] = tk::pinned_sigmoid(x[i]);
            kf = has_bias ? sc[i] + b[i] : sc[i];
        } else {
            sc[i] = x[i];
            kf = x[i];
        }
        key[i] = mine ? order_key(kf) : 0u;
    }

    // group limit: groups are runs of lpg lanes inside a half
    if (a.n_groups > 1) {
        uint32_t m1 = 0, m2 = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            m2 = max(m2, min(m1, key[i]));
            m1 = max(m1, key[i]);
        }
        const int lpg = a.lanes_per_group;
        if (lpg >= 2) merge_top2_dpp<tk::kQuadXor1>(m1, m2);
        if (lpg >= 4) merge_top2_dpp<tk::kQuadXor2>(m1, m2);
        if (lpg >= 8) merge_top2_dpp<tk::kHalfMirror>(m1, m2);
        if (lpg >= 16) merge_top2_dpp<tk::kMirror>(m1, m2);
        const float gs = (a.group_topn == 2) ? key_value(m1) + key_value(m2) : key_value(m1);
        const uint32_t og = order_key(gs);
        // lane i of group g compares g with groups i, i + lpg, ...; a ballot
        // over the group's lanes counts the groups that beat g
        const int g = hl / lpg, i = hl & (lpg - 1);
        const uint64_t seg = ((1ull << lpg) - 1ull) << (lane & ~(lpg - 1));
        int rank = 0;
        for (int gp0 = 0; gp0 < a.n_groups; gp0 += lpg) {
            const int gp = gp0 + i;
            const bool real = gp < a.n_groups;
            const uint32_t o = static_cast<uint32_t>(
                __shfl(static_cast<int>(og), (half << 5) + (real ? gp : 0) * lpg));
            const bool beats = real && (o > og || (o == og && gp < g));
            rank += __popcll(__ballot(beats) & seg);
        }
        if (rank >= a.topk_groups) {
#pragma unroll
            for (int i2 = 0; i2 < EPL; ++i2) key[i2] = 0;
        }
    }

    // the lane's eight keys sorted descending as (key << 32 | 7 - i)
    // composites (equal keys keep the lower expert first), by a 19-comparator
    // network; then split into keys and a packed list of 3-bit local indices,
    // head in the low bits
    uint32_t lk[EPL];
    uint32_t li_packed = 0;
    {
        uint64_t c[EPL];
#pragma unroll
        for (int i = 0; i < EPL; ++i) c[i] = (static_cast<uint64_t>(key[i]) << 32) | (EPL - 1 - i);
        cas_desc(c[0], c[2]); cas_desc(c[1], c[3]); cas_desc(c[4], c[6]); cas_desc(c[5], c[7]);
        cas_desc(c[0], c[4]); cas_desc(c[1], c[5]); cas_desc(c[2], c[6]); cas_desc(c[3], c[7]);
        cas_desc(c[0], c[1]); cas_desc(c[2], c[3]); cas_desc(c[4], c[5]); cas_desc(c[6], c[7]);
        cas_desc(c[2], c[4]); cas_desc(c[3], c[5]);
        cas_desc(c[1], c[4]); cas_desc(c[3], c[6]);
        cas_desc(c[1], c[2]); cas_desc(c[3], c[4]); cas_desc(c[5], c[6]);
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            lk[i] = static_cast<uint32_t>(c[i] >> 32);
            li_packed |= (EPL - 1 - static_cast<uint32_t>(c[i] & 7u)) << (3 * i);
        }
    }

    // k rounds: each half's maximum head, the lowest lane of the half that
    // holds it (a ballot split in two), and a pop of that lane's list
    int my_e = 0;
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const uint32_t m = max_half_u32(lk[0]);
        const uint64_t won = __ballot(lk[0] == m);
        // each half has a lane at its maximum, so neither half of the ballot is 0
        const int wl0 = tk::uniform(__builtin_ctz(static_cast<uint32_t>(won)));
        const int wl1 = 32 + tk::uniform(__builtin_ctz(static_cast<uint32_t>(won >> 32)));
        const int li0 = readlane_i(static_cast<int>(li_packed & 7u), wl0);
        const int li1 = readlane_i(static_cast<int>(li_packed & 7u), wl1);
        const int e = half ? (wl1 - 32) * EPL + li1 : wl0 * EPL + li0;
        if (hl == j) my_e = e;
        if (lane == wl0 || lane == wl1) {
#pragma unroll
            for (int i = 0; i + 1 < EPL; ++i) lk[i] = lk[i + 1];
            lk[EPL - 1] = 0;
            li_packed >>= 3;
        }
    }

    // weights, sums in slot order: lane j of a half fetches the score of its
    // slot's expert from the lane that holds it
    const int src_lane = (half << 5) + my_e / EPL, src_i = my_e % EPL;
    float sv = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const float v = __shfl(sc[i], src_lane);
        if (i == src_i) sv = v;
    }
    float z0 = 0.f, z1 = 0.f, x00 = 0.f, x01 = 0.f;
    if constexpr (!SIGMOID) {
        x00 = readlane_f(sv, 0);
        x01 = readlane_f(sv, 32);
    }
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const float v0 = readlane_f(sv, j), v1 = readlane_f(sv, 32 + j);
        const float a0 = SIGMOID ? v0 : expf(v0 - x00), a1 = SIGMOID ? v1 : expf(v1 - x01);
        z0 = (j == 0) ? a0 : z0 + a0;
        z1 = (j == 0) ? a1 : z1 + a1;
    }
    if (live && hl < K) {
        const float z = half ? z1 : z0;
        const float num = SIGMOID ? sv : expf(sv - (half ? x01 : x00));
        const size_t o = static_cast<size_t>(t) * K + hl;
        a.topk_idx[o] = my_e;
        a.topk_w[o] = (num / z) * a.route_scale;
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
    if (epl >= 4 && E % 4 == 0 && (!tk::aligned16(logits) || (bias && !tk::aligned16(bias))))
        return fail(TK_ERR_ARG,
                    "tk_route: logits and bias must be 16-byte aligned when E %% 4 == 0 and E > 128");

    const bool half_ok = T >= kHalfMinTokens && E > 128 && E <= 256 && E % 8 == 0 && k <= 8 &&
                         (opts->n_groups == 1 || (E / opts->n_groups) % 8 == 0);
    if (opts->renormalize && half_ok && (opts->n_groups == 1 || opts->group_topn <= 2)) {
        const FastArgs f{logits, bias, topk_idx, topk_w, T, E, opts->n_groups,
                         opts->topk_groups, opts->group_topn,
                         opts->n_groups > 1 ? E / opts->n_groups / 8 : 0, opts->route_scale};
        const int64_t tokens_per_block = 2 * tk::kWavesPerBlock;
        const dim3 grid(static_cast<unsigned>((static_cast<int64_t>(T) + tokens_per_block - 1) /
                                              tokens_per_block)),
            block(tk::kBlock);
        const bool sig = opts->score == TK_SCORE_SIGMOID;
        hipError_t e = hipErrorInvalidValue;
#define TK_ROUTE_HALF(K_)                                                                          \
    e = sig ? tk::launch(route_half_kernel<K_, true>, grid, block, 0, stream, f)                   \
            : tk::launch(route_half_kernel<K_, false>, grid, block, 0, stream, f)
        switch (k) {
        case 1: TK_ROUTE_HALF(1); break;
        case 2: TK_ROUTE_HALF(2); break;
        case 3: TK_ROUTE_HALF(3); break;
        case 4: TK_ROUTE_HALF(4); break;
        case 5: TK_ROUTE_HALF(5); break;
        case 6: TK_ROUTE_HALF(6); break;
        case 7: TK_ROUTE_HALF(7); break;
        default: TK_ROUTE_HALF(8); break;   // k == 8
        }
#undef TK_ROUTE_HALF
        return tk::launched(e, "tk_route");
    }
    if (opts->renormalize && epl <= 4 && (opts->n_groups == 1 || opts->group_topn <= 2)) {
        const FastArgs f{logits, bias, topk_idx, topk_w, T, E, opts->n_groups,
                         opts->topk_groups, opts->group_topn, lpg, opts->route_scale};
        const dim3 grid(static_cast<unsigned>((static_cast<int64_t>(T) + tk::kWavesPerBlock - 1) /
                                              tk::kWavesPerBlock)),
            block(tk::kBlock);
        const bool sig = opts->score == TK_SCORE_SIGMOID;
        hipError_t e = hipErrorInvalidValue;
        bool launched = true;
#define TK_ROUTE_FAST(EPL_, K_)                                                                    \
    e = sig ? tk::launch(route_fast_kernel<EPL_, K_, true>, grid, block, 0, stream, f)             \
            : tk::launch(route_fast_kernel<EPL_, K_, false>, grid, block, 0, stream, f)
        switch (epl * 100 + k) {
        case 101: TK_ROUTE_FAST(1, 1); break;
        case 102: TK_ROUTE_FAST(1, 2); break;
        case 103: TK_ROUTE_FAST(1, 3); break;
        case 104: TK_ROUTE_FAST(1, 4); break;
        case 105: TK_ROUTE_FAST(1, 5); break;
        case 106: TK_ROUTE_FAST(1, 6); break;
        case 107: TK_ROUTE_FAST(1, 7); break;
        case 108: TK_ROUTE_FAST(1, 8); break;
        case 201: TK_ROUTE_FAST(2, 1); break;
        case 202: TK_ROUTE_FAST(2, 2); break;
        case 203: TK_ROUTE_FAST(2, 3); break;
        case 204: TK_ROUTE_FAST(2, 4); break;
        case 205: TK_ROUTE_FAST(2, 5); break;
        case 206: TK_ROUTE_FAST(2, 6); break;
        case 207: TK_ROUTE_FAST(2, 7); break;
        case 208: TK_ROUTE_FAST(2, 8); break;
        case 401: TK_ROUTE_FAST(4, 1); break;
        case 402: TK_ROUTE_FAST(4, 2); break;
        case 403: TK_ROUTE_FAST(4, 3); break;
        case 404: TK_ROUTE_FAST(4, 4); break;
        case 405: TK_ROUTE_FAST(4, 5); break;
        case 406: TK_ROUTE_FAST(4, 6); break;
        case 407: TK_ROUTE_FAST(4, 7); break;
        case 408: TK_ROUTE_FAST(4, 8); break;
        default: launched = false; break;
        }
#undef TK_ROUTE_FAST
        if (launched) return tk::launched(e, "tk_route");
    }

    RouteArgs a{logits, bias, topk_idx, topk_w, T, E, k,
                opts->score, opts->n_groups, opts->topk_groups, opts->group_topn,
                opts->renormalize ? 1 : 0, lpg, opts->route_scale};
    const dim3 grid(static_cast<unsigned>((static_cast<int64_t>(T) + tk::kWavesPerBlock - 1) /
                                          tk::kWavesPerBlock)),
        block(tk::kBlock);
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
