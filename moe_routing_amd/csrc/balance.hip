// tk_balance_loss: per-expert load statistics and the load-balance loss of
// one batch -- the load-balancing loss computation of TileKernels' moe/
// module ("刚刚！DeepSeek开源高性能GPU算子库TileKernels", item moe/), in the form
// DeepSeek-V3 trains with:
//   count_e = routes (t, j) with topk_idx[t,j] = e;  f_e = E/(k*T) * count_e
//   P_e     = (1/T) sum_t p_{t,e}, p = sigmoid scores / their sum over all E
//             experts (the pinned sigmoid of tk_route), or softmax probabilities
//   loss    = sum_e f_e * P_e
//
// Two launches, every sum in a fixed order (deterministic):
//   1. partial  one workgroup of 8 waves per tile of 32 tokens, one wave per
//               token at a time (lane l holds experts [l*EPL, l*EPL+EPL), as
//               in tk_route): the token's scores, their wave-wide sum (DPP
//               row steps, then the rows in order), p;
//               each wave accumulates p over its tokens in token order, the
//               workgroup adds its waves in wave order -> part_p[tile][e];
//               LDS integer histogram of the tile's routes -> part_c[tile][e]
//   2. final    a workgroup per 32 experts: eight thread groups per expert
//               take the tiles g, g+8, ... in order and are added in group
//               order, giving f and P; the last workgroup to finish (a
//               counter in the workspace, zeroed by the partial pass) then
//               sums f*P over all experts in fp64, in expert order.  The
//               last one reads every other workgroup's f and P after their
//               release fences, so the loss does not depend on which
//               workgroup it is.
#include "tk_internal.h"

namespace {

constexpr int kTileTokens = 32;      // tokens per partial workgroup (4 per wave)
constexpr int kPartialWaves = 8;
constexpr int kPartialThreads = kPartialWaves * 64;
constexpr int kFinalThreads = 256;
constexpr int kFinalExperts = 32;                          // experts per final workgroup
constexpr int kFinalGroups = kFinalThreads / kFinalExperts;  // 8 tile groups

template <int EPL, bool SIGMOID>
__global__ __launch_bounds__(kPartialThreads) void balance_partial_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ idx, int T, int E, int k,
    float* __restrict__ part_p, int32_t* __restrict__ part_c, uint32_t* __restrict__ done)
{
    __shared__ float wave_acc[kPartialWaves][tk::kWave * EPL];
    if (blockIdx.x == 0 && threadIdx.x == 0) *done = 0u;   // the final pass counts on it
    extern __shared__ int32_t hist[];
    const int lane = threadIdx.x & (tk::kWave - 1);
    const int wave = tk::uniform(threadIdx.x / tk::kWave);
    const int tile = blockIdx.x;
    const int t0 = tile * kTileTokens;
    for (int e = threadIdx.x; e < E; e += kPartialThreads) hist[e] = 0;
    __syncthreads();
    // routes of the tile
    for (int i = threadIdx.x; i < kTileTokens * k; i += kPartialThreads) {
        const int t = t0 + i / k;
        if (t < T) {
            const int32_t e = idx[static_cast<size_t>(t0) * k + i];
            if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
        }
    }
    // normalised scores, accumulated in token order by each wave
    float acc[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) acc[i] = 0.f;
    const int e0 = lane * EPL;
    for (int tt = wave; tt < kTileTokens; tt += kPartialWaves) {
        const int t = t0 + tt;
        if (t >= T) break;
        const float* row = logits + static_cast<size_t>(t) * E;
        float s[EPL];
#pragma unroll
        for (int i = 0; i < EPL; ++i) s[i] = (e0 + i < E) ? row[e0 + i] : 0.f;
        float m = 0.f;
        if constexpr (!SIGMOID) {
            m = -__builtin_inff();
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (e0 + i < E) m = fmaxf(m, s[i]);
            m = tk::max_wave_f32(m);
        }
        float z = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            if (e0 + i < E) s[i] = SIGMOID ? tk::pinned_sigmoid(s[i]) : expf(s[i] - m);
            else s[i] = 0.f;
            z += s[i];
        }
        z = tk::sum_wave_f32(z);
#pragma unroll
        for (int i = 0; i < EPL; ++i) acc[i] += s[i] / z;
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) wave_acc[wave][e0 + i] = acc[i];
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kPartialThreads) {
        float v = wave_acc[0][e];
#pragma unroll
        for (int w = 1; w < kPartialWaves; ++w) v += wave_acc[w][e];
        part_p[static_cast<size_t>(tile) * E + e] = v;
        part_c[static_cast<size_t>(tile) * E + e] = hist[e];
    }
}

__global__ __launch_bounds__(kFinalThreads) void balance_final_kernel(
    const float* __restrict__ part_p, const int32_t* __restrict__ part_c, int n_tiles, int T,
    int E, int k, float* __restrict__ f, float* __restrict__ P, float* __restrict__ loss,
    uint32_t* __restrict__ done)
{
    __shared__ float sp[kFinalGroups][kFinalExperts];
    __shared__ int32_t sc[kFinalGroups][kFinalExperts];
    __shared__ double red[kFinalThreads];
    __shared__ bool last;
    const int cl = threadIdx.x % kFinalExperts, g = threadIdx.x / kFinalExperts;
    const int e = blockIdx.x * kFinalExperts + cl;
    float v = 0.f;
    int32_t c = 0;
    if (e < E) {
        for (int t0 = g; t0 < n_tiles; t0 += kFinalGroups * 8) {   // eight tiles' loads in flight
            float pv[8];
            int32_t cv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int t = t0 + i * kFinalGroups;
                pv[i] = t < n_tiles ? part_p[static_cast<size_t>(t) * E + e] : 0.f;
                cv[i] = t < n_tiles ? part_c[static_cast<size_t>(t) * E + e] : 0;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (t0 + i * kFinalGroups < n_tiles) {
                    v += pv[i];
                    c += cv[i];
                }
            }
        }
    }
    sp[g][cl] = v;
    sc[g][cl] = c;
    __syncthreads();
    const double scale = static_cast<double>(E) / (static_cast<double>(k) * static_cast<double>(T));
    if (g == 0 && e < E) {
        int64_t cnt = c;
#pragma unroll
        for (int h = 1; h < kFinalGroups; ++h) {
            v += sp[h][cl];
            cnt += sc[h][cl];
        }
        P[e] = v / static_cast<float>(T);
        f[e] = static_cast<float>(scale * static_cast<double>(cnt));
    }
    // the last workgroup to get here forms the loss from every workgroup's f and P
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) last = atomicAdd(done, 1u) == gridDim.x - 1;
    __syncthreads();
    if (!last) return;
    __threadfence();
    double my = 0.0;
    for (int i = threadIdx.x; i < E; i += kFinalThreads) {
        const float fe = __hip_atomic_load(f + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const float pe = __hip_atomic_load(P + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        my += static_cast<double>(fe) * static_cast<double>(pe);
    }
    red[threadIdx.x] = my;
    __syncthreads();
    for (int w = kFinalThreads / 2; w > 0; w >>= 1) {
        if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) loss[0] = static_cast<float>(red[0]);
}

int experts_per_lane(int E)
{
    int epl = 1;
    while (epl * tk::kWave < E) epl *= 2;
    return epl;
}

}  // namespace

TK_EXPORT size_t tk_balance_workspace_bytes(int32_t T, int32_t E)
{
    if (T <= 0 || E <= 0) return 0;
    const size_t n_tiles = (static_cast<size_t>(T) + kTileTokens - 1) / kTileTokens;
    // per-tile partial sums and counts, then the final pass's counter
    return n_tiles * static_cast<size_t>(E) * (sizeof(float) + sizeof(int32_t)) + 16;
}

TK_EXPORT tk_status tk_balance_loss(const float* logits, const int32_t* topk_idx, int32_t T,
                                    int32_t E, int32_t k, int32_t score, float* f, float* P,
                                    float* loss, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream)
{
    using tk::fail;
    if (T < 1) return fail(TK_ERR_ARG, "tk_balance_loss: T=%d < 1", T);
    if (E < 1) return fail(TK_ERR_ARG, "tk_balance_loss: E=%d < 1", E);
    if (E > TK_MAX_EXPERTS)
        return fail(TK_ERR_UNSUPPORTED, "tk_balance_loss: E=%d > %d", E, TK_MAX_EXPERTS);
    if (k < 1 || k > TK_MAX_TOPK) return fail(TK_ERR_ARG, "tk_balance_loss: k=%d invalid", k);
    if (score != TK_SCORE_SOFTMAX && score != TK_SCORE_SIGMOID)
        return fail(TK_ERR_ARG, "tk_balance_loss: unknown score %d", score);
    if (logits == nullptr || topk_idx == nullptr || f == nullptr || P == nullptr || loss == nullptr)
        return fail(TK_ERR_ARG, "tk_balance_loss: NULL pointer");
    const size_t need = tk_balance_workspace_bytes(T, E);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(TK_ERR_ARG, "tk_balance_loss: workspace of %zu bytes < %zu needed",
                    workspace_bytes, need);
    if (!tk::aligned4(logits) || !tk::aligned4(topk_idx) || !tk::aligned4(f) ||
        !tk::aligned4(P) || !tk::aligned4(loss) || !tk::aligned4(workspace))
        return fail(TK_ERR_ARG, "tk_balance_loss: tensors must be 4-byte aligned");
    const int n_tiles = static_cast<int>((static_cast<int64_t>(T) + kTileTokens - 1) / kTileTokens);
    float* part_p = static_cast<float*>(workspace);
    int32_t* part_c = reinterpret_cast<int32_t*>(part_p + static_cast<size_t>(n_tiles) * E);
    auto* done = reinterpret_cast<uint32_t*>(part_c + static_cast<size_t>(n_tiles) * E);
    const dim3 grid(n_tiles), block(kPartialThreads);
    const size_t lds = static_cast<size_t>(E) * sizeof(int32_t);
    const bool sig = score == TK_SCORE_SIGMOID;
    hipError_t e;
#define TK_BALANCE(EPL_)                                                                           \
    e = sig ? tk::launch(balance_partial_kernel<EPL_, true>, grid, block, lds, stream, logits,     \
                         topk_idx, T, E, k, part_p, part_c, done)                                  \
            : tk::launch(balance_partial_kernel<EPL_, false>, grid, block, lds, stream, logits,    \
                         topk_idx, T, E, k, part_p, part_c, done)
    switch (experts_per_lane(E)) {
    case 1: TK_BALANCE(1); break;
    case 2: TK_BALANCE(2); break;
    case 4: TK_BALANCE(4); break;
    case 8: TK_BALANCE(8); break;
    default: TK_BALANCE(16); break;
    }
#undef TK_BALANCE
    if (e != hipSuccess) return tk::launched(e, "tk_balance_loss (partial)");
    e = tk::launch(balance_final_kernel, dim3((E + kFinalExperts - 1) / kFinalExperts),
                   dim3(kFinalThreads), 0, stream, part_p, part_c, n_tiles, T, E, k, f, P, loss, done);
    return tk::launched(e, "tk_balance_loss (final)");
}
