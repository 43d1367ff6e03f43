// tk_map: token-to-expert mapping (counts, offsets, stable positions) with a
// local-expert mask; the "token-to-expert mapping" and "tensor-parallel mask"
// ops of TileKernels' moe/ module ("刚刚！DeepSeek开源高性能GPU算子库TileKernels",
// item moe/).
//
// Three launches, no atomics on global memory, so every output is a pure
// function of topk_idx:
//   1. hist    one workgroup per tile of tokens: LDS histogram of the local
//              experts -> tile_counts[tile][e] in the workspace
//   2. scan    one workgroup: per expert, exclusive scan over tiles; block
//              scan over experts -> counts, offsets; the workspace becomes
//              tile_base[tile][e] = first row of expert e owned by the tile
//   3. scatter one workgroup per tile: a bit mask per (expert, 32-token
//              sub-tile) in LDS; the rank of token t among the tile's tokens
//              routed to e is (tokens of e in earlier sub-tiles) + popcount of
//              the bits below t in its own sub-tile.  pos = tile_base + rank.
// Ranks follow token order, which is the stable order because a token is
// routed to an expert at most once (repeats in a row are dropped).
#include "tk_internal.h"

namespace {

constexpr int kSub = 32;                 // tokens per sub-tile (one mask word)
constexpr int kMaskWords = 4096;         // LDS budget: n_local * sub-tiles <= this

// Sub-tiles per tile for n_local local experts (tile = 32 * S tokens).
__host__ __device__ inline int subtiles_per_tile(int n_local)
{
    int s = kMaskWords / n_local;
    return s > 32 ? 32 : (s < 1 ? 1 : s);
}

// Token t's k expert ids as local indices (id - lo); -1 for an id outside
// [lo, hi) and for a repeat of an id earlier in the row.
template <int KMAX>
__device__ __forceinline__ void load_local_ids(const int32_t* __restrict__ idx, int t, int k,
                                               int lo, int hi, int (&e)[KMAX])
{
    const int32_t* r = idx + static_cast<size_t>(t) * k;
    int raw[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) raw[j] = (j < k) ? r[j] : -1;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        bool keep = (j < k) && raw[j] >= lo && raw[j] < hi;
#pragma unroll
        for (int jj = 0; jj < j; ++jj) keep = keep && (raw[jj] != raw[j]);
        e[j] = keep ? raw[j] - lo : -1;
    }
}

template <int KMAX>
__global__ __launch_bounds__(tk::kBlock) void map_hist_kernel(
    const int32_t* __restrict__ idx, int T, int k, int lo, int hi, int tile_tokens,
    int32_t* __restrict__ tile_counts)
{
    extern __shared__ int32_t cnt[];
    const int nl = hi - lo;
    for (int i = threadIdx.x; i < nl; i += tk::kBlock) cnt[i] = 0;
    __syncthreads();
    const int t0 = blockIdx.x * tile_tokens;
    for (int tl = threadIdx.x; tl < tile_tokens; tl += tk::kBlock) {
        const int t = t0 + tl;
        if (t >= T) break;
        int e[KMAX];
        load_local_ids<KMAX>(idx, t, k, lo, hi, e);
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (e[j] >= 0) atomicAdd(&cnt[e[j]], 1);
    }
    __syncthreads();
    int32_t* out = tile_counts + static_cast<size_t>(blockIdx.x) * nl;
    for (int i = threadIdx.x; i < nl; i += tk::kBlock) out[i] = cnt[i];
}

constexpr int kScanThreads = 1024;

// tile_counts[tile][e] -> tile_base[tile][e] (in place); counts, offsets.
__global__ __launch_bounds__(kScanThreads) void map_scan_kernel(
    int32_t* __restrict__ tiles, int n_tiles, int nl, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets)
{
    __shared__ int32_t tot[TK_MAX_EXPERTS];
    __shared__ int32_t wave_sum[kScanThreads / tk::kWave];
    // per expert: exclusive scan over tiles (coalesced across experts)
    for (int e = threadIdx.x; e < nl; e += kScanThreads) {
        int32_t run = 0;
        for (int tile = 0; tile < n_tiles; ++tile) {
            int32_t* p = tiles + static_cast<size_t>(tile) * nl + e;
            const int32_t c = *p;
            *p = run;
            run += c;
        }
        tot[e] = run;
        counts[e] = run;
    }
    __syncthreads();
    // exclusive scan of tot over experts (nl <= 1024 = one element per thread)
    const int lane = threadIdx.x & (tk::kWave - 1), wave = threadIdx.x / tk::kWave;
    const int v = (threadIdx.x < nl) ? tot[threadIdx.x] : 0;
    int inc = v;
#pragma unroll
    for (int off = 1; off < tk::kWave; off <<= 1) {
        const int o = __shfl_up(inc, off);
        if (lane >= off) inc += o;
    }
    if (lane == tk::kWave - 1) wave_sum[wave] = inc;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wave_sum[w];
    const int excl = before + inc - v;
    __syncthreads();
    if (threadIdx.x < nl) {
        tot[threadIdx.x] = excl;
        offsets[threadIdx.x] = excl;
    }
    if (threadIdx.x == nl - 1) offsets[nl] = excl + v;
    __syncthreads();
    for (int e = threadIdx.x; e < nl; e += kScanThreads) {
        const int32_t base = tot[e];
        for (int tile = 0; tile < n_tiles; ++tile) tiles[static_cast<size_t>(tile) * nl + e] += base;
    }
}

template <int KMAX>
__global__ __launch_bounds__(tk::kBlock) void map_scatter_kernel(
    const int32_t* __restrict__ idx, int T, int k, int lo, int hi, int S,
    const int32_t* __restrict__ tile_base, int32_t* __restrict__ pos, int32_t* __restrict__ row_src)
{
    extern __shared__ uint32_t lds[];
    const int nl = hi - lo;
    uint32_t* mask = lds;              // [nl][S]
    uint32_t* before = lds + nl * S;   // [nl][S] tokens of e in earlier sub-tiles
    const int tile_tokens = S * kSub;
    for (int i = threadIdx.x; i < nl * S; i += tk::kBlock) mask[i] = 0;
    __syncthreads();
    const int t0 = blockIdx.x * tile_tokens;
    for (int tl = threadIdx.x; tl < tile_tokens; tl += tk::kBlock) {
        const int t = t0 + tl;
        if (t >= T) break;
        int e[KMAX];
        load_local_ids<KMAX>(idx, t, k, lo, hi, e);
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (e[j] >= 0) atomicOr(&mask[e[j] * S + tl / kSub], 1u << (tl % kSub));
    }
    __syncthreads();
    for (int ex = threadIdx.x; ex < nl; ex += tk::kBlock) {
        uint32_t run = 0;
        for (int s = 0; s < S; ++s) {
            before[ex * S + s] = run;
            run += __popc(mask[ex * S + s]);
        }
    }
    __syncthreads();
    const int32_t* base = tile_base + static_cast<size_t>(blockIdx.x) * nl;
    for (int tl = threadIdx.x; tl < tile_tokens; tl += tk::kBlock) {
        const int t = t0 + tl;
        if (t >= T) break;
        int e[KMAX];
        load_local_ids<KMAX>(idx, t, k, lo, hi, e);
        const uint32_t below = (1u << (tl % kSub)) - 1u;
        const int s = tl / kSub;
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            if (j >= k) break;
            int32_t p = -1;
            if (e[j] >= 0) {
                const int w = e[j] * S + s;
                p = base[e[j]] + static_cast<int32_t>(before[w] + __popc(mask[w] & below));
                if (row_src != nullptr) row_src[p] = t;
            }
            pos[static_cast<size_t>(t) * k + j] = p;
        }
    }
}

}  // namespace

TK_EXPORT size_t tk_map_workspace_bytes(int32_t T, int32_t k, int32_t n_local)
{
    (void)k;
    if (T <= 0 || n_local <= 0) return 0;
    const int tile_tokens = subtiles_per_tile(n_local) * kSub;
    const size_t n_tiles = (static_cast<size_t>(T) + tile_tokens - 1) / tile_tokens;
    return n_tiles * static_cast<size_t>(n_local) * sizeof(int32_t);
}

TK_EXPORT tk_status tk_map(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                           int32_t local_begin, int32_t local_end, int32_t* counts,
                           int32_t* offsets, int32_t* pos, int32_t* row_src, void* workspace,
                           size_t workspace_bytes, hipStream_t stream)
{
    using tk::fail;
    if (T < 0) return fail(TK_ERR_ARG, "tk_map: T=%d < 0", T);
    if (k < 1) return fail(TK_ERR_ARG, "tk_map: k=%d < 1", k);
    if (k > TK_MAX_TOPK) return fail(TK_ERR_UNSUPPORTED, "tk_map: k=%d > %d", k, TK_MAX_TOPK);
    if (E < 1 || E > TK_MAX_EXPERTS)
        return fail(E < 1 ? TK_ERR_ARG : TK_ERR_UNSUPPORTED, "tk_map: E=%d not in [1, %d]", E,
                    TK_MAX_EXPERTS);
    if (local_begin < 0 || local_end > E || local_begin >= local_end)
        return fail(TK_ERR_ARG, "tk_map: local range [%d, %d) not a non-empty part of [0, %d)",
                    local_begin, local_end, E);
    if (static_cast<int64_t>(T) * k > INT32_MAX)
        return fail(TK_ERR_ARG, "tk_map: T*k exceeds int32 positions");
    if (counts == nullptr || offsets == nullptr)
        return fail(TK_ERR_ARG, "tk_map: NULL counts/offsets");
    if (T > 0 && (topk_idx == nullptr || pos == nullptr))
        return fail(TK_ERR_ARG, "tk_map: NULL topk_idx/pos");
    const int nl = local_end - local_begin;
    const size_t need = tk_map_workspace_bytes(T, k, nl);
    if (workspace_bytes < need)
        return fail(TK_ERR_ARG, "tk_map: workspace of %zu bytes < %zu needed", workspace_bytes, need);
    if (need > 0 && (workspace == nullptr || !tk::aligned4(workspace)))
        return fail(TK_ERR_ARG, "tk_map: workspace NULL or not 4-byte aligned");

    const int S = subtiles_per_tile(nl);
    const int tile_tokens = S * kSub;
    const int n_tiles = (T + tile_tokens - 1) / tile_tokens;
    int32_t* tiles = static_cast<int32_t*>(workspace);
    const dim3 block(tk::kBlock);
    hipError_t e = hipSuccess;
    if (n_tiles > 0) {
        e = (k <= 8)
            ? tk::launch(map_hist_kernel<8>, dim3(n_tiles), block, nl * sizeof(int32_t), stream,
                         topk_idx, T, k, local_begin, local_end, tile_tokens, tiles)
            : tk::launch(map_hist_kernel<TK_MAX_TOPK>, dim3(n_tiles), block, nl * sizeof(int32_t),
                         stream, topk_idx, T, k, local_begin, local_end, tile_tokens, tiles);
        if (e != hipSuccess) return tk::launched(e, "tk_map (hist)");
    }
    e = tk::launch(map_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, tiles, n_tiles, nl,
                   counts, offsets);
    if (e != hipSuccess) return tk::launched(e, "tk_map (scan)");
    if (n_tiles > 0) {
        const size_t lds = 2 * static_cast<size_t>(nl) * S * sizeof(uint32_t);
        e = (k <= 8)
            ? tk::launch(map_scatter_kernel<8>, dim3(n_tiles), block, lds, stream, topk_idx, T, k,
                         local_begin, local_end, S, tiles, pos, row_src)
            : tk::launch(map_scatter_kernel<TK_MAX_TOPK>, dim3(n_tiles), block, lds, stream,
                         topk_idx, T, k, local_begin, local_end, S, tiles, pos, row_src);
    }
    return tk::launched(e, "tk_map (scatter)");
}
