// tk_map: token-to-expert mapping (counts, offsets, stable positions) with a
// local-expert mask; the token-to-expert mapping and tensor-parallel mask
// ops of TileKernels' moe/ module ("刚刚！DeepSeek开源高性能GPU算子库TileKernels",
// item moe/).
//
// Tokens are cut into tiles of 32*S <= 256 tokens (S sub-tiles of 32), one
// token per thread.  Two launches at the usual sizes (one when all tokens fit
// in one tile: map_single_kernel), no atomics on global memory, so every
// output is a pure function of topk_idx:
//   1. count  one workgroup per tile: LDS histogram of the tile's local
//             routes -> cnt[tile][e] (tile-major: each tile writes whole
//             lines of its own) in the workspace
//   2. place  one workgroup per tile: per expert, the sum over all tiles
//             (total) and over the tiles before this one (before); a block
//             scan of the totals gives offsets; then a bit mask per
//             (expert, sub-tile) in LDS ranks the tile's tokens:
//               pos = offsets[e] + before[e] + (tokens of e in earlier
//                     sub-tiles) + popcount(bits below t in t's sub-tile)
// The place kernel issues its global loads (its tokens' ids, then its
// experts' count columns, 32 tiles per batch, coalesced across the threads
// that own neighbouring experts) before waiting on any of them, so their
// latencies overlap.  When the count matrix is large, a third launch (scan,
// between the two) turns the counts into per-tile prefixes once, so that
// place reads one entry instead of a whole column per expert.
// Ranks follow token order, which is the stable order because a token is
// routed to an expert at most once (repeats in a row are dropped).
// tk_map_aligned pads every expert's segment to a multiple of `align` rows
// (the layout an M-blocked grouped GEMM reads); tk_map is align = 1.
#include <mutex>

#include "tk_internal.h"

namespace {

constexpr int kSub = 32;               // tokens per sub-tile (one mask word)
constexpr int kThreads = 256;          // threads of the count and place kernels
constexpr int kMaxSub = kThreads / kSub;  // one token per thread: tiles <= 256 tokens
constexpr int kMaxFusedInts = 32768;   // count matrix read whole by each place workgroup
constexpr int kLdsWords = 12288;       // place kernel LDS budget (48 KiB)
constexpr int kScanThreads = 1024;
constexpr int kBatch = 32;             // count loads in flight per thread (place, scan)

struct Tiling {
    int S;          // sub-tiles per tile
    int tile;       // tokens per tile
    int n_tiles;
    bool fused;     // place computes prefixes itself
};

__host__ inline Tiling tiling(int T, int n_local)
{
    Tiling g{};
    int s_max = (kLdsWords - 3 * n_local) / (2 * n_local);  // mask + before words per tile
    s_max = s_max < 1 ? 1 : (s_max > kMaxSub ? kMaxSub : s_max);
    const int64_t s = (static_cast<int64_t>(T) + kSub - 1) / kSub;   // no more sub-tiles than tokens need
    g.S = s < 1 ? 1 : (s > s_max ? s_max : static_cast<int>(s));
    g.tile = g.S * kSub;
    g.n_tiles = T > 0 ? static_cast<int>((static_cast<int64_t>(T) + g.tile - 1) / g.tile) : 0;
    g.fused = static_cast<int64_t>(g.n_tiles) * n_local <= kMaxFusedInts;
    return g;
}

// Token t's k expert ids as stored (loads only, so that a caller can issue
// more loads before the first use); -1 past k.
template <int KMAX>
__device__ __forceinline__ void load_raw_ids(const int32_t* __restrict__ idx, int t, int k,
                                             int (&raw)[KMAX])
{
    const int32_t* r = idx + static_cast<size_t>(t) * k;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) raw[j] = (j < k) ? r[j] : -1;
}

// Stored ids -> local indices (id - lo); -1 for an id outside [lo, hi) and
// for a repeat of an id earlier in the row.
template <int KMAX>
__device__ __forceinline__ void local_ids(const int (&raw)[KMAX], int k, int lo, int hi,
                                          int (&e)[KMAX])
{
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        bool keep = (j < k) && raw[j] >= lo && raw[j] < hi;
#pragma unroll
        for (int jj = 0; jj < j; ++jj) keep = keep && (raw[jj] != raw[j]);
        e[j] = keep ? raw[j] - lo : -1;
    }
}

template <int KMAX>
__device__ __forceinline__ void load_local_ids(const int32_t* __restrict__ idx, int t, int k,
                                               int lo, int hi, int (&e)[KMAX])
{
    int raw[KMAX];
    load_raw_ids<KMAX>(idx, t, k, raw);
    local_ids<KMAX>(raw, k, lo, hi, e);
}

template <int KMAX>
__global__ __launch_bounds__(kThreads) void map_count_kernel(
    const int32_t* __restrict__ idx, int T, int k, int lo, int hi, int tile_tokens,
    int32_t* __restrict__ cnt)
{
    extern __shared__ int32_t hist[];
    const int nl = hi - lo;
    const int t = blockIdx.x * tile_tokens + threadIdx.x;
    const bool mine = threadIdx.x < tile_tokens && t < T;
    int e[KMAX];
    if (mine) load_local_ids<KMAX>(idx, t, k, lo, hi, e);
    for (int i = threadIdx.x; i < nl; i += kThreads) hist[i] = 0;
    __syncthreads();
    if (mine) {
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (e[j] >= 0) atomicAdd(&hist[e[j]], 1);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nl; i += kThreads)
        cnt[static_cast<size_t>(blockIdx.x) * nl + i] = hist[i];
}

// Many tiles: cnt[tile][e] -> exclusive prefix over tiles (in place), and
// totals[e] = the sum over all tiles.  One workgroup, a thread per expert;
// each batch of kBatch tiles is loaded before any of it is rewritten.
__global__ __launch_bounds__(kScanThreads) void map_scan_kernel(
    int32_t* __restrict__ cnt, int n_tiles, int nl, int32_t* __restrict__ totals)
{
    for (int e = threadIdx.x; e < nl; e += kScanThreads) {
        int32_t run = 0;
        for (int c0 = 0; c0 < n_tiles; c0 += kBatch) {
            int32_t v[kBatch];
#pragma unroll
            for (int b = 0; b < kBatch; ++b)
                v[b] = (c0 + b < n_tiles) ? cnt[static_cast<size_t>(c0 + b) * nl + e] : 0;
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                if (c0 + b < n_tiles) cnt[static_cast<size_t>(c0 + b) * nl + e] = run;
                run += v[b];
            }
        }
        totals[e] = run;
    }
}

// Exclusive scan over the workgroup of per-thread values (kThreads threads);
// returns this thread's exclusive prefix and writes the grand total to *total.
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t v, int32_t* wave_sums, int32_t* total)
{
    const int lane = threadIdx.x & (tk::kWave - 1), wave = threadIdx.x / tk::kWave;
    int32_t inc = v;
#pragma unroll
    for (int off = 1; off < tk::kWave; off <<= 1) {
        const int32_t o = __shfl_up(inc, off);
        if (lane >= off) inc += o;
    }
    if (lane == tk::kWave - 1) wave_sums[wave] = inc;
    __syncthreads();
    int32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kThreads / tk::kWave; ++w) {
        const int32_t s = wave_sums[w];
        before += (w < wave) ? s : 0;
        all += s;
    }
    *total = all;
    return before + inc - v;
}

// row_src = -1 on the padding rows at the end of each expert's segment (they
// have no source token).  The n_tiles workgroups share the experts (tile,
// tile + n_tiles, ...); a workgroup's threads write one expert's run of
// padding rows together, so the stores are coalesced and no workgroup walks
// every segment.
__device__ __forceinline__ void write_padding(int32_t* __restrict__ row_src,
                                              const int32_t* pad_off, const int32_t* pad_cnt,
                                              int nl, int tile, int n_tiles)
{
    for (int ex = tile; ex < nl; ex += n_tiles) {
        const int32_t o = pad_off[ex], n = pad_cnt[ex];
        for (int i = threadIdx.x; i < n; i += kThreads) row_src[o + i] = -1;
    }
}

template <int KMAX>
__global__ __launch_bounds__(kThreads) void map_place_kernel(
    const int32_t* __restrict__ idx, int T, int k, int lo, int hi, int S, int n_tiles, int fused, int align, const int32_t* __restrict__ cnt, const int32_t* __restrict__ totals,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ pos,
    int32_t* __restrict__ row_src)
{
    extern __shared__ uint32_t lds[];
    __shared__ int32_t wave_sums[kThreads / tk::kWave];
    const int nl = hi - lo;
    uint32_t* mask = lds;                                          // [nl][S]
    uint32_t* before_sub = lds + nl * S;                           // [nl][S]
    int32_t* base = reinterpret_cast<int32_t*>(lds + 2 * nl * S);  // [nl]
    int32_t* pad_off = base + nl;                                  // [nl] first padding row
    int32_t* pad_cnt = pad_off + nl;                               // [nl] padding rows
    const int tile = blockIdx.x;
    const int tile_tokens = S * kSub;
    const int tl = threadIdx.x;
    const int t = tile * tile_tokens + tl;
    const bool mine = tl < tile_tokens && t < T;

    // 0. this thread's token: its stored expert ids.  Only the loads here:
    //    the count loads below go out before any of them is waited on.
    int raw[KMAX];
    if (mine) load_raw_ids<KMAX>(idx, t, k, raw);

    // 1. per expert: total over all tiles, sum over the tiles before this one
    //    (this thread owns the ept consecutive experts [e0, e0 + ept)).  A
    //    column is read kBatch tiles at a time, every load of a batch issued
    //    before the first is used (up to kBatch tiles is one round trip).
    const int ept = (nl + kThreads - 1) / kThreads;
    const int e0 = threadIdx.x * ept;
    int32_t my_total = 0;
    for (int i = 0; i < ept; ++i) {
        const int ex = e0 + i;
        if (ex >= nl) break;
        int32_t tot = 0, bef = 0;
        if (fused) {
            for (int c0 = 0; c0 < n_tiles; c0 += kBatch) {
                int32_t v[kBatch];
#pragma unroll
                for (int b = 0; b < kBatch; ++b)
                    v[b] = (c0 + b < n_tiles) ? cnt[static_cast<size_t>(c0 + b) * nl + ex] : 0;
#pragma unroll
                for (int b = 0; b < kBatch; ++b) {
                    tot += v[b];
                    bef += (c0 + b < tile) ? v[b] : 0;
                }
            }
        } else {
            tot = totals[ex];
            bef = cnt[static_cast<size_t>(tile) * nl + ex];
        }
        base[ex] = bef;
        my_total += (tot + align - 1) / align * align;   // the expert's segment, padded
        // keep the expert's total until the scan below has produced offsets
        before_sub[ex] = static_cast<uint32_t>(tot);
    }
    for (int i = threadIdx.x; i < nl * S; i += kThreads) mask[i] = 0;
    int e[KMAX];
    if (mine) local_ids<KMAX>(raw, k, lo, hi, e);
    __syncthreads();

    // 2. bit masks per (expert, sub-tile); offsets = exclusive scan of the
    //    padded segment lengths
    if (mine) {
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (e[j] >= 0) atomicOr(&mask[e[j] * S + tl / kSub], 1u << (tl % kSub));
    }
    int32_t grand = 0;
    int32_t run = block_exclusive_scan(my_total, wave_sums, &grand);   // syncs the block
    for (int i = 0; i < ept; ++i) {
        const int ex = e0 + i;
        if (ex >= nl) break;
        const int32_t tot = static_cast<int32_t>(before_sub[ex]);
        const int32_t padded = (tot + align - 1) / align * align;
        if (tile == 0) {
            counts[ex] = tot;
            offsets[ex] = run;
        }
        pad_off[ex] = run + tot;
        pad_cnt[ex] = padded - tot;
        base[ex] += run;
        run += padded;
    }
    if (tile == 0 && threadIdx.x == 0) offsets[nl] = grand;
    __syncthreads();
    if (row_src != nullptr && align > 1) write_padding(row_src, pad_off, pad_cnt, nl, tile, n_tiles);

    // 3. tokens of each expert in the earlier sub-tiles of this tile (the
    //    expert's S mask words are read into registers before any prefix is
    //    written: mask and before_sub share one LDS array)
    for (int ex = threadIdx.x; ex < nl; ex += kThreads) {
        uint32_t m[kMaxSub];
#pragma unroll
        for (int sb = 0; sb < kMaxSub; ++sb)   // clamped index: no branch per read
            m[sb] = mask[ex * S + (sb < S ? sb : S - 1)];
        uint32_t r = 0;
#pragma unroll
        for (int sb = 0; sb < kMaxSub; ++sb) {
            if (sb < S) before_sub[ex * S + sb] = r;
            r += __popc(m[sb]);
        }
    }
    __syncthreads();

    // 4. positions: every route's three LDS words are read before any is
    //    used (a masked route reads expert 0's words and discards them)
    if (!mine) return;
    const uint32_t below = (1u << (tl % kSub)) - 1u;
    const int sb = tl / kSub;
    int32_t bb[KMAX];
    uint32_t bs[KMAX], mk[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        if (j >= k) break;
        const int ee = e[j] >= 0 ? e[j] : 0;
        const int w = ee * S + sb;
        bb[j] = base[ee];
        bs[j] = before_sub[w];
        mk[j] = mask[w];
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        if (j >= k) break;
        int32_t p = -1;
        if (e[j] >= 0) {
            p = bb[j] + static_cast<int32_t>(bs[j] + __popc(mk[j] & below));
            if (row_src != nullptr) row_src[p] = t;
        }
        pos[static_cast<size_t>(t) * k + j] = p;
    }
}

// All tokens in one tile (T <= the tile size): one workgroup does the whole
// map in one launch.  Each expert's count is the popcount of its sub-tile
// masks, so no count matrix and no second launch are needed; the offsets
// scan and the positions are those of the place kernel.
template <int KMAX>
__global__ __launch_bounds__(kThreads) void map_single_kernel(
    const int32_t* __restrict__ idx, int T, int k, int lo, int hi, int S, int align,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ pos,
    int32_t* __restrict__ row_src)
{
    extern __shared__ uint32_t lds[];
    __shared__ int32_t wave_sums[kThreads / tk::kWave];
    const int nl = hi - lo;
    uint32_t* mask = lds;                                          // [nl][S]
    uint32_t* before_sub = lds + nl * S;                           // [nl][S]
    int32_t* base = reinterpret_cast<int32_t*>(lds + 2 * nl * S);  // [nl]
    int32_t* pad_off = base + nl;                                  // [nl] first padding row
    int32_t* pad_cnt = pad_off + nl;                               // [nl] padding rows
    const int t = threadIdx.x;
    const bool mine = t < S * kSub && t < T;

    int raw[KMAX];
    if (mine) load_raw_ids<KMAX>(idx, t, k, raw);
    for (int i = threadIdx.x; i < nl * S; i += kThreads) mask[i] = 0;
    int e[KMAX];
    if (mine) local_ids<KMAX>(raw, k, lo, hi, e);
    __syncthreads();
    if (mine) {
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (e[j] >= 0) atomicOr(&mask[e[j] * S + t / kSub], 1u << (t % kSub));
    }
    __syncthreads();

    // per expert (this thread owns [e0, e0 + ept), ept <= 4): sub-tile
    // prefixes and the count; offsets = exclusive scan of the padded counts
    constexpr int kMaxEpt = TK_MAX_EXPERTS / kThreads;
    const int ept = (nl + kThreads - 1) / kThreads;
    const int e0 = threadIdx.x * ept;
    int32_t tot[kMaxEpt];
    int32_t my_total = 0;
#pragma unroll
    for (int i = 0; i < kMaxEpt; ++i) {
        tot[i] = 0;
        const int ex = e0 + i;
        if (i >= ept || ex >= nl) continue;
        uint32_t m[kMaxSub];
#pragma unroll
        for (int sb = 0; sb < kMaxSub; ++sb) m[sb] = mask[ex * S + (sb < S ? sb : S - 1)];
        uint32_t r = 0;
#pragma unroll
        for (int sb = 0; sb < kMaxSub; ++sb) {
            if (sb >= S) break;
            before_sub[ex * S + sb] = r;
            r += __popc(m[sb]);
        }
        tot[i] = static_cast<int32_t>(r);
        my_total += (tot[i] + align - 1) / align * align;
    }
    int32_t grand = 0;
    int32_t run = block_exclusive_scan(my_total, wave_sums, &grand);   // syncs the block
#pragma unroll
    for (int i = 0; i < kMaxEpt; ++i) {
        const int ex = e0 + i;
        if (i >= ept || ex >= nl) continue;
        const int32_t padded = (tot[i] + align - 1) / align * align;
        counts[ex] = tot[i];
        offsets[ex] = run;
        pad_off[ex] = run + tot[i];
        pad_cnt[ex] = padded - tot[i];
        base[ex] = run;
        run += padded;
    }
    if (threadIdx.x == 0) offsets[nl] = grand;
    __syncthreads();
    if (row_src != nullptr && align > 1) write_padding(row_src, pad_off, pad_cnt, nl, 0, 1);

    if (!mine) return;
    const uint32_t below = (1u << (t % kSub)) - 1u;
    const int sb = t / kSub;
    int32_t bb[KMAX];
    uint32_t bs[KMAX], mk[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        if (j >= k) break;
        const int ee = e[j] >= 0 ? e[j] : 0;
        const int w = ee * S + sb;
        bb[j] = base[ee];
        bs[j] = before_sub[w];
        mk[j] = mask[w];
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        if (j >= k) break;
        int32_t p = -1;
        if (e[j] >= 0) {
            p = bb[j] + static_cast<int32_t>(bs[j] + __popc(mk[j] & below));
            if (row_src != nullptr) row_src[p] = t;
        }
        pos[static_cast<size_t>(t) * k + j] = p;
    }
}

// Zero counts and offsets when no token is given.
__global__ void map_empty_kernel(int nl, int32_t* __restrict__ counts, int32_t* __restrict__ offsets)
{
    for (int i = threadIdx.x; i <= nl; i += blockDim.x) {
        if (i < nl) counts[i] = 0;
        offsets[i] = 0;
    }
}

}  // namespace

TK_EXPORT size_t tk_map_workspace_bytes(int32_t T, int32_t k, int32_t n_local)
{
    (void)k;
    if (T <= 0 || n_local <= 0) return 0;
    const Tiling g = tiling(T, n_local);
    // cnt[n_tiles][n_local] + totals[n_local]
    return (static_cast<size_t>(g.n_tiles) * n_local + static_cast<size_t>(n_local)) * sizeof(int32_t);
}

namespace {

// Host-side argument checks shared by every map entry point (all but the
// workspace's); TK_OK or the failure status.
tk_status map_check(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E, int32_t local_begin,
                    int32_t local_end, int32_t align, const int32_t* counts,
                    const int32_t* offsets, const int32_t* pos, const int32_t* row_src)
{
    using tk::fail;
    if (align < 1) return fail(TK_ERR_ARG, "tk_map: align=%d < 1", align);
    if (T < 0) return fail(TK_ERR_ARG, "tk_map: T=%d < 0", T);
    if (k < 1) return fail(TK_ERR_ARG, "tk_map: k=%d < 1", k);
    if (k > TK_MAX_TOPK) return fail(TK_ERR_UNSUPPORTED, "tk_map: k=%d > %d", k, TK_MAX_TOPK);
    if (E < 1 || E > TK_MAX_EXPERTS)
        return fail(E < 1 ? TK_ERR_ARG : TK_ERR_UNSUPPORTED, "tk_map: E=%d not in [1, %d]", E,
                    TK_MAX_EXPERTS);
    if (local_begin < 0 || local_end > E || local_begin >= local_end)
        return fail(TK_ERR_ARG, "tk_map: local range [%d, %d) not a non-empty part of [0, %d)",
                    local_begin, local_end, E);
    if (static_cast<int64_t>(T) * k +
            static_cast<int64_t>(local_end - local_begin) * (align - 1) > INT32_MAX)
        return fail(TK_ERR_ARG, "tk_map: T*k plus padding exceeds int32 positions");
    if (counts == nullptr || offsets == nullptr)
        return fail(TK_ERR_ARG, "tk_map: NULL counts/offsets");
    if (T > 0 && (topk_idx == nullptr || pos == nullptr))
        return fail(TK_ERR_ARG, "tk_map: NULL topk_idx/pos");
    if (!tk::aligned4(counts) || !tk::aligned4(offsets) || (pos && !tk::aligned4(pos)) ||
        (row_src && !tk::aligned4(row_src)) || (topk_idx && !tk::aligned4(topk_idx)))
        return fail(TK_ERR_ARG, "tk_map: int32 tensors must be 4-byte aligned");
    return TK_OK;
}

}  // namespace

TK_EXPORT tk_status tk_map_aligned(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                                   int32_t local_begin, int32_t local_end, int32_t align,
                                   int32_t* counts, int32_t* offsets, int32_t* pos,
                                   int32_t* row_src, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream)
{
    using tk::fail;
    const tk_status st = map_check(topk_idx, T, k, E, local_begin, local_end, align, counts,
                                   offsets, pos, row_src);
    if (st != TK_OK) return st;
    const int nl = local_end - local_begin;
    const size_t need = tk_map_workspace_bytes(T, k, nl);
    if (workspace_bytes < need)
        return fail(TK_ERR_ARG, "tk_map: workspace of %zu bytes < %zu needed", workspace_bytes, need);
    if (need > 0 && (workspace == nullptr || !tk::aligned16(workspace)))
        return fail(TK_ERR_ARG, "tk_map: workspace NULL or not 16-byte aligned");

    hipError_t e;
    if (T == 0) {
        e = tk::launch(map_empty_kernel, dim3(1), dim3(kThreads), 0, stream, nl, counts, offsets);
        return tk::launched(e, "tk_map (empty)");
    }
    const Tiling g = tiling(T, nl);
    int32_t* cnt = static_cast<int32_t*>(workspace);
    int32_t* totals = cnt + static_cast<size_t>(g.n_tiles) * nl;
    const dim3 grid(g.n_tiles), block(kThreads);
    const bool small_k = k <= 8;
    const size_t lds = (2 * static_cast<size_t>(nl) * g.S + 3 * nl) * sizeof(uint32_t);
    if (g.n_tiles == 1) {
        e = small_k
            ? tk::launch(map_single_kernel<8>, grid, block, lds, stream, topk_idx, T, k,
                         local_begin, local_end, g.S, align, counts, offsets, pos, row_src)
            : tk::launch(map_single_kernel<TK_MAX_TOPK>, grid, block, lds, stream, topk_idx, T, k,
                         local_begin, local_end, g.S, align, counts, offsets, pos, row_src);
        return tk::launched(e, "tk_map (single tile)");
    }
    e = small_k
        ? tk::launch(map_count_kernel<8>, grid, block, nl * sizeof(int32_t), stream, topk_idx, T, k,
                     local_begin, local_end, g.tile, cnt)
        : tk::launch(map_count_kernel<TK_MAX_TOPK>, grid, block, nl * sizeof(int32_t), stream,
                     topk_idx, T, k, local_begin, local_end, g.tile, cnt);
    if (e != hipSuccess) return tk::launched(e, "tk_map (count)");
    if (!g.fused) {
        e = tk::launch(map_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, cnt, g.n_tiles, nl,
                       totals);
        if (e != hipSuccess) return tk::launched(e, "tk_map (scan)");
    }
    e = small_k
        ? tk::launch(map_place_kernel<8>, grid, block, lds, stream, topk_idx, T, k, local_begin,
                     local_end, g.S, g.n_tiles, g.fused ? 1 : 0, align, cnt, totals,
                     counts, offsets, pos, row_src)
        : tk::launch(map_place_kernel<TK_MAX_TOPK>, grid, block, lds, stream, topk_idx, T, k,
                     local_begin, local_end, g.S, g.n_tiles, g.fused ? 1 : 0, align, cnt,
                     totals, counts, offsets, pos, row_src);
    return tk::launched(e, "tk_map (place)");
}

TK_EXPORT tk_status tk_map(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                           int32_t local_begin, int32_t local_end, int32_t* counts,
                           int32_t* offsets, int32_t* pos, int32_t* row_src, void* workspace,
                           size_t workspace_bytes, hipStream_t stream)
{
    return tk_map_aligned(topk_idx, T, k, E, local_begin, local_end, 1, counts, offsets, pos,
                          row_src, workspace, workspace_bytes, stream);
}

// ------------------------------------------------------------ no allocation
// tk_map_noalloc: tk_map with its count matrix in a fixed device array
// instead of a caller-provided workspace.  Each GPU the library runs on holds
// its own copy of the array (TK_MAP_NOALLOC_SCRATCH_BYTES) until the process
// ends.  In host code `scratch` names a host-side stand-in, not the device
// array, so kernels receive the address hipGetSymbolAddress returns, looked
// up once per device with that device current.  The map overwrites every
// count it later reads, so nothing in the array needs clearing between calls.
static __device__ __align__(256) int32_t scratch[TK_MAP_NOALLOC_SCRATCH_BYTES / sizeof(int32_t)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's device address on device `dev` (the current device),
// looked up on the first call there; or an error status.
tk_status scratch_on_device(int dev, void** out)
{
    if (dev < 0 || dev >= kMaxDevices)
        return tk::fail(TK_ERR_UNSUPPORTED, "tk_map_noalloc: device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return tk::fail(TK_ERR_DEVICE, "tk_map_noalloc: hipGetSymbolAddress: %s",
                            hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return TK_OK;
}

}  // namespace

TK_EXPORT tk_status tk_map_noalloc(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                                   int32_t local_begin, int32_t local_end, int32_t* counts,
                                   int32_t* offsets, int32_t* pos, int32_t* row_src,
                                   hipStream_t stream)
{
    using tk::fail;
    tk_status st = map_check(topk_idx, T, k, E, local_begin, local_end, 1, counts, offsets, pos,
                             row_src);
    if (st != TK_OK) return st;
    const size_t need = tk_map_workspace_bytes(T, k, local_end - local_begin);
    if (need > TK_MAP_NOALLOC_SCRATCH_BYTES)
        return fail(TK_ERR_ARG,
                    "tk_map_noalloc: T=%d with %d local experts needs %zu bytes of scratch, more "
                    "than the %d the library holds; use tk_map with a workspace",
                    T, local_end - local_begin, need, TK_MAP_NOALLOC_SCRATCH_BYTES);
    int dev = -1, stream_dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipStreamGetDevice(stream, &stream_dev);
    if (e != hipSuccess)
        return fail(TK_ERR_DEVICE, "tk_map_noalloc: device query: %s", hipGetErrorString(e));
    if (stream_dev != dev)
        return fail(TK_ERR_ARG, "tk_map_noalloc: stream is on device %d, current device is %d",
                    stream_dev, dev);
    void* ws = nullptr;
    st = scratch_on_device(dev, &ws);
    if (st != TK_OK) return st;
    return tk_map_aligned(topk_idx, T, k, E, local_begin, local_end, 1, counts, offsets, pos,
                          row_src, ws, TK_MAP_NOALLOC_SCRATCH_BYTES, stream);
}
