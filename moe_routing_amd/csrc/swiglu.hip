// tk_swiglu_quant: SwiGLU activation fused with per-token 1x128 FP8 E4M3
// quantisation, optionally applying each expanded row's routing weight --
// the SwiGLU and FP8 quantisation fusion of TileKernels' quant/ module
// ("刚刚！DeepSeek开源高性能GPU算子库TileKernels", item quant/: SwiGLU activation,
// FP8 quantisation and transpose done in one pass instead of three HBM round
// trips; "剛剛，DeepSeek開始頻繁更新：Tile Kernels、DeepEP V2", feature list), and
// the SwiGLU-with-weight-to-FP8 helper the DeepGEMM section of "DeepSeek 的
// GPU 内核帝国…" lists (section 第二层：DeepGEMM, kernel list).
//
// Row r of h holds 2*I bf16 values, gate g = h[r, 0..I) and up u = h[r, I..2I).
// In fp32, one IEEE operation per step:
//   s = 1/(1 + E(-g))   (the pinned sigmoid shared with tk_route)
//   a = RN(RN(g*s)*u);  weighted: a = RN(a*w_r)
// then the 1x128 block codec of tk_expand_quant: amax = max(max |a|, 1e-4),
// scale = RN(amax/448), q = E4M3(RN(a/scale)).
//
// The sigmoid is not evaluated per element: g is bf16, so s = sigmoid(g) is
// one of a few thousand distinct fp32 values (outside a band of magnitudes it
// is exactly 1/2, 1 or 0).  The build tabulates the pinned sigmoid over that
// band (31 KB, sigmoid_table.h); every workgroup copies the table into LDS
// once and reads s with one LDS load after a clamp and an index -- about
// eight instructions where exp and an IEEE division took about thirty.  The
// values are the pinned sigmoid's, bit for bit.
//
// One wave per row, in chunks of 1024 output columns.  The grid is persistent
// (at most kSBlocks workgroups of 8 waves, so the table is copied about a
// thousand times, not once per row); each wave strides over the rows.  In a
// chunk each lane owns 16 consecutive output columns: two 16-byte loads of
// gate and two of up, one 16-byte store of codes, and lane 0 of each 8-lane
// group (one 128-column block) stores the block's scale.  Inputs and outputs
// are touched once: streaming loads and stores.  With the sigmoid a lookup,
// the kernel streams at about the rate of a device copy.
//
// The weight of row r is found from the map's outputs: t = row_src[r] and the
// slot j with pos[t, j] == r give w_r = topk_w[t, j]; a row no slot points at
// gets weight 0.  These are two dependent loads, so they are issued one or
// two rows ahead of the row that needs them.
//
// tk_swiglu_quant_t adds the transpose of the fusion: the same activations
// also quantised as a^T (I, rows) in 1x128 blocks along its rows (128 tokens
// of one channel, the layout a weight-gradient GEMM reads), both outputs from
// one pass over h.
#include <algorithm>

#include "sigmoid_table.h"
#include "tk_internal.h"

namespace {

constexpr int kChunk = 1024;   // output columns per unit (16 per lane)

// sigmoid of the bf16 values in the table's band, interleaved by sign; the
// entries are written at build time by sigmoid_table_gen (same pinned steps)
__device__ __align__(16) const float kSigmoidBf16[tk::kSigEntries] = {
#include "sigmoid_table.inc"
};
static_assert(tk::kSigEntries % 4 == 0, "the table is copied in 16-byte pieces");

// All THREADS threads of the workgroup copy the table into LDS (the caller
// places the barrier).
template <int THREADS>
__device__ __forceinline__ void load_sigmoid_table(float* lds)
{
    const auto* src = reinterpret_cast<const tk::u32x4*>(kSigmoidBf16);
    auto* dst = reinterpret_cast<tk::u32x4*>(lds);
    for (int i = threadIdx.x; i < static_cast<int>(tk::kSigEntries / 4); i += THREADS) dst[i] = src[i];
}

// sigmoid(g) for the bf16 g with magnitude bits m (15 bits) and sign bit sgn,
// read from the LDS table; silu = RN(g * sigmoid(g)).
__device__ __forceinline__ float sigmoid_bf16(uint32_t m, uint32_t sgn, const float* tab)
{
    const uint32_t c = m < tk::kSigLo - 1 ? tk::kSigLo - 1 : (m > tk::kSigHi ? tk::kSigHi : m);
    return tab[((c - (tk::kSigLo - 1)) << 1) | sgn];
}
__device__ __forceinline__ float sigmoid_lo(uint32_t w, const float* tab)
{
    return sigmoid_bf16(w & 0x7FFFu, (w >> 15) & 1u, tab);
}
__device__ __forceinline__ float sigmoid_hi(uint32_t w, const float* tab)
{
    return sigmoid_bf16((w >> 16) & 0x7FFFu, w >> 31, tab);
}
__device__ __forceinline__ float silu_lo(uint32_t w, const float* tab) { return tk::bf16_lo(w) * sigmoid_lo(w, tab); }
__device__ __forceinline__ float silu_hi(uint32_t w, const float* tab) { return tk::bf16_hi(w) * sigmoid_hi(w, tab); }

struct SwigluArgs {
    const uint16_t* h;
    int64_t cap;
    const int32_t* n_rows;
    int I;
    const int32_t* row_src;
    const int32_t* pos;
    const float* topk_w;
    int T, k;
    uint8_t* out;
    float* scales;
};

// The weight of expanded row r: its token t = row_src[r], and the slot j of t
// with pos[t, j] == r carries it (0 when t is out of range or no slot points
// at r, e.g. a padding row).  Lane j < k holds slot j: one load of pos and one
// of topk_w per lane, then a ballot picks the slot (a token's slots point at
// distinct rows, so at most one lane matches).
__device__ __forceinline__ float select_weight(int32_t p, float w, uint32_t r)
{
    const uint64_t hit = __ballot(p == static_cast<int32_t>(r));
    if (hit == 0) return 0.0f;
    const int j = tk::uniform(__ffsll(static_cast<long long>(hit)) - 1);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j));
}
__device__ __forceinline__ float pick_weight(const SwigluArgs& a, int t, int lane, uint32_t r)
{
    int32_t p = -1;
    float w = 0.0f;
    if (t >= 0 && t < a.T && lane < a.k) {
        p = a.pos[static_cast<size_t>(t) * a.k + lane];
        w = a.topk_w[static_cast<size_t>(t) * a.k + lane];
    }
    return select_weight(p, w, r);
}

constexpr int kSThreads = 512;                 // 8 waves per workgroup
constexpr int kSWaves = kSThreads / tk::kWave;
constexpr int kSBlocks = 1024;                 // 4 per CU of a 256-CU device
constexpr int kSStageScales = 64;              // scales per row gathered in LDS (I <= 8192)

template <bool WEIGHTED>
__global__ __launch_bounds__(kSThreads) void swiglu_quant_kernel(SwigluArgs a)
{
    __shared__ __align__(16) float sig[tk::kSigEntries];
    load_sigmoid_table<kSThreads>(sig);
    __syncthreads();

    const int lane = threadIdx.x & (tk::kWave - 1);
    int64_t rows64 = a.cap;
    if (a.n_rows != nullptr) {
        const int64_t n = *a.n_rows;
        rows64 = n < 0 ? 0 : (n < a.cap ? n : a.cap);
    }
    // the host bounds rows_capacity below 2^31 / 8: 32-bit row indices, and
    // r + 2 * stride does not wrap
    const uint32_t rows = static_cast<uint32_t>(rows64);
    const uint32_t stride = gridDim.x * kSWaves;
    const int wave = tk::uniform(threadIdx.x / tk::kWave);
    uint32_t r = blockIdx.x * kSWaves + wave;
    // A workgroup's waves take 8 adjacent rows per iteration, so their scales
    // (I/128 per row; 64 bytes at I = 2048) share cache lines: when a row has
    // at most kSStageScales of them they are gathered in LDS and leave as
    // whole lines after the iteration, instead of as 32-byte pieces from
    // different waves (1-1.5 us of about 127).
    __shared__ float sc_stage[kSWaves * kSStageScales];
    const int nbr = a.I / 128;
    const bool stage_sc = nbr <= kSStageScales;

    // Routing weights run ahead of the rows: while row r is processed, the
    // token of row r + 2*stride and the slots of row r + stride's token are
    // in flight, so their dependent loads never wait in line.
    float w = 1.0f;
    int t1 = -1;
    if constexpr (WEIGHTED) {
        const int t0 = r < rows ? a.row_src[r] : -1;
        w = pick_weight(a, t0, lane, r);
        t1 = r + stride < rows ? a.row_src[r + stride] : -1;
    }
    // the loop runs while the workgroup's first row is in range (uniform, as
    // the barriers need); a wave past the last row only takes the barriers
    for (uint32_t base = blockIdx.x * kSWaves; base < rows; base += stride, r += stride) {
        const bool live = r < rows;
        int t2 = -1;
        int32_t p1 = -1;
        float w1 = 0.0f;
        if constexpr (WEIGHTED) {
            if (r + 2 * stride < rows) t2 = a.row_src[r + 2 * stride];
            if (t1 >= 0 && t1 < a.T && lane < a.k) {
                p1 = a.pos[static_cast<size_t>(t1) * a.k + lane];
                w1 = a.topk_w[static_cast<size_t>(t1) * a.k + lane];
            }
        }
        const uint16_t* hr = a.h + static_cast<size_t>(r) * 2 * a.I;
        uint8_t* orow = a.out + static_cast<size_t>(r) * a.I;
        float* srow = a.scales + static_cast<size_t>(r) * (a.I / 128);
        for (int col0 = 0; live && col0 < a.I; col0 += kChunk) {
            const int col = col0 + lane * 16;
            const bool active = col < a.I;   // I % 128 == 0: 8-lane groups are wholly in or out
            tk::u32x4 g0 = tk::u32x4{0u, 0u, 0u, 0u}, g1 = g0, u0 = g0, u1 = g0;
            if (active) {
                g0 = tk::load_stream(hr + col);
                g1 = tk::load_stream(hr + col + 8);
                u0 = tk::load_stream(hr + a.I + col);
                u1 = tk::load_stream(hr + a.I + col + 8);
            }
            const uint32_t gw[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
            const uint32_t uw[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
            float v[16];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float va = silu_lo(gw[i], sig) * tk::bf16_lo(uw[i]);
                float vb = silu_hi(gw[i], sig) * tk::bf16_hi(uw[i]);
                if constexpr (WEIGHTED) {
                    va = va * w;
                    vb = vb * w;
                }
                v[2 * i] = va;
                v[2 * i + 1] = vb;
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
                tk::store_stream(orow + col, q);
                if ((lane & 7) == 0) {
                    if (stage_sc) sc_stage[wave * kSStageScales + col / 128] = scale;
                    else srow[col / 128] = scale;
                }
            }
        }
        if (stage_sc) {
            __syncthreads();   // the iteration's rows' scales staged
            const uint32_t nr = rows - base < kSWaves ? rows - base : kSWaves;
            for (int i = threadIdx.x; i < static_cast<int>(nr) * nbr; i += kSThreads) {
                const int rr = i / nbr;
                a.scales[static_cast<size_t>(base) * nbr + i] = sc_stage[rr * kSStageScales + i - rr * nbr];
            }
            __syncthreads();   // read out before the next iteration stages
        }
        if constexpr (WEIGHTED) {
            w = select_weight(p1, w1, r + stride);
            t1 = t2;
        }
    }
}

// RN(g * sigmoid(g)) elementwise for n bf16 values (the SwiGLU gate factor).
__global__ __launch_bounds__(tk::kBlock) void silu_kernel(const uint16_t* __restrict__ g, int64_t n,
                                                          float* __restrict__ out)
{
    __shared__ __align__(16) float sig[tk::kSigEntries];
    load_sigmoid_table<tk::kBlock>(sig);
    __syncthreads();
    const int64_t stride = static_cast<int64_t>(gridDim.x) * tk::kBlock;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * tk::kBlock + threadIdx.x; i < n; i += stride)
        out[i] = silu_lo(g[i], sig);
}

// ---------------------------------------------------------------- transposed
// One workgroup of 512 threads per tile of 128 rows x 128 output columns
// computes the tile's activations once and writes them twice: row-major codes
// with 1x128 blocks along each row (the tile's 128 columns), and the
// transpose a^T with 1x128 blocks along each of its rows (the tile's 128 rows
// of one column).  Thread (rg, cg) = (tid / 16, tid % 16) holds rows 4*rg..
// and columns 8*cg.. of the tile (32 values): a row's 128 columns live in 16
// consecutive lanes (DPP row max), a column's 128 rows in 32 row groups across
// the eight waves (LDS max).  The transposed codes are staged in LDS and leave
// as whole 16-byte pieces of out_t's rows.  The LDS layouts keep the lanes of
// one instruction on different banks: a staged row's 16-byte slots are
// rotated per column group, the column scales are stored transposed and the
// column partial maxima padded (each of these was a 4- to 16-way bank
// conflict, about 3 % of the time).  The grid is persistent (at most kTBlocks
// workgroups, each striding over the tiles), so the sigmoid table is copied
// once per workgroup.
constexpr int kTile = 128;
constexpr int kTThreads = 512;
constexpr int kTRows = 4;                         // rows per thread
constexpr int kTGroups = kTile / kTRows;          // 32 row groups
constexpr int kTPitch = kTile + 16;               // bytes per staged out_t row (padded)
static_assert(kTRows == 4, "a row group's rows are handed out by quad broadcasts");
// Tile t = (row tile) * tiles_c + (column tile): the column tiles of one row
// tile are consecutive, so workgroups running side by side read whole rows of
// h.  A workgroup's tiles are t, t + G, t + 2G, ... (G workgroups); the step
// moves (row tile, column tile) by (G / tiles_c, G % tiles_c) with a carry,
// so the loop divides nothing (a 64-bit division is over a hundred scalar
// instructions).
struct TileCursor {
    int64_t tr;
    int tc;
    __device__ __forceinline__ void advance(int64_t step_r, int step_c, int tiles_c)
    {
        tr += step_r;
        tc += step_c;
        if (tc >= tiles_c) {
            tc -= tiles_c;
            ++tr;
        }
    }
};

// lane i of each lane quad, to all four lanes (DPP quad_perm [i,i,i,i]); i is
// a compile-time constant after unrolling
__device__ __forceinline__ float quad_lane(float x, int i)
{
    switch (i) {
    case 0: return tk::dpp_f32<0x00>(x);
    case 1: return tk::dpp_f32<0x55>(x);
    case 2: return tk::dpp_f32<0xAA>(x);
    default: return tk::dpp_f32<0xFF>(x);
    }
}

constexpr int kTBlocks = 512;                     // 2 per CU of a 256-CU device

// (5 waves per SIMD, two workgroups per CU: the weighted form needs about 94
// VGPRs.  Held to the 80 that six waves allow -- three workgroups per CU,
// the LDS limit -- it spilled loop values to scratch and ran slower.)
template <bool WEIGHTED>
__global__ __launch_bounds__(kTThreads) __attribute__((amdgpu_waves_per_eu(5)))
void swiglu_quant_t_kernel(SwigluArgs a, int64_t tiles, uint8_t* __restrict__ out_t,
                           float* __restrict__ scales_t)
{
    __shared__ __align__(16) float sig[tk::kSigEntries];
    __shared__ float w_row[kTile];
    __shared__ float col_scale[kTile];
    __shared__ float col_inv[kTile];
    // the column partial maxima, then (once they are reduced) the staged codes
    __shared__ __align__(16) uint8_t stage[kTile * kTPitch];
    static_assert(sizeof(float) * kTGroups * kTile <= kTile * kTPitch, "stage too small");
    constexpr int kPartPitch = kTile + 4;   // padded: the row groups' writes fall on different banks
    static_assert(sizeof(float) * kTGroups * kPartPitch <= kTile * kTPitch, "stage too small");
    auto col_part = reinterpret_cast<float (*)[kPartPitch]>(stage);
    load_sigmoid_table<kTThreads>(sig);

    const int tiles_c = a.I / kTile;
    const int rg = threadIdx.x >> 4, cg = threadIdx.x & 15;
    const int64_t R = a.cap;

    // Routing weights run one tile ahead.  Four threads share a tile row
    // (wrow = tid / 4): thread wsub loads slots wsub and wsub + 4 of the row's
    // token once the previous tile's codes are staged, and picks the weight
    // after that tile's stores; slots from 8 on (k > 8) are read when the weight is picked.  The
    // matching slot's weight bits are OR-ed across the quad (a token's slots
    // point at distinct rows, so at most one thread matches; none leaves +0).
    const int wrow = threadIdx.x >> 2, wsub = threadIdx.x & 3;
    int32_t pa = -1, pb = -1;
    float wa = 0.0f, wb = 0.0f;
    auto load_slots = [&](int t) {
        pa = pb = -1;
        if (t >= 0 && t < a.T) {
            const size_t base = static_cast<size_t>(t) * a.k;
            if (wsub < a.k) {
                pa = a.pos[base + wsub];
                wa = a.topk_w[base + wsub];
            }
            if (wsub + 4 < a.k) {
                pb = a.pos[base + wsub + 4];
                wb = a.topk_w[base + wsub + 4];
            }
        }
    };
    auto pick_weight = [&](int t, int64_t row) {
        const int32_t r = static_cast<int32_t>(row);
        uint32_t bits = 0;
        if (pa == r) bits = __float_as_uint(wa);
        if (pb == r) bits = __float_as_uint(wb);
        if (t >= 0 && t < a.T) {
            for (int j = wsub + 8; j < a.k; j += 4) {
                const size_t sl = static_cast<size_t>(t) * a.k + j;
                if (a.pos[sl] == r) bits = __float_as_uint(a.topk_w[sl]);
            }
        }
        bits |= tk::dpp_u32<tk::kQuadXor1>(bits);
        bits |= tk::dpp_u32<tk::kQuadXor2>(bits);
        if (wsub == 0) w_row[wrow] = __uint_as_float(bits);
    };
    const int64_t step_r = gridDim.x / tiles_c;
    const int step_c = static_cast<int>(gridDim.x % tiles_c);
    TileCursor cur{blockIdx.x / tiles_c, static_cast<int>(blockIdx.x % tiles_c)};
    if constexpr (WEIGHTED) {
        if (blockIdx.x < tiles) {
            const int64_t row = cur.tr * kTile + wrow;
            const int t = a.row_src[row];
            load_slots(t);
            pick_weight(t, row);
        }
    }
    __syncthreads();   // the table and the first tile's weights

    for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        const int64_t tr = cur.tr;
        const int tc = cur.tc;
        const int64_t r0 = tr * kTile;
        const int c0 = tc * kTile;
        const int64_t next = tile + gridDim.x;
        cur.advance(step_r, step_c, tiles_c);   // the next tile's coordinates
        const int64_t next_row = cur.tr * kTile + wrow;

        tk::u32x4 gw[kTRows], uw[kTRows];
#pragma unroll
        for (int i = 0; i < kTRows; ++i) {
            const uint16_t* hr = a.h + static_cast<size_t>(r0 + rg * kTRows + i) * 2 * a.I;
            gw[i] = tk::load_stream(hr + c0 + cg * 8);
            uw[i] = tk::load_stream(hr + a.I + c0 + cg * 8);
        }
        int tok_next = -1;
        if constexpr (WEIGHTED) {
            if (next < tiles) tok_next = a.row_src[next_row];
        }

        float v[kTRows][8];
#pragma unroll
        for (int i = 0; i < kTRows; ++i) {
            const uint32_t g4[4] = {gw[i].x, gw[i].y, gw[i].z, gw[i].w};
            const uint32_t u4[4] = {uw[i].x, uw[i].y, uw[i].z, uw[i].w};
            // the row's eight table reads go out together, then the arithmetic
            float sg[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sg[2 * j] = sigmoid_lo(g4[j], sig);
                sg[2 * j + 1] = sigmoid_hi(g4[j], sig);
            }
            const float w = WEIGHTED ? w_row[rg * kTRows + i] : 1.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float va = (tk::bf16_lo(g4[j]) * sg[2 * j]) * tk::bf16_lo(u4[j]);
                float vb = (tk::bf16_hi(g4[j]) * sg[2 * j + 1]) * tk::bf16_hi(u4[j]);
                if constexpr (WEIGHTED) {
                    va = va * w;
                    vb = vb * w;
                }
                v[i][2 * j] = va;
                v[i][2 * j + 1] = vb;
            }
        }

        // column partial maxima first (the LDS round trip overlaps the row codes)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float m = 0.f;
#pragma unroll
            for (int i = 0; i < kTRows; ++i) m = fmaxf(m, fabsf(v[i][j]));
            col_part[rg][cg * 8 + j] = m;
        }

        // row-major codes: one 1x128 block per tile row.  The row maxima are
        // 16-lane DPP maxima; then lane cg forms the scale and reciprocal of
        // row cg & 3 only, and a quad broadcast hands row i's pair to every
        // lane: one pair of IEEE divisions per lane instead of four.
        float rm[kTRows];
#pragma unroll
        for (int i = 0; i < kTRows; ++i) {
            float m = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[i][j]));
            m = fmaxf(m, tk::dpp_f32<tk::kQuadXor1>(m));
            m = fmaxf(m, tk::dpp_f32<tk::kQuadXor2>(m));
            m = fmaxf(m, tk::dpp_f32<tk::kHalfMirror>(m));
            rm[i] = fmaxf(m, tk::dpp_f32<tk::kMirror>(m));   // the 16 lanes of this row group
        }
        const int mine = cg & 3;
        const float m_mine = mine == 0 ? rm[0] : (mine == 1 ? rm[1] : (mine == 2 ? rm[2] : rm[3]));
        const float s_mine = fmaxf(m_mine, 1e-4f) / 448.0f;
        const float inv_mine = 1.0f / s_mine;
#pragma unroll
        for (int i = 0; i < kTRows; ++i) {
            const float scale = quad_lane(s_mine, i), inv = quad_lane(inv_mine, i);
            uint2 o;
            o.x = tk::pack_fp8x4(tk::fp8_quotient(v[i][0], scale, inv), tk::fp8_quotient(v[i][1], scale, inv),
                                 tk::fp8_quotient(v[i][2], scale, inv), tk::fp8_quotient(v[i][3], scale, inv));
            o.y = tk::pack_fp8x4(tk::fp8_quotient(v[i][4], scale, inv), tk::fp8_quotient(v[i][5], scale, inv),
                                 tk::fp8_quotient(v[i][6], scale, inv), tk::fp8_quotient(v[i][7], scale, inv));
            const int64_t r = r0 + rg * kTRows + i;
            *reinterpret_cast<uint2*>(a.out + static_cast<size_t>(r) * a.I + c0 + cg * 8) = o;
            if (cg == 0) a.scales[static_cast<size_t>(r) * (a.I / 128) + tc] = scale;
        }

        // transposed codes: one 1x128 block per tile column
        __syncthreads();   // col_part complete; w_row read out
        if (threadIdx.x < kTile) {
            float m = col_part[0][threadIdx.x];
#pragma unroll
            for (int g = 1; g < kTGroups; ++g) m = fmaxf(m, col_part[g][threadIdx.x]);
            const float scale = fmaxf(m, 1e-4f) / 448.0f;
            // stored transposed (column c at (c % 8) * 16 + c / 8): a thread's eight columns
            // cg*8 .. cg*8+7 are then read at j*16 + cg, sixteen distinct banks per read
            const int ti = (threadIdx.x & 7) * 16 + (threadIdx.x >> 3);
            col_scale[ti] = scale;
            col_inv[ti] = 1.0f / scale;
            scales_t[static_cast<size_t>(c0 + threadIdx.x) * (R / kTile) + tr] = scale;
        }
        __syncthreads();   // col_scale ready, col_part consumed: stage now holds codes
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float scale = col_scale[j * 16 + cg], inv = col_inv[j * 16 + cg];
            const uint32_t q = tk::pack_fp8x4(tk::fp8_quotient(v[0][j], scale, inv),
                                              tk::fp8_quotient(v[1][j], scale, inv),
                                              tk::fp8_quotient(v[2][j], scale, inv),
                                              tk::fp8_quotient(v[3][j], scale, inv));
            // 16-byte slot (rg / 4) of the column's staged row, rotated by cg & 7 so that the
            // lanes of one store instruction spread over the LDS banks
            const int slot = (rg >> 2) ^ (cg & 7);
            *reinterpret_cast<uint32_t*>(stage + (cg * 8 + j) * kTPitch + slot * 16 + (rg & 3) * 4) = q;
        }
        if constexpr (WEIGHTED) load_slots(tok_next);   // the next tile's slots
        __syncthreads();
        // 128 out_t rows of 128 bytes: 8 threads per row, 16 bytes each
        for (int i = threadIdx.x; i < kTile * 8; i += kTThreads) {
            const int c = i >> 3, part = i & 7;
            const int slot = part ^ ((c >> 3) & 7);
            const tk::u32x4 q = *reinterpret_cast<const tk::u32x4*>(stage + c * kTPitch + slot * 16);
            tk::store_stream(out_t + static_cast<size_t>(c0 + c) * R + r0 + part * 16, q);
        }
        if constexpr (WEIGHTED) {
            if (next < tiles) pick_weight(tok_next, next_row);
        }
        __syncthreads();   // stage read out before the next tile; its weights published
    }
}

}  // namespace

TK_EXPORT tk_status tk_swiglu_quant(const void* h_bf16, int64_t rows_capacity,
                                    const int32_t* n_rows, int32_t I, const int32_t* row_src,
                                    const int32_t* pos, const float* topk_w, int32_t T, int32_t k,
                                    void* out, float* scales, hipStream_t stream)
{
    using tk::fail;
    if (rows_capacity < 0) return fail(TK_ERR_ARG, "tk_swiglu_quant: rows_capacity < 0");
    if (I < 128 || I % 128 != 0)
        return fail(TK_ERR_ARG, "tk_swiglu_quant: I=%d must be a positive multiple of 128", I);
    const int n_weight_args = (row_src != nullptr) + (pos != nullptr) + (topk_w != nullptr);
    if (n_weight_args != 0 && n_weight_args != 3)
        return fail(TK_ERR_ARG, "tk_swiglu_quant: row_src, pos and topk_w go together");
    const bool weighted = n_weight_args == 3;
    if (weighted && (T < 0 || k < 1 || k > TK_MAX_TOPK))
        return fail(TK_ERR_ARG, "tk_swiglu_quant: T=%d, k=%d invalid for the weights", T, k);
    if (rows_capacity == 0) return tk::ok();
    if (h_bf16 == nullptr || out == nullptr || scales == nullptr)
        return fail(TK_ERR_ARG, "tk_swiglu_quant: NULL tensor pointer");
    if (!tk::aligned16(h_bf16) || !tk::aligned16(out) || !tk::aligned4(scales) ||
        (n_rows && !tk::aligned4(n_rows)) || (row_src && !tk::aligned4(row_src)) ||
        (pos && !tk::aligned4(pos)) || (topk_w && !tk::aligned4(topk_w)))
        return fail(TK_ERR_ARG, "tk_swiglu_quant: h/out must be 16-byte aligned, the rest 4-byte");
    if (rows_capacity > INT32_MAX / 8) return fail(TK_ERR_UNSUPPORTED, "tk_swiglu_quant: too many rows");
    const int64_t blocks = std::min<int64_t>((rows_capacity + kSWaves - 1) / kSWaves, kSBlocks);
    const SwigluArgs args{static_cast<const uint16_t*>(h_bf16), rows_capacity, n_rows, I,
                          row_src, pos, topk_w, T, k, static_cast<uint8_t*>(out), scales};
    const dim3 grid(static_cast<unsigned>(blocks)), block(kSThreads);
    const hipError_t e = weighted
        ? tk::launch(swiglu_quant_kernel<true>, grid, block, 0, stream, args)
        : tk::launch(swiglu_quant_kernel<false>, grid, block, 0, stream, args);
    return tk::launched(e, "tk_swiglu_quant");
}

TK_EXPORT tk_status tk_swiglu_quant_t(const void* h_bf16, int64_t rows, int32_t I,
                                      const int32_t* row_src, const int32_t* pos,
                                      const float* topk_w, int32_t T, int32_t k, void* out,
                                      float* scales, void* out_t, float* scales_t,
                                      hipStream_t stream)
{
    using tk::fail;
    if (rows < 0 || rows % kTile != 0)
        return fail(TK_ERR_ARG, "tk_swiglu_quant_t: rows=%lld must be a multiple of 128",
                    static_cast<long long>(rows));
    if (I < 128 || I % 128 != 0)
        return fail(TK_ERR_ARG, "tk_swiglu_quant_t: I=%d must be a positive multiple of 128", I);
    const int n_weight_args = (row_src != nullptr) + (pos != nullptr) + (topk_w != nullptr);
    if (n_weight_args != 0 && n_weight_args != 3)
        return fail(TK_ERR_ARG, "tk_swiglu_quant_t: row_src, pos and topk_w go together");
    const bool weighted = n_weight_args == 3;
    if (weighted && (T < 0 || k < 1 || k > TK_MAX_TOPK))
        return fail(TK_ERR_ARG, "tk_swiglu_quant_t: T=%d, k=%d invalid for the weights", T, k);
    if (rows == 0) return tk::ok();
    if (h_bf16 == nullptr || out == nullptr || scales == nullptr || out_t == nullptr ||
        scales_t == nullptr)
        return fail(TK_ERR_ARG, "tk_swiglu_quant_t: NULL tensor pointer");
    if (!tk::aligned16(h_bf16) || !tk::aligned16(out) || !tk::aligned16(out_t) ||
        !tk::aligned4(scales) || !tk::aligned4(scales_t) || (row_src && !tk::aligned4(row_src)) ||
        (pos && !tk::aligned4(pos)) || (topk_w && !tk::aligned4(topk_w)))
        return fail(TK_ERR_ARG, "tk_swiglu_quant_t: h/out/out_t must be 16-byte aligned, the rest 4-byte");
    const int64_t tiles = rows / kTile * (I / kTile);
    const SwigluArgs args{static_cast<const uint16_t*>(h_bf16), rows, nullptr, I,
                          row_src, pos, topk_w, T, k, static_cast<uint8_t*>(out), scales};
    const dim3 grid(static_cast<unsigned>(std::min<int64_t>(tiles, kTBlocks))), block(kTThreads);
    auto* ot = static_cast<uint8_t*>(out_t);
    const hipError_t e = weighted
        ? tk::launch(swiglu_quant_t_kernel<true>, grid, block, 0, stream, args, tiles, ot, scales_t)
        : tk::launch(swiglu_quant_t_kernel<false>, grid, block, 0, stream, args, tiles, ot, scales_t);
    return tk::launched(e, "tk_swiglu_quant_t");
}

TK_EXPORT tk_status tk_silu_bf16(const void* g_bf16, int64_t n, float* out, hipStream_t stream)
{
    using tk::fail;
    if (n < 0) return fail(TK_ERR_ARG, "tk_silu_bf16: n < 0");
    if (n == 0) return tk::ok();
    if (g_bf16 == nullptr || out == nullptr) return fail(TK_ERR_ARG, "tk_silu_bf16: NULL pointer");
    if (reinterpret_cast<uintptr_t>(g_bf16) % 2 != 0 || !tk::aligned4(out))
        return fail(TK_ERR_ARG, "tk_silu_bf16: g must be 2-byte and out 4-byte aligned");
    const int64_t blocks = std::min<int64_t>((n + tk::kBlock - 1) / tk::kBlock, 1024);
    const hipError_t e = tk::launch(silu_kernel, dim3(static_cast<unsigned>(blocks)), dim3(tk::kBlock), 0,
                                    stream, static_cast<const uint16_t*>(g_bf16), n, out);
    return tk::launched(e, "tk_silu_bf16");
}
