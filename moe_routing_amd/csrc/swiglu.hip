// tk_swiglu_quant: SwiGLU activation fused with per-token 1x128 FP8 E4M3
// quantisation, optionally applying each expanded row's routing weight --
// the "SwiGLU + FP8 quantisation" fusion of TileKernels' quant/ module
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
// Work unit = (row, 1024 output columns); one wave per unit, 4 waves per
// workgroup.  Each lane owns 16 consecutive output columns: two 16-byte loads
// of gate and two of up, one 16-byte store of codes, and lane 0 of each
// 8-lane group (one 128-column block) stores the block's scale.  Inputs and
// outputs are touched once: streaming loads and stores.  At ~45 VALU
// instructions per element (the sigmoid's exp polynomial and IEEE division
// dominate) this kernel is bound by vector ALU issue, not HBM.
//
// The weight of row r is found from the map's outputs: t = row_src[r] and the
// slot j with pos[t, j] == r give w_r = topk_w[t, j]; a row no slot points at
// gets weight 0.
//
// tk_swiglu_quant_t adds the transpose of the fusion: the same activations
// also quantised as a^T (I, rows) in 1x128 blocks along its rows (128 tokens
// of one channel, the layout a weight-gradient GEMM reads), both outputs from
// one pass over h.
#include "tk_internal.h"

namespace {

constexpr int kChunk = 1024;   // output columns per unit (16 per lane)

struct SwigluArgs {
    const uint16_t* h;
    int64_t cap;
    const int32_t* n_rows;
    int I;
    int chunks;
    const int32_t* row_src;
    const int32_t* pos;
    const float* topk_w;
    int T, k;
    uint8_t* out;
    float* scales;
};

template <bool WEIGHTED>
__global__ __launch_bounds__(tk::kBlock) void swiglu_quant_kernel(SwigluArgs a)
{
    const int lane = threadIdx.x & (tk::kWave - 1);
    const int64_t u = static_cast<int64_t>(blockIdx.x) * tk::kWavesPerBlock +
                      tk::uniform(threadIdx.x / tk::kWave);
    int64_t rows = a.cap;
    if (a.n_rows != nullptr) {
        const int64_t n = *a.n_rows;
        rows = n < 0 ? 0 : (n < a.cap ? n : a.cap);
    }
    if (u >= rows * a.chunks) return;
    const int64_t r = u / a.chunks;
    const int col0 = static_cast<int>(u - r * a.chunks) * kChunk;
    const int col = col0 + lane * 16;
    const bool active = col < a.I;   // I % 128 == 0: 8-lane groups are wholly in or out

    const uint16_t* hr = a.h + static_cast<size_t>(r) * 2 * a.I;
    tk::u32x4 g0 = tk::u32x4{0u, 0u, 0u, 0u}, g1 = g0, u0 = g0, u1 = g0;
    if (active) {
        g0 = tk::load_stream(hr + col);
        g1 = tk::load_stream(hr + col + 8);
        u0 = tk::load_stream(hr + a.I + col);
        u1 = tk::load_stream(hr + a.I + col + 8);
    }
    // the row weight's three dependent loads overlap the row's loads above
    float w = 1.0f;
    if constexpr (WEIGHTED) {
        w = 0.0f;
        const int t = a.row_src[r];
        if (t >= 0 && t < a.T) {
            const int32_t* p = a.pos + static_cast<size_t>(t) * a.k;
            for (int j = 0; j < a.k; ++j)
                if (p[j] == r) w = a.topk_w[static_cast<size_t>(t) * a.k + j];
        }
    }

    const uint32_t gw[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const uint32_t uw[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
    float v[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float ga = tk::bf16_lo(gw[i]), gb = tk::bf16_hi(gw[i]);
        const float ua = tk::bf16_lo(uw[i]), ub = tk::bf16_hi(uw[i]);
        float va = (ga * tk::pinned_sigmoid(ga)) * ua;
        float vb = (gb * tk::pinned_sigmoid(gb)) * ub;
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
        tk::store_stream(a.out + static_cast<size_t>(r) * a.I + col, q);
        if ((lane & 7) == 0) a.scales[static_cast<size_t>(r) * (a.I / 128) + col / 128] = scale;
    }
}

// ---------------------------------------------------------------- transposed
// One workgroup of 512 threads per tile of 128 rows x 128 output columns
// computes the tile's activations once and writes them twice: row-major codes
// with 1x128 blocks along each row (the tile's 128 columns), and the
// transpose a^T with 1x128 blocks along each of its rows (the tile's 128 rows
// of one column).  Thread (rg, cg) = (tid / 16, tid % 16) holds rows 4*rg..
// and columns 8*cg.. of the tile (32 values, so the kernel keeps enough waves
// resident to hide its ALU latency): a row's 128 columns live in 16
// consecutive lanes (DPP row max), a column's 128 rows in 32 row groups
// across the eight waves (LDS max).  The transposed codes are staged in LDS
// and leave as whole 16-byte pieces of out_t's rows.
constexpr int kTile = 128;
constexpr int kTThreads = 512;
constexpr int kTRows = 4;                         // rows per thread
constexpr int kTGroups = kTile / kTRows;          // 32 row groups
constexpr int kTPitch = kTile + 16;               // bytes per staged out_t row (padded)

template <bool WEIGHTED>
__global__ __launch_bounds__(kTThreads) void swiglu_quant_t_kernel(SwigluArgs a, uint8_t* __restrict__ out_t,
                                                                 float* __restrict__ scales_t)
{
    __shared__ float w_row[kTile];
    __shared__ float col_part[kTGroups][kTile];
    __shared__ float col_scale[kTile];
    __shared__ uint8_t codes_t[kTile * kTPitch];
    const int tiles_c = a.I / kTile;
    const int64_t tr = blockIdx.x / tiles_c;
    const int tc = static_cast<int>(blockIdx.x - tr * tiles_c);
    const int64_t r0 = tr * kTile;
    const int c0 = tc * kTile;
    const int rg = threadIdx.x >> 4, cg = threadIdx.x & 15;
    const int64_t R = a.cap;

    // the tile's row loads first; the row weights' dependent loads overlap them
    tk::u32x4 gw[kTRows], uw[kTRows];
#pragma unroll
    for (int i = 0; i < kTRows; ++i) {
        const uint16_t* hr = a.h + static_cast<size_t>(r0 + rg * kTRows + i) * 2 * a.I;
        gw[i] = tk::load_stream(hr + c0 + cg * 8);
        uw[i] = tk::load_stream(hr + a.I + c0 + cg * 8);
    }
    if (threadIdx.x < kTile) {
        float w = 1.0f;
        if constexpr (WEIGHTED) {
            const int64_t r = r0 + threadIdx.x;
            w = 0.0f;
            const int t = a.row_src[r];
            if (t >= 0 && t < a.T) {
                const int32_t* p = a.pos + static_cast<size_t>(t) * a.k;
                for (int j = 0; j < a.k; ++j)
                    if (p[j] == r) w = a.topk_w[static_cast<size_t>(t) * a.k + j];
            }
        }
        w_row[threadIdx.x] = w;
    }
    __syncthreads();

    float v[kTRows][8];
#pragma unroll
    for (int i = 0; i < kTRows; ++i) {
        const uint32_t g4[4] = {gw[i].x, gw[i].y, gw[i].z, gw[i].w};
        const uint32_t u4[4] = {uw[i].x, uw[i].y, uw[i].z, uw[i].w};
        const float w = w_row[rg * kTRows + i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float ga = tk::bf16_lo(g4[j]), gb = tk::bf16_hi(g4[j]);
            const float ua = tk::bf16_lo(u4[j]), ub = tk::bf16_hi(u4[j]);
            float va = (ga * tk::pinned_sigmoid(ga)) * ua;
            float vb = (gb * tk::pinned_sigmoid(gb)) * ub;
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

    // row-major codes: one 1x128 block per tile row
#pragma unroll
    for (int i = 0; i < kTRows; ++i) {
        float m = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[i][j]));
        m = fmaxf(m, tk::dpp_f32<tk::kQuadXor1>(m));
        m = fmaxf(m, tk::dpp_f32<tk::kQuadXor2>(m));
        m = fmaxf(m, tk::dpp_f32<tk::kHalfMirror>(m));
        m = fmaxf(m, tk::dpp_f32<tk::kMirror>(m));      // the 16 lanes of this row group
        const float scale = fmaxf(m, 1e-4f) / 448.0f;
        const float inv = 1.0f / scale;
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
    __syncthreads();
    if (threadIdx.x < kTile) {
        float m = col_part[0][threadIdx.x];
#pragma unroll
        for (int g = 1; g < kTGroups; ++g) m = fmaxf(m, col_part[g][threadIdx.x]);
        const float scale = fmaxf(m, 1e-4f) / 448.0f;
        col_scale[threadIdx.x] = scale;
        scales_t[static_cast<size_t>(c0 + threadIdx.x) * (R / kTile) + tr] = scale;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float scale = col_scale[cg * 8 + j];
        const float inv = 1.0f / scale;
        const uint32_t q = tk::pack_fp8x4(tk::fp8_quotient(v[0][j], scale, inv), tk::fp8_quotient(v[1][j], scale, inv),
                                          tk::fp8_quotient(v[2][j], scale, inv), tk::fp8_quotient(v[3][j], scale, inv));
        *reinterpret_cast<uint32_t*>(codes_t + (cg * 8 + j) * kTPitch + rg * kTRows) = q;
    }
    __syncthreads();
    // 128 out_t rows of 128 bytes: 8 threads per row, 16 bytes each
    for (int i = threadIdx.x; i < kTile * 8; i += kTThreads) {
        const int c = i >> 3, part = i & 7;
        const tk::u32x4 q = *reinterpret_cast<const tk::u32x4*>(codes_t + c * kTPitch + part * 16);
        tk::store_stream(out_t + static_cast<size_t>(c0 + c) * R + r0 + part * 16, q);
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
    const int chunks = (I + kChunk - 1) / kChunk;
    const int64_t units = rows_capacity * chunks;
    const int64_t blocks = (units + tk::kWavesPerBlock - 1) / tk::kWavesPerBlock;
    if (blocks > INT32_MAX) return fail(TK_ERR_UNSUPPORTED, "tk_swiglu_quant: too many rows");
    const SwigluArgs args{static_cast<const uint16_t*>(h_bf16), rows_capacity, n_rows, I, chunks,
                          row_src, pos, topk_w, T, k, static_cast<uint8_t*>(out), scales};
    const dim3 grid(static_cast<unsigned>(blocks)), block(tk::kBlock);
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
    if (tiles > INT32_MAX) return fail(TK_ERR_UNSUPPORTED, "tk_swiglu_quant_t: too many rows");
    const SwigluArgs args{static_cast<const uint16_t*>(h_bf16), rows, nullptr, I, 0,
                          row_src, pos, topk_w, T, k, static_cast<uint8_t*>(out), scales};
    const dim3 grid(static_cast<unsigned>(tiles)), block(kTThreads);
    auto* ot = static_cast<uint8_t*>(out_t);
    const hipError_t e = weighted
        ? tk::launch(swiglu_quant_t_kernel<true>, grid, block, 0, stream, args, ot, scales_t)
        : tk::launch(swiglu_quant_t_kernel<false>, grid, block, 0, stream, args, ot, scales_t);
    return tk::launched(e, "tk_swiglu_quant_t");
}
